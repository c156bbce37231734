"""Pins for the exp2 emulation and the bf16 helpers against numbers printed on
the pages (tests/golden/pages_constants.json) and against library routines."""
import json
import os

import numpy as np
import torch

import oracle
from oracle.exp2poly import max_rel_error

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def _all_f32_in(lo_exp, hi_exp):
    """Every float32 value in [2^lo_exp, 2^hi_exp)."""
    lo = np.float32(2.0 ** lo_exp).view(np.uint32)
    hi = np.float32(2.0 ** hi_exp).view(np.uint32)
    return np.arange(lo, hi, dtype=np.uint32).view(np.float32)


def test_refit_reproduces_printed_coefficients():
    coeffs, err = oracle.fit_exp2_minimax()
    printed = GOLD["exp2_poly_coeffs"]["value"]
    assert coeffs[0] == printed[0] == 1.0
    for mine, page in zip(coeffs[1:], printed[1:]):
        assert round(mine, 4) == page, (mine, page)
    assert err <= GOLD["exp2_poly_max_rel_err_fp32"]["value"]


def test_poly_error_bound_brute_force_float32():
    """Every float32 f in [2^-10, 1): the refit polynomial's relative error is
    within the printed 8.77e-5; the 4-digit printed coefficients are not."""
    coeffs, _ = oracle.fit_exp2_minimax()
    bound = GOLD["exp2_poly_max_rel_err_fp32"]["value"]
    worst = 0.0
    for e in range(-10, 0):
        f = _all_f32_in(e, e + 1)
        worst = max(worst, max_rel_error(coeffs, f))
    assert worst <= bound, worst
    assert max_rel_error(oracle.PAGE_COEFFS, np.linspace(0, 1, 100001)) > bound


def test_cody_waite_exp2_on_attention_range():
    coeffs, _ = oracle.fit_exp2_minimax()
    bound = GOLD["exp2_poly_max_rel_err_fp32"]["value"]
    x = np.linspace(-126.0, 8.0, 3_000_001).astype(np.float32)
    y = oracle.exp2_cody_waite(x, coeffs).astype(np.float64)
    rel = np.abs(y / np.exp2(x.astype(np.float64)) - 1.0)
    assert rel.max() <= bound, rel.max()


def test_cody_waite_exact_at_integers_and_flushes():
    coeffs, _ = oracle.fit_exp2_minimax()
    n = np.arange(-126, 9, dtype=np.float32)
    np.testing.assert_array_equal(oracle.exp2_cody_waite(n, coeffs), np.exp2(n))
    z = oracle.exp2_cody_waite(np.array([-126.5, -200.0, -np.inf], dtype=np.float32), coeffs)
    np.testing.assert_array_equal(z, 0.0)


def test_round_bf16_matches_torch():
    x = torch.cat([torch.randn(200000) * 7, torch.randn(1000) * 1e-38, torch.randn(1000) * 1e30])
    mine = oracle.round_bf16(x.double().numpy())
    ref = x.to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(mine, ref)


def test_bf16_max_relative_rounding_error_is_page_value():
    """Max relative error of RNE rounding to bf16 over every float32 in [1, 2)
    equals the printed BF16 quantisation error 3.89e-3 (= 2^-8 / (1 + 2^-8))."""
    x = _all_f32_in(0, 1).astype(np.float64)
    rel = np.abs(oracle.round_bf16(x) - x) / x
    assert round(float(rel.max()), 5) == GOLD["bf16_quant_rel_err"]["value"]
    assert abs(rel.max() - 2.0 ** -8 / (1 + 2.0 ** -8)) < 1e-15


def test_bf16_ulp():
    np.testing.assert_array_equal(oracle.bf16_ulp([1.0, 1.5, 4.0, 7.99, -0.5]),
                                  [2.0 ** -7, 2.0 ** -7, 2.0 ** -5, 2.0 ** -5, 2.0 ** -8])
