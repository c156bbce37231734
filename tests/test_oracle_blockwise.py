"""Pins for the blockwise (online softmax, conditional rescale) algorithm model.

The pages claim that skipping rescales whose max jump is at most tau keeps the
output exact because the final normalisation uses the true statistics.  The
model is run with tau = 8 (the pages' value), tau = 0 (rescale on every growth
of the max) and compared with the definition; inputs with Q and K scaled by 3
produce max jumps above tau so both branches are exercised.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import make_inputs


def _scaled_inputs(s, hq, hkv, d, seed, mult=3.0):
    inp = make_inputs(1, s, s, hq, hkv, d, seed=seed, scaled_heads=True)
    return inp


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block_n,group_rows", [(16, 8), (32, 32), (64, 16)])
def test_conditional_rescale_equals_definition(causal, block_n, group_rows):
    d = 32
    inp = _scaled_inputs(96, 4, 2, d, seed=100 + block_n)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal)
    for tau in (8.0, 0.0):
        st = {}
        ob, lb = oracle.blockwise_forward(inp["q"], inp["k"], inp["v"], scale, causal,
                                          block_m=64, block_n=block_n, group_rows=group_rows,
                                          tau=tau, stats=st)
        np.testing.assert_allclose(ob, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lb, lse, rtol=0, atol=1e-12)
        if tau == 8.0:
            assert st["rescaled"] > 0 and st["skipped"] > 0, st
            # unnormalised p never exceeds 2^tau
            assert st["max_p"] <= 2.0 ** 8 * (1 + 1e-12)


def test_tau8_skips_more_than_tau0():
    inp = _scaled_inputs(128, 2, 2, 16, seed=7)
    n = {}
    for tau in (8.0, 0.0):
        st = {}
        oracle.blockwise_forward(inp["q"], inp["k"], inp["v"], 0.25, False, block_n=16,
                                 group_rows=16, tau=tau, stats=st)
        n[tau] = st["skipped"]
    assert n[8.0] > n[0.0]


@pytest.mark.parametrize("causal", [False, True])
def test_float32_model_close_to_definition(causal):
    """Single-precision arithmetic with bf16-rounded P (what a bf16 MFMA sees)
    stays within the bf16 product error of the float64 definition."""
    d = 64
    inp = _scaled_inputs(128, 2, 2, d, seed=13)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal)
    ob, lb = oracle.blockwise_forward(inp["q"], inp["k"], inp["v"], scale, causal, block_n=32,
                                      group_rows=32, dtype=np.float32)
    np.testing.assert_allclose(ob, o, rtol=0, atol=2e-5)
    np.testing.assert_allclose(lb, lse, rtol=0, atol=2e-5)
    ob, lb = oracle.blockwise_forward(inp["q"], inp["k"], inp["v"], scale, causal, block_n=32,
                                      group_rows=32, dtype=np.float32, round_p=oracle.round_bf16)
    err = np.abs(ob - o)
    assert err.max() < 2.0 ** -9 * np.abs(o).max() * 2, err.max()
    np.testing.assert_allclose(lb, lse, rtol=0, atol=2e-5)


def test_emulated_exp2_reaches_definition_within_poly_bound():
    d = 32
    inp = _scaled_inputs(64, 2, 1, d, seed=17)
    scale = 1.0 / math.sqrt(d)
    coeffs, _ = oracle.fit_exp2_minimax()
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, True)
    ob, lb = oracle.blockwise_forward(inp["q"], inp["k"], inp["v"], scale, True, block_n=16,
                                      group_rows=16, exp2=lambda x: oracle.exp2_cody_waite(x, coeffs),
                                      dtype=np.float32)
    # relative error of every p is below 8.6e-5, so LSE moves by at most ~1e-4
    assert np.max(np.abs(lb - lse)) < 1.2e-4
    assert np.max(np.abs(ob - o)) < 2e-4 * np.abs(o).max()
