"""Pins for the oracle's backward (dQ, dK, dV of exact attention).

Checked against central finite differences of the oracle's own forward (which
is pinned separately), against torch float64 autograd through
scaled_dot_product_attention, and against identities that follow from the
definition (rows of P sum to one, so sum_j dV_j = sum_i dO_i and
sum_j dK_j = 0 per KV head).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.attention import _f64
from workloads import make_inputs


def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention_forward(q, k, v, scale, causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("hkv,causal", [(2, False), (2, True), (1, True), (1, False)])
def test_backward_matches_central_finite_differences(hkv, causal):
    inp = make_inputs(1, 7, 7, 2, hkv, 4, seed=31 + hkv)
    q, k, v, do = (_f64(inp[n]).copy() for n in ("q", "k", "v", "do"))
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            fp = _loss(q, k, v, do, scale, causal)
            x[idx] = old - h
            fm = _loss(q, k, v, do, scale, causal)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        rel = np.linalg.norm(num - g) / np.linalg.norm(g)
        assert rel < 1e-7, (name, rel)


@pytest.mark.parametrize("b,s,hq,hkv,d,causal", [(1, 33, 2, 2, 16, True), (2, 40, 4, 2, 8, False),
                                                (1, 70, 4, 1, 32, True)])
def test_backward_matches_torch_autograd_float64(b, s, hq, hkv, d, causal):
    inp = make_inputs(b, s, s, hq, hkv, d, seed=41 + s)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    qt, kt, vt = (inp[n].double().transpose(1, 2).clone().requires_grad_(True)
                  for n in ("q", "k", "v"))
    out = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale,
                                         enable_gqa=hq != hkv)
    out.backward(inp["do"].double().transpose(1, 2))
    for mine, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(mine, ref.transpose(1, 2).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    hq, hkv = 4, 2
    inp = make_inputs(2, 45, 45, hq, hkv, 16, seed=51)
    scale = 0.25
    dq, dk, dv = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    do = _f64(inp["do"])
    # sum over keys of dV = sum over queries (and grouped heads) of dO
    want = do.reshape(2, 45, hkv, hq // hkv, 16).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), want, rtol=0, atol=1e-11)
    # sum over keys of dK = 0 (rows of dS sum to zero)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, rtol=0, atol=1e-11)
    # D_i = sum_j P_ij dP_ij  (D = rowsum(dO o O))
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal)
    dd = oracle.rowsum_do_o(do, o)                                    # [B, S, Hq]
    p = oracle.attention_probs(inp["q"], inp["k"], scale, causal, lse)  # [B, Hq, S, S]
    vr = oracle.repeat_kv(inp["v"], hq // hkv)
    dp = np.einsum("bihd,bjhd->bhij", do, vr)
    np.testing.assert_allclose(np.einsum("bhij,bhij->bih", p, dp), dd, rtol=0, atol=1e-11)


def test_gqa_backward_is_group_sum_of_mha():
    hq, hkv = 6, 2
    inp = make_inputs(1, 30, 30, hq, hkv, 8, seed=61)
    scale = 0.3
    dq, dk, dv = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True)
    kr, vr = oracle.repeat_kv(inp["k"], 3), oracle.repeat_kv(inp["v"], 3)
    dq2, dk2, dv2 = oracle.attention_backward(inp["q"], kr, vr, inp["do"], scale, True)
    np.testing.assert_allclose(dq, dq2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(1, 30, hkv, 3, 8).sum(3), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(1, 30, hkv, 3, 8).sum(3), rtol=0, atol=1e-13)


def test_varlen_backward_equals_per_sequence():
    lengths = [9, 0, 1, 31]
    inp = make_inputs(0, 0, 0, 4, 2, 8, seed=71, lengths=lengths)
    scale = 0.3
    dq, dk, dv = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True,
                                           inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    cu = inp["cu_seqlens_q"].tolist()
    for s, n in enumerate(lengths):
        if n == 0:
            continue
        sl = slice(cu[s], cu[s + 1])
        g = oracle.attention_backward(inp["q"][None, sl], inp["k"][None, sl], inp["v"][None, sl],
                                      inp["do"][None, sl], scale, True)
        for a, b in zip((dq, dk, dv), g):
            np.testing.assert_array_equal(a[sl], b[0])


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_and_columns_match_full_backward(causal):
    """The per-row dQ and per-column dK/dV helpers used on full-size outputs
    agree with the full backward (itself pinned by finite differences)."""
    inp = make_inputs(1, 90, 90, 1, 1, 16, seed=81)
    q, k, v, do = (_f64(inp[n])[0, :, 0] for n in ("q", "k", "v", "do"))
    dq, dk, dv = oracle.head_backward(q, k, v, do, 0.25, causal)
    rows = np.array([0, 1, 45, 89])
    np.testing.assert_allclose(oracle.head_dq_rows(q, k, v, do, 0.25, causal, rows), dq[rows],
                               rtol=0, atol=1e-13)
    cols = np.array([0, 30, 88, 89])
    dkc, dvc = oracle.head_dkdv_cols(q, k, v, do, 0.25, causal, cols)
    np.testing.assert_allclose(dkc, dk[cols], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dvc, dv[cols], rtol=0, atol=1e-13)
