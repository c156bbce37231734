"""Pins for the oracle's causal mask when query and key lengths differ.

The pages only use the square lower-triangular mask. The reading taken for
Sq != Sk aligns the diagonal to the last query and last key (bottom-right):
query i sees key j iff j <= i + Sk - Sq; a row that sees no key gets O = 0,
LSE = -inf and zero gradients. Pinned against torch's own lower-right causal
bias (an independent library definition of that mask) through float64 CPU
scaled_dot_product_attention and its autograd, against the square causal
problem whose last Sq rows it is, and against central finite differences.
"""
import math
import warnings

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
from oracle.attention import _f64
from workloads import make_inputs


def _sdpa_lower_right(q, k, v, scale, grad_out=None):
    """float64 SDPA with torch's lower-right causal bias on BSHD inputs;
    returns O (and dQ, dK, dV when ``grad_out`` is given). GQA by repeating
    K/V heads inside the graph, so autograd sums their gradients per group."""
    g = q.shape[2] // k.shape[2]
    qt = q.double().transpose(1, 2).clone().requires_grad_(True)
    kt = k.double().transpose(1, 2).clone().requires_grad_(True)
    vt = v.double().transpose(1, 2).clone().requires_grad_(True)
    with warnings.catch_warnings():
        # torch warns that rows above the diagonal (Sq > Sk) may come out NaN;
        # its CPU float64 path returns 0 for them, which the tests rely on
        warnings.simplefilter("ignore", UserWarning)
        bias = causal_lower_right(q.shape[1], k.shape[1])
        out = F.scaled_dot_product_attention(qt, kt.repeat_interleave(g, dim=1),
                                             vt.repeat_interleave(g, dim=1),
                                             attn_mask=bias, scale=scale)
    o = out.detach().transpose(1, 2).numpy()
    if grad_out is None:
        return o
    out.backward(grad_out.double().transpose(1, 2))
    return o, tuple(t.grad.transpose(1, 2).numpy() for t in (qt, kt, vt))


@pytest.mark.parametrize("sq,sk,hq,hkv", [(5, 37, 2, 2), (33, 70, 4, 1), (1, 50, 2, 1),
                                         (40, 40, 2, 2), (70, 33, 4, 2), (9, 3, 2, 2)])
def test_forward_matches_torch_lower_right_bias(sq, sk, hq, hkv):
    inp = make_inputs(2, sq, sk, hq, hkv, 16, seed=300 + sq + sk)
    scale = 1.0 / math.sqrt(16)
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, True)
    ref = _sdpa_lower_right(inp["q"], inp["k"], inp["v"], scale)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    # rows above the diagonal (only when Sq > Sk) see nothing
    empty = max(0, sq - sk)
    assert np.all(o[:, :empty] == 0) and np.all(np.isneginf(lse[:, :, :empty]))
    assert np.all(np.isfinite(lse[:, :, empty:]))


def test_lse_matches_logsumexp_of_visible_scores():
    """LSE against torch.logsumexp over the scores torch's bias leaves visible."""
    inp = make_inputs(1, 21, 45, 2, 2, 8, seed=77)
    scale = 0.4
    _, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, True)
    qt = inp["q"].double().transpose(1, 2)
    kt = inp["k"].double().transpose(1, 2)
    bias = causal_lower_right(21, 45)._materialize(torch.device("cpu"))
    s = (scale * qt @ kt.transpose(-1, -2)).masked_fill(~bias, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_short_query_block_is_the_tail_of_the_square_problem():
    """Sq < Sk: the result equals the last Sq rows of the square causal problem
    (Sk queries, torch is_causal) whose last Sq queries are these."""
    sq, sk = 19, 64
    big = make_inputs(1, sk, sk, 2, 1, 32, seed=12)
    q_tail = big["q"][:, sk - sq:]
    scale = 0.25
    o, lse = oracle.attention_forward(q_tail, big["k"], big["v"], scale, True)
    qt = big["q"].double().transpose(1, 2)
    kt = big["k"].double().repeat_interleave(2, dim=2).transpose(1, 2)
    vt = big["v"].double().repeat_interleave(2, dim=2).transpose(1, 2)
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    np.testing.assert_allclose(o, ref.transpose(1, 2).numpy()[:, sk - sq:], rtol=0, atol=1e-12)


def test_single_query_sees_every_key():
    """Sq = 1 (one new token against a key cache): plain non-causal attention."""
    inp = make_inputs(1, 1, 57, 2, 2, 16, seed=9)
    o_c, lse_c = oracle.attention_forward(inp["q"], inp["k"], inp["v"], 0.3, True)
    o_n, lse_n = oracle.attention_forward(inp["q"], inp["k"], inp["v"], 0.3, False)
    np.testing.assert_array_equal(o_c, o_n)
    np.testing.assert_array_equal(lse_c, lse_n)


def test_long_query_rows_below_offset_match_square_problem():
    """Sq > Sk: rows Sq - Sk .. Sq - 1 form the square causal problem with the
    same keys (torch is_causal); the rows before them are O = 0."""
    sq, sk = 50, 20
    inp = make_inputs(1, sq, sk, 2, 2, 16, seed=14)
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], 0.3, True)
    qt = inp["q"][:, sq - sk:].double().transpose(1, 2)
    kt = inp["k"].double().transpose(1, 2)
    vt = inp["v"].double().transpose(1, 2)
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.3)
    np.testing.assert_allclose(o[:, sq - sk:], ref.transpose(1, 2).numpy(), rtol=0, atol=1e-12)
    assert np.all(o[:, :sq - sk] == 0)


@pytest.mark.parametrize("sq,sk,hq,hkv", [(13, 40, 2, 1), (40, 13, 2, 2), (1, 30, 4, 2)])
def test_backward_matches_torch_autograd_lower_right(sq, sk, hq, hkv):
    inp = make_inputs(1, sq, sk, hq, hkv, 8, seed=500 + sq)
    scale = 0.35
    dq, dk, dv = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True)
    _, (gq, gk, gv) = _sdpa_lower_right(inp["q"], inp["k"], inp["v"], scale, grad_out=inp["do"])
    for mine, ref in ((dq, gq), (dk, gk), (dv, gv)):
        np.testing.assert_allclose(mine, ref, rtol=0, atol=1e-12)
    if sq > sk:
        assert np.all(dq[:, :sq - sk] == 0)


def test_backward_equals_square_problem_with_zero_upstream_on_prefix():
    """Sq < Sk: with dO = 0 on the first Sk - Sq queries of the square causal
    problem, its dK, dV are those of the short query block, and its dQ on the
    last rows is the short block's dQ (torch autograd, is_causal)."""
    sq, sk = 11, 32
    big = make_inputs(1, sk, sk, 2, 2, 8, seed=21)
    do = big["do"].clone()
    do[:, :sk - sq] = 0
    scale = 0.5
    dq, dk, dv = oracle.attention_backward(big["q"][:, sk - sq:], big["k"], big["v"],
                                           do[:, sk - sq:], scale, True)
    qt, kt, vt = (big[n].double().transpose(1, 2).clone().requires_grad_(True)
                  for n in ("q", "k", "v"))
    out = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    out.backward(do.double().transpose(1, 2))
    np.testing.assert_allclose(dq, qt.grad.transpose(1, 2).numpy()[:, sk - sq:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("sq,sk", [(4, 9), (9, 4)])
def test_backward_matches_central_finite_differences(sq, sk):
    inp = make_inputs(1, sq, sk, 2, 1, 4, seed=61 + sq)
    q, k, v, do = (_f64(inp[n]).copy() for n in ("q", "k", "v", "do"))
    scale = 0.7

    def loss():
        o, _ = oracle.attention_forward(q, k, v, scale, True)
        return float(np.sum(o * do))

    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, True)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            fp = loss()
            x[idx] = old - h
            fm = loss()
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        rel = np.linalg.norm(num - g) / np.linalg.norm(g)
        assert rel < 1e-7, (name, rel)


def test_varlen_mixed_lengths_equals_per_sequence():
    """Packed sequences with different query and key lengths per sequence."""
    lq, lk = [3, 17, 9, 0], [10, 17, 4, 6]
    cq = torch.tensor(np.concatenate([[0], np.cumsum(lq)]), dtype=torch.int32)
    ck = torch.tensor(np.concatenate([[0], np.cumsum(lk)]), dtype=torch.int32)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(sum(lq), 2, 8, generator=g).bfloat16()
    k = torch.randn(sum(lk), 1, 8, generator=g).bfloat16()
    v = torch.randn(sum(lk), 1, 8, generator=g).bfloat16()
    o, lse = oracle.attention_forward(q, k, v, 0.4, True, cq, ck)
    for s in range(len(lq)):
        qs = slice(int(cq[s]), int(cq[s + 1]))
        ks = slice(int(ck[s]), int(ck[s + 1]))
        os_, ls_ = oracle.attention_forward(q[None, qs], k[None, ks], v[None, ks], 0.4, True)
        np.testing.assert_array_equal(o[qs], os_[0])
        np.testing.assert_array_equal(lse[:, qs], ls_[0])


def test_blockwise_model_reaches_definition_with_offset():
    """The tiled conditional-rescale model with a bottom-right diagonal."""
    for sq, sk in ((40, 100), (100, 40)):
        inp = make_inputs(1, sq, sk, 2, 1, 16, seed=sq)
        o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], 0.5, True)
        o, lse = oracle.blockwise_forward(inp["q"], inp["k"], inp["v"], 0.5, True,
                                          block_m=32, block_n=16, group_rows=8)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        fin = np.isfinite(lse_ref)
        np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=0, atol=1e-12)
        assert np.array_equal(np.isneginf(lse), ~fin)
