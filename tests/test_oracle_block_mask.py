"""Pins for the oracle's block-sparse masks (one entry per 128 x 128 block of
(query, key) pairs per (batch, query head), ANDed with the causal rule).

Checked against torch's float64 CPU scaled_dot_product_attention with the
equivalent boolean element mask (an independent library routine) and its
autograd, against central finite differences of the oracle's forward, and
against special cases: an all-set mask is no mask, and rows whose blocks are
all cleared see no key (O = 0, LSE = -inf, zero gradient) while every other
row equals the attention of the remaining rows alone.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.attention import BLOCK, _f64
from workloads import make_inputs


def _random_mask(b, h, sq, sk, seed, keep_first_col=True, density=0.5):
    nqb, nkb = -(-sq // BLOCK), -(-sk // BLOCK)
    g = torch.Generator().manual_seed(seed)
    m = torch.rand((b, h, nqb, nkb), generator=g) < density
    if keep_first_col:      # key block 0 holds key 0, which every causal row sees
        m[..., 0] = True
    return m


def _element_mask(m, sq, sk, causal):
    """[B, H, Sq, Sk] boolean: block entry AND the (bottom-right) causal rule."""
    e = m.repeat_interleave(BLOCK, dim=2).repeat_interleave(BLOCK, dim=3)[:, :, :sq, :sk]
    if causal:
        tri = torch.arange(sk)[None, :] <= torch.arange(sq)[:, None] + (sk - sq)
        e = e & tri
    return e


def _sdpa(q, k, v, scale, emask, grad=False, do=None):
    qt, kt, vt = (x.double().transpose(1, 2).clone().requires_grad_(grad) for x in (q, k, v))
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=emask, scale=scale,
                                         enable_gqa=qt.shape[1] != kt.shape[1])
    if not grad:
        return out.transpose(1, 2).detach().numpy()
    out.backward(do.double().transpose(1, 2))
    return (out.transpose(1, 2).detach().numpy(),
            *(x.grad.transpose(1, 2).numpy() for x in (qt, kt, vt)))


@pytest.mark.parametrize("b,sq,sk,hq,hkv,d,causal", [
    (1, 300, 300, 2, 2, 16, False), (1, 300, 300, 2, 2, 16, True), (2, 257, 400, 4, 2, 8, False),
    (1, 384, 384, 2, 1, 8, True), (1, 200, 520, 2, 2, 8, True)])
def test_forward_with_block_mask_matches_torch_sdpa(b, sq, sk, hq, hkv, d, causal):
    inp = make_inputs(b, sq, sk, hq, hkv, d, seed=500 + sq + sk)
    m = _random_mask(b, hq, sq, sk, seed=sq)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal, block_mask=m)
    em = _element_mask(m, sq, sk, causal)
    ref = _sdpa(inp["q"], inp["k"], inp["v"], scale, em)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    # LSE with torch.logsumexp over the visible scores
    g = hq // hkv
    s = scale * inp["q"].double().transpose(1, 2) @ \
        inp["k"].double().repeat_interleave(g, dim=2).transpose(1, 2).transpose(-1, -2)
    want = torch.logsumexp(s.masked_fill(~em, float("-inf")), dim=-1).numpy()
    np.testing.assert_allclose(lse, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_with_block_mask_matches_torch_autograd(causal):
    b, s, hq, hkv, d = 1, 300, 4, 2, 8
    inp = make_inputs(b, s, s, hq, hkv, d, seed=61)
    m = _random_mask(b, hq, s, s, seed=62)
    scale = 0.4
    grads = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal,
                                      block_mask=m)
    _, *ref = _sdpa(inp["q"], inp["k"], inp["v"], scale, _element_mask(m, s, s, causal),
                    grad=True, do=inp["do"])
    for mine, r in zip(grads, ref):
        np.testing.assert_allclose(mine, r, rtol=0, atol=1e-11)


def test_backward_with_block_mask_matches_finite_differences():
    b, s, hq, hkv, d = 1, 200, 2, 1, 2
    inp = make_inputs(b, s, s, hq, hkv, d, seed=71)
    q, k, v, do = (_f64(inp[n]).copy() for n in ("q", "k", "v", "do"))
    m = np.array([[[[True, False], [False, True]], [[True, True], [True, False]]]])
    scale = 0.6
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, False, block_mask=m)

    def loss():
        o, _ = oracle.attention_forward(q, k, v, scale, False, block_mask=m)
        return float(np.sum(o * do))

    h = 1e-6
    rng = np.random.default_rng(0)
    for name, x, gr in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        idxs = [tuple(int(rng.integers(0, n)) for n in x.shape) for _ in range(40)]
        for idx in idxs:
            old = x[idx]
            x[idx] = old + h
            fp = loss()
            x[idx] = old - h
            fm = loss()
            x[idx] = old
            num = (fp - fm) / (2 * h)
            assert abs(num - gr[idx]) <= 1e-7 * max(1.0, abs(gr[idx])), (name, idx, num, gr[idx])


@pytest.mark.parametrize("causal", [False, True])
def test_all_set_mask_is_no_mask(causal):
    inp = make_inputs(2, 300, 300, 2, 2, 16, seed=81)
    m = torch.ones((2, 2, 3, 3), dtype=torch.bool)
    a = oracle.attention_forward(inp["q"], inp["k"], inp["v"], 0.25, causal, block_mask=m)
    b = oracle.attention_forward(inp["q"], inp["k"], inp["v"], 0.25, causal)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    ga = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], 0.25, causal,
                                   block_mask=m)
    gb = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], 0.25, causal)
    for x, y in zip(ga, gb):
        assert np.array_equal(x, y)


def test_rows_with_every_block_cleared_see_no_key():
    """Block row 1 of head 0 cleared: its 128 rows see nothing (O = 0, LSE =
    -inf, dQ = 0); the other rows, and dK, dV, equal torch on the remaining
    rows alone (the cleared rows contribute nothing to dK, dV)."""
    b, s, hq, d = 1, 300, 2, 8
    inp = make_inputs(b, s, s, hq, hq, d, seed=91)
    m = torch.ones((1, hq, 3, 3), dtype=torch.bool)
    m[0, 0, 1, :] = False
    scale = 0.5
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, False, block_mask=m)
    dq, dk, dv = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, False,
                                           block_mask=m)
    dead = slice(128, 256)
    assert np.all(o[0, dead, 0] == 0) and np.all(np.isneginf(lse[0, 0, dead]))
    assert np.all(dq[0, dead, 0] == 0)
    keep = np.r_[0:128, 256:300]
    q0, do0 = inp["q"][:, keep, :1], inp["do"][:, keep, :1]
    ref_o, ref_dq, ref_dk, ref_dv = _sdpa(q0, inp["k"][:, :, :1], inp["v"][:, :, :1], scale,
                                          None, grad=True, do=do0)
    np.testing.assert_allclose(o[:, keep, :1], ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq[:, keep, :1], ref_dq, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk[:, :, :1], ref_dk, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv[:, :, :1], ref_dv, rtol=0, atol=1e-11)
