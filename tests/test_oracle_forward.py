"""Pins for the oracle's forward (definition of exact attention and its LSE).

The oracle is checked against things other than itself: torch's float64 CPU
scaled_dot_product_attention (an independent library routine for the same
definition), closed forms, and invariants.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.attention import head_forward, _f64
from workloads import make_inputs


def _sdpa64(q, k, v, scale, causal):
    """torch CPU float64 SDPA on BSHD inputs (GQA via enable_gqa)."""
    qt = q.double().transpose(1, 2)
    kt = k.double().transpose(1, 2)
    vt = v.double().transpose(1, 2)
    out = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale,
                                         enable_gqa=qt.shape[1] != kt.shape[1])
    return out.transpose(1, 2).numpy()


def _lse64(q, k, scale, causal):
    """log-sum-exp with torch.logsumexp (library routine), [B, Hq, Sq]."""
    g = q.shape[2] // k.shape[2]
    qt = q.double().transpose(1, 2)
    kt = k.double().repeat_interleave(g, dim=2).transpose(1, 2)
    s = scale * qt @ kt.transpose(-1, -2)
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    return torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("b,s,hq,hkv,d,causal", [
    (1, 37, 2, 2, 16, False), (1, 37, 2, 2, 16, True), (2, 64, 4, 1, 8, True),
    (2, 65, 4, 2, 32, False), (1, 130, 2, 2, 64, True)])
def test_forward_matches_torch_sdpa_float64(b, s, hq, hkv, d, causal):
    inp = make_inputs(b, s, s, hq, hkv, d, seed=11 + s)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal)
    ref = _sdpa64(inp["q"], inp["k"], inp["v"], scale, causal)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _lse64(inp["q"], inp["k"], scale, causal), rtol=0, atol=1e-12)


def test_causal_row0_is_v0():
    """Causal row 0 sees only key 0: O_0 = V_0 and LSE_0 = alpha q_0 . k_0."""
    inp = make_inputs(2, 33, 33, 3, 3, 16, seed=5)
    scale = 0.3
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, True)
    q, k, v = (_f64(inp[n]) for n in ("q", "k", "v"))
    np.testing.assert_allclose(o[:, 0], v[:, 0], rtol=0, atol=1e-14)
    want = scale * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0])
    np.testing.assert_allclose(lse[:, :, 0], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(causal):
    """All keys equal: softmax is uniform over the visible keys, so O_i is the
    mean of the visible V rows and LSE_i = alpha q_i . k + ln(n_visible)."""
    s, d = 40, 8
    inp = make_inputs(1, s, s, 2, 2, d, seed=7)
    k = inp["k"].clone()
    k[:] = k[:, :1]
    scale = 0.5
    o, lse = oracle.attention_forward(inp["q"], k, inp["v"], scale, causal)
    v = _f64(inp["v"])
    q = _f64(inp["q"])
    kk = _f64(k)[0, 0]
    for i in (0, 1, 17, s - 1):
        n = i + 1 if causal else s
        np.testing.assert_allclose(o[0, i], v[0, :n].mean(axis=0), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0, :, i], scale * np.sum(q[0, i] * kk, axis=-1) + math.log(n),
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    inp = make_inputs(1, 50, 50, 2, 1, 16, seed=9)
    scale = 0.25
    _, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal)
    p = oracle.attention_probs(inp["q"], inp["k"], scale, causal, lse)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-13)
    if causal:
        assert np.all(np.triu(p[0, 0], 1) == 0)


def test_gqa_equals_mha_with_repeated_kv():
    inp = make_inputs(2, 48, 48, 8, 2, 16, seed=21)
    scale = 0.25
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, True)
    kr = oracle.repeat_kv(inp["k"], 4)
    vr = oracle.repeat_kv(inp["v"], 4)
    o2, lse2 = oracle.attention_forward(inp["q"], kr, vr, scale, True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    # head h uses KV head h // 4: heads 0..3 must differ from heads 4..7 in general
    assert not np.allclose(o[:, :, 0], o[:, :, 4])


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_per_sequence(causal):
    lengths = [5, 1, 0, 37, 64]
    inp = make_inputs(0, 0, 0, 4, 2, 16, seed=3, lengths=lengths)
    scale = 0.25
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal,
                                      inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    cu = inp["cu_seqlens_q"].tolist()
    for s, n in enumerate(lengths):
        if n == 0:
            continue
        sl = slice(cu[s], cu[s + 1])
        os_, ls_ = oracle.attention_forward(inp["q"][None, sl], inp["k"][None, sl],
                                            inp["v"][None, sl], scale, causal)
        np.testing.assert_array_equal(o[sl], os_[0])
        np.testing.assert_array_equal(lse[:, sl], ls_[0])


def test_sampled_rows_match_full_rows():
    inp = make_inputs(1, 300, 300, 1, 1, 32, seed=4)
    q, k, v = (_f64(inp[n])[0, :, 0] for n in ("q", "k", "v"))
    o, lse = head_forward(q, k, v, 0.2, True)
    rows = np.array([0, 7, 128, 299])
    o2, lse2 = head_forward(q, k, v, 0.2, True, rows=rows)
    np.testing.assert_array_equal(o[rows], o2)
    np.testing.assert_array_equal(lse[rows], lse2)


def test_empty_key_sequence_gives_zero_and_neg_inf():
    """Reading for a row that sees no key: O = 0, LSE = -inf (pages silent)."""
    q = np.ones((3, 4))
    k = np.zeros((0, 4))
    v = np.zeros((0, 4))
    o, lse = head_forward(q, k, v, 1.0, False)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
