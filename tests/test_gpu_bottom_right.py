"""Causal attention with unequal query and key lengths on the HIP path.

The diagonal is aligned to the last query and last key: query i sees key j iff
j <= i + Sk - Sq (a query block appended to a key cache); with Sq > Sk the
first Sq - Sk queries see no key and get O = 0, LSE = -inf, dQ = 0. Every case
is compared with the float64 oracle through the C ABI, in each kernel design.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_71_amd as ea
import oracle
from parity import check_grads, check_lse, check_o
from workloads import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


DESIGNS = {"recompute": dict(bwd_design=ea.BWD_RECOMPUTE),
           "fused": dict(bwd_design=ea.BWD_FUSED_DQ),
           "stored": dict(bwd_design=ea.BWD_STORED_DS)}


@pytest.fixture(params=list(DESIGNS))
def design(request):
    """Backward design under test (per-call options)."""
    return DESIGNS[request.param]


def _dev(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


def _empty_rows_are_zero(o, lse, dq, n_empty):
    if n_empty <= 0:
        return
    assert torch.all(o[:, :n_empty] == 0)
    assert torch.all(torch.isneginf(lse[:, :, :n_empty]))
    assert torch.all(dq[:, :n_empty] == 0)


@pytest.mark.parametrize("sq,sk,hq,hkv,d", [
    (130, 333, 2, 2, 64), (333, 130, 2, 2, 128), (1, 700, 2, 1, 128), (257, 1000, 2, 2, 256),
    (700, 300, 2, 2, 256), (200, 517, 4, 1, 128), (300, 301, 2, 2, 64), (64, 2000, 2, 2, 64)])
def test_causal_unequal_lengths_match_oracle(sq, sk, hq, hkv, d, design):
    inp = make_inputs(1, sq, sk, hq, hkv, d, seed=1000 + sq + sk)
    g = _dev(inp)
    scale = 1.0 / math.sqrt(d)
    what = f"s{sq}/{sk} hq{hq} hkv{hkv} d{d}"
    print(f"[bottom-right] {what} design {design}", flush=True)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True, softmax_scale=scale)
    dq, dk, dv = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=True, softmax_scale=scale,
                        options=design)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, True)
    check_o(o, o_ref, what)
    check_lse(lse, lse_ref, what)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True)
    check_grads((dq, dk, dv), ref, what)
    _empty_rows_are_zero(o, lse, dq, sq - sk)


@pytest.mark.parametrize("sq,sk,d", [(300, 900, 128), (900, 300, 64)])
def test_causal_unequal_lengths_deterministic(sq, sk, d, design):
    """Deterministic mode (ordered dQ adds in the fused design) with a shifted
    diagonal: bit-identical over three runs, status clean, oracle parity."""
    hq, hkv = 4, 2
    inp = make_inputs(1, sq, sk, hq, hkv, d, seed=2000 + sq)
    g = _dev(inp)
    scale = 1.0 / math.sqrt(d)
    print(f"[bottom-right det] s{sq}/{sk} d{d} design {design}", flush=True)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True, softmax_scale=scale)
    p = ea.make_params(1, sq, sk, hq, hkv, d, scale, True, True, options=design)
    ws = torch.empty(ea.bwd_workspace_size(p), dtype=torch.uint8, device=DEV)
    runs = []
    for _ in range(3):
        runs.append(ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=True,
                           softmax_scale=scale, deterministic=True, workspace=ws, options=design))
        torch.cuda.synchronize()
        assert ea.bwd_status(p, ws) == 0
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True)
    check_grads(runs[0], ref, f"det s{sq}/{sk} d{d}")


def test_varlen_causal_per_sequence_lengths(design):
    """Packed sequences whose query and key lengths differ per sequence: more
    keys than queries, fewer, equal, no queries, no keys."""
    lq = [40, 300, 7, 0, 129, 513, 5]
    lk = [260, 100, 7, 30, 0, 1000, 5]
    hq, hkv, d = 4, 2, 128
    inp = make_inputs(0, 0, 0, hq, hkv, d, seed=47, lengths=lq, lengths_k=lk)
    g = _dev(inp)
    scale = 1.0 / math.sqrt(d)
    print(f"[bottom-right varlen] design {design}", flush=True)
    o, lse = ea.fwd_varlen(g["q"], g["k"], g["v"], g["cu_seqlens_q"], g["cu_seqlens_k"], max(lq),
                           max(lk), causal=True, softmax_scale=scale)
    dq, dk, dv = ea.bwd_varlen(g["q"], g["k"], g["v"], o, g["do"], lse, g["cu_seqlens_q"],
                               g["cu_seqlens_k"], max(lq), max(lk), causal=True,
                               softmax_scale=scale, options=design)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, True,
                                              inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    check_o(o, o_ref, "varlen bottom-right")
    check_lse(lse, lse_ref, "varlen bottom-right")
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True,
                                    inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    check_grads((dq, dk, dv), ref, "varlen bottom-right")
    # the 300-query sequence has 100 keys: its first 200 rows see nothing
    r0 = lq[0]
    assert torch.all(o[r0:r0 + 200] == 0) and torch.all(dq[r0:r0 + 200] == 0)
    assert torch.all(torch.isneginf(lse[:, r0:r0 + 200]))
    # the sequence with no keys: every row empty
    r4 = sum(lq[:4])
    assert torch.all(o[r4:r4 + lq[4]] == 0) and torch.all(dq[r4:r4 + lq[4]] == 0)


def test_single_query_row_equals_non_causal():
    """Sq = 1 against 3000 keys: the last query sees every key, so causal and
    non-causal results are the same bits (same kernel, no mask hides a key)."""
    inp = make_inputs(2, 1, 3000, 4, 2, 128, seed=5, with_grad=False)
    g = _dev(inp)
    o1, l1 = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    o2, l2 = ea.fwd(g["q"], g["k"], g["v"], causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, _ = oracle.attention_forward(inp["q"], inp["k"], inp["v"], 1 / math.sqrt(128), True)
    check_o(o1, o_ref, "sq1")
