"""The allocation-free backward (attn_bwd_noalloc) against attn_bwd.

attn_bwd_noalloc runs the recomputing backward with its workspace in the
library's static device scratch instead of a caller-provided one. Through the
C ABI it must give the same bits as attn_bwd with the recomputing design, on
two calls in a row (the second smaller, reusing the scratch the first left
behind), and refuse shapes beyond the scratch before launching anything.
"""
import ctypes
import math

import pytest
import torch

import exact_attention_71_amd as ea
from workloads import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RECOMPUTE = dict(bwd_design=ea.BWD_RECOMPUTE)


def _case(b, s, hq, hkv, d, causal, seed):
    inp = make_inputs(b, s, s, hq, hkv, d, seed=seed)
    g = {k: v.to(DEV) for k, v in inp.items()}
    scale = 1.0 / math.sqrt(d)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=causal, softmax_scale=scale)
    return g, o, lse, scale


def test_noalloc_backward_equals_attn_bwd_on_two_calls_in_a_row():
    lib = ea.load()
    for (b, s, hq, hkv, d, causal, seed) in ((2, 1500, 8, 2, 128, True, 301),
                                             (1, 300, 2, 1, 64, False, 302)):
        print(f"[noalloc] b{b} s{s} hq{hq} hkv{hkv} d{d} causal{causal}", flush=True)
        g, o, lse, scale = _case(b, s, hq, hkv, d, causal, seed)
        want = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=causal,
                      softmax_scale=scale, options=RECOMPUTE)
        p = ea.make_params(b, s, s, hq, hkv, d, scale, causal, False)
        dq, dk, dv = (torch.full_like(g[n], float("nan")) for n in ("q", "k", "v"))
        st = lib.attn_bwd_noalloc(ctypes.byref(p), g["q"].data_ptr(), g["k"].data_ptr(),
                                  g["v"].data_ptr(), o.data_ptr(), g["do"].data_ptr(),
                                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        for a, w in zip((dq, dk, dv), want):
            assert torch.equal(a, w)
        # the binding's wrapper (argument marshalling only) gives the same bits
        got = ea.bwd_noalloc(g["q"], g["k"], g["v"], o, g["do"], lse, causal=causal,
                             softmax_scale=scale)
        torch.cuda.synchronize()
        for a, w in zip(got, want):
            assert torch.equal(a, w)


def test_noalloc_backward_refuses_what_it_cannot_hold():
    lib = ea.load()
    fake = 0x10000   # never dereferenced: every refusal happens before a launch
    args = [fake] * 9 + [None]
    # 32 MiB of scratch holds 8 bytes per (query row, query head): 2^22 pairs
    big = ea.make_params(1, 1 << 19, 1 << 19, 8, 8, 64, 0.125, True, False)
    assert lib.attn_bwd_noalloc(ctypes.byref(big), *args) == 2
    for design in (ea.BWD_STORED_DS, ea.BWD_FUSED_DQ):
        p = ea.make_params(1, 256, 256, 2, 2, 128, 0.1, True, False,
                           options=dict(bwd_design=design))
        assert lib.attn_bwd_noalloc(ctypes.byref(p), *args) == 2
    p = ea.make_params(1, 256, 256, 2, 2, 128, 0.1, True, False)
    assert lib.attn_bwd_noalloc(ctypes.byref(p), None, *args[1:]) == 1
