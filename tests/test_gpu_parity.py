"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Sizes here are small enough for the oracle to finish in seconds while still
spanning several tiles and a ragged tail; the full-size workloads are sampled
in test_gpu_fullsize.py.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_71_amd as ea
import oracle
from parity import check_grads, check_lse, check_o, to64
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


DESIGNS = {"recompute": dict(bwd_design=ea.BWD_RECOMPUTE),
           "fused": dict(bwd_design=ea.BWD_FUSED_DQ),
           "stored": dict(bwd_design=ea.BWD_STORED_DS)}


@pytest.fixture(params=list(DESIGNS))
def bwd_mode(request):
    """Backward design under test, as per-call options: the dQ kernel
    recomputing S and dP, the dQ kernel reading the dS the dK/dV kernel stored
    (fixed and packed lengths), or dQ fused into the key-block kernel with
    fp32 atomics (semaphore-ordered when deterministic)."""
    return DESIGNS[request.param]


def _dev(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


def _run_fixed(b, s, hq, hkv, d, causal, seed, scaled=False, det=False, sk=None, bwd=True,
               opts=None):
    sk = s if sk is None else sk
    inp = make_inputs(b, s, sk, hq, hkv, d, seed=seed, scaled_heads=scaled)
    g = _dev(inp)
    scale = 1.0 / math.sqrt(d)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal)
    what = f"b{b} s{s}/{sk} hq{hq} hkv{hkv} d{d} causal{causal}"
    check_o(o, o_ref, what)
    check_lse(lse, lse_ref, what)
    if not bwd:
        return
    dq, dk, dv = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=causal,
                        softmax_scale=scale, deterministic=det, options=opts)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    check_grads((dq, dk, dv), ref, what)


def test_small_workload_fwd_bwd(bwd_mode):
    w = WORKLOADS["small"]
    inp = workload_inputs(w)
    g = _dev(inp)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=False, softmax_scale=w.scale)
    dq, dk, dv = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=False,
                        softmax_scale=w.scale, options=bwd_mode)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], w.scale, False)
    e = check_o(o, o_ref, "small")
    assert e["max_abs"] <= 1e-2          # plain criterion holds at this size
    check_lse(lse, lse_ref, "small")
    check_grads((dq, dk, dv), oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"],
                                                        w.scale, False), "small")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths(d, causal, bwd_mode):
    _run_fixed(1, 300, 2, 2, d, causal, seed=100 + d, opts=bwd_mode)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (4, 1), (6, 3)])
def test_grouped_heads(hq, hkv, bwd_mode):
    _run_fixed(2, 200, hq, hkv, 128, True, seed=7 + hq + hkv, opts=bwd_mode)


def test_non_causal_unequal_lengths():
    _run_fixed(2, 130, 2, 1, 64, False, seed=3, sk=333)


def test_scaled_heads_exercise_rescale(bwd_mode):
    """Q, K x3 on half the heads: logit std ~9, max jumps above tau occur."""
    _run_fixed(1, 1024, 4, 4, 128, True, seed=31, scaled=True, opts=bwd_mode)
    _run_fixed(1, 700, 2, 2, 64, False, seed=32, scaled=True, opts=bwd_mode)


def test_lse_is_optional_and_output_unchanged():
    inp = make_inputs(1, 256, 256, 2, 2, 128, seed=5, with_grad=False)
    g = _dev(inp)
    o1, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    o2, none = ea.fwd(g["q"], g["k"], g["v"], causal=True, return_lse=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_matches_oracle(causal, bwd_mode):
    lengths = [1, 17, 300, 0, 513, 64, 129]
    hq, hkv, d = 4, 2, 128
    inp = make_inputs(0, 0, 0, hq, hkv, d, seed=41, lengths=lengths)
    g = _dev(inp)
    scale = 1.0 / math.sqrt(d)
    mx = max(lengths)
    o, lse = ea.fwd_varlen(g["q"], g["k"], g["v"], g["cu_seqlens_q"], g["cu_seqlens_k"], mx, mx,
                           causal=causal, softmax_scale=scale)
    dq, dk, dv = ea.bwd_varlen(g["q"], g["k"], g["v"], o, g["do"], lse, g["cu_seqlens_q"],
                               g["cu_seqlens_k"], mx, mx, causal=causal, softmax_scale=scale,
                               options=bwd_mode)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal,
                                              inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    check_o(o, o_ref, "varlen")
    check_lse(lse, lse_ref, "varlen")
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal,
                                    inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    check_grads((dq, dk, dv), ref, "varlen")


@pytest.mark.parametrize("nseq,uses_list", [(250, True), (420, False)])
def test_varlen_many_sequences(nseq, uses_list, bwd_mode):
    """Many short packed sequences: up to the ranking bound the key-block
    kernel walks one longest-first list over all key blocks; past it, the
    per-sequence order. Both must match the oracle."""
    rng = np.random.default_rng(nseq)
    lengths = [int(x) for x in rng.integers(0, 100, nseq)]
    hq, hkv, d = 2, 1, 64
    inp = make_inputs(0, 0, 0, hq, hkv, d, seed=47, lengths=lengths)
    cu = inp["cu_seqlens_q"].tolist()
    p = ea.make_params(nseq, max(lengths), max(lengths), hq, hkv, d, 0.125, True,
                       total_q=cu[-1], total_k=cu[-1])
    assert (ea.varlen_key_order(p, cu, cu) is not None) == uses_list
    g = _dev(inp)
    mx = max(lengths)
    o, lse = ea.fwd_varlen(g["q"], g["k"], g["v"], g["cu_seqlens_q"], g["cu_seqlens_k"], mx, mx,
                           causal=True, softmax_scale=0.125)
    dq, dk, dv = ea.bwd_varlen(g["q"], g["k"], g["v"], o, g["do"], lse, g["cu_seqlens_q"],
                               g["cu_seqlens_k"], mx, mx, causal=True, softmax_scale=0.125,
                               options=bwd_mode)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], 0.125, True,
                                              inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    what = f"varlen {nseq} sequences"
    check_o(o, o_ref, what)
    check_lse(lse, lse_ref, what)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], 0.125, True,
                                    inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    check_grads((dq, dk, dv), ref, what)


@pytest.mark.parametrize("lq,lk", [([0, 0, 0], [0, 0, 0]), ([5, 300, 0], [0, 0, 0]),
                                   ([0, 0, 0], [70, 0, 260])])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_with_no_queries_or_no_keys(lq, lk, causal, bwd_mode):
    """Packed batches whose queries or keys are all empty (tensors with no
    elements, null data pointers): rows that see no key give O = 0, LSE = -inf
    and dQ = 0; keys that no query sees give dK = dV = 0."""
    hq, hkv, d = 4, 2, 128
    inp = make_inputs(0, 0, 0, hq, hkv, d, seed=53, lengths=lq, lengths_k=lk)
    g = _dev(inp)
    o, lse = ea.fwd_varlen(g["q"], g["k"], g["v"], g["cu_seqlens_q"], g["cu_seqlens_k"],
                           max(lq), max(lk), causal=causal, softmax_scale=0.1)
    dq, dk, dv = ea.bwd_varlen(g["q"], g["k"], g["v"], o, g["do"], lse, g["cu_seqlens_q"],
                               g["cu_seqlens_k"], max(lq), max(lk), causal=causal,
                               softmax_scale=0.1, options=bwd_mode)
    torch.cuda.synchronize()
    assert o.shape == g["q"].shape and dk.shape == g["k"].shape
    assert torch.all(o == 0) and torch.all(dq == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(dk == 0) and torch.all(dv == 0)


@pytest.mark.parametrize("sq,sk", [(200, 0), (0, 200), (0, 0)])
def test_fixed_length_with_no_queries_or_no_keys(sq, sk, bwd_mode):
    b, hq, hkv, d = 2, 4, 2, 64
    inp = make_inputs(b, sq, sk, hq, hkv, d, seed=57)
    g = _dev(inp)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True, softmax_scale=0.1)
    dq, dk, dv = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=True,
                        softmax_scale=0.1, options=bwd_mode)
    torch.cuda.synchronize()
    assert o.shape == (b, sq, hq, d) and dk.shape == (b, sk, hkv, d)
    assert torch.all(o == 0) and torch.all(dq == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_varlen_non_causal_different_key_lengths(bwd_mode):
    lq, lk = [40, 300, 7], [260, 0, 90]
    hq, hkv, d = 2, 1, 64
    inp = make_inputs(0, 0, 0, hq, hkv, d, seed=43, lengths=lq, lengths_k=lk)
    g = _dev(inp)
    scale = 0.125
    o, lse = ea.fwd_varlen(g["q"], g["k"], g["v"], g["cu_seqlens_q"], g["cu_seqlens_k"], max(lq),
                           max(lk), causal=False, softmax_scale=scale)
    dq, dk, dv = ea.bwd_varlen(g["q"], g["k"], g["v"], o, g["do"], lse, g["cu_seqlens_q"],
                               g["cu_seqlens_k"], max(lq), max(lk), softmax_scale=scale,
                               options=bwd_mode)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, False,
                                              inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    check_o(o, o_ref, "varlen-k")
    check_lse(lse, lse_ref, "varlen-k")      # the empty key sequence gives -inf rows
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, False,
                                    inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    assert torch.all(dq[40:340] == 0)        # rows that see no key have zero gradient
    check_grads((dq, dk, dv), ref, "varlen-k")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_deterministic_backward_is_bit_identical(d, bwd_mode):
    s, hq, hkv = 640, 4, 2
    inp = make_inputs(1, s, s, hq, hkv, d, seed=51 + d)
    g = _dev(inp)
    scale = 1.0 / math.sqrt(d)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True, softmax_scale=scale)
    p = ea.make_params(1, s, s, hq, hkv, d, scale, True, True, options=bwd_mode)
    ws = torch.empty(ea.bwd_workspace_size(p), dtype=torch.uint8, device=DEV)
    runs = []
    for _ in range(3):
        runs.append(ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=True,
                           softmax_scale=scale, deterministic=True, workspace=ws,
                           options=bwd_mode))
        torch.cuda.synchronize()
        assert ea.bwd_status(p, ws) == 0
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True)
    check_grads(runs[0], ref, f"det d{d}")


def test_backward_phases_equal_full_backward(bwd_mode):
    s, hq, hkv, d = 384, 2, 2, 128
    inp = make_inputs(1, s, s, hq, hkv, d, seed=61)
    g = _dev(inp)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    p = ea.make_params(1, s, s, hq, hkv, d, 1.0 / math.sqrt(d), True, True, options=bwd_mode)
    ws = torch.empty(ea.bwd_workspace_size(p), dtype=torch.uint8, device=DEV)
    full = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=True, deterministic=True,
                  options=bwd_mode)
    dq, dk, dv = (torch.empty_like(x) for x in (g["q"], g["k"], g["v"]))
    for ph in (ea.BWD_PREPROCESS, ea.BWD_MAIN, ea.BWD_DQ, ea.BWD_POSTPROCESS):
        ea.bwd_phases(p, ph, g["q"], g["k"], g["v"], o, g["do"], lse, dq, dk, dv, ws)
    torch.cuda.synchronize()
    for a, b in zip(full, (dq, dk, dv)):
        assert torch.equal(a, b)


def test_forward_independent_of_tile_order():
    """No cross-tile reduction in the forward: any tile order gives the same bits."""
    inp = make_inputs(2, 1024, 1024, 8, 8, 128, seed=71, with_grad=False)
    g = _dev(inp)
    o1, l1 = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    o2, l2 = ea.fwd(g["q"], g["k"], g["v"], causal=True, options=dict(tile_order=1))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("emu,tau", [(2, 8), (1, 8), (4, 8), (0, 0), (0, 16), (4, 0)])
def test_tau_and_exp_emulation_variants_match_oracle(d, emu, tau):
    """The forward's knobs (FMA-path exp2 on emu of every 8 elements; rescale
    threshold tau in log2 units) all reach the definition: the conditional
    rescale and the polynomial change rounding, not the result."""
    inp = make_inputs(1, 700, 700, 2, 2, d, seed=81 + d, scaled_heads=True, with_grad=False)
    g = _dev(inp)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True,
                    options=dict(exp_emulation=emu, tau=-1.0 if tau == 0 else float(tau)))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], 1 / math.sqrt(d), True)
    e = check_o(o, o_ref, f"emu{emu} tau{tau} d{d}")
    el = check_lse(lse, lse_ref, f"emu{emu} tau{tau} d{d}")
    print(f"[tau/exp accuracy] d={d} emu={emu} tau={tau} O {e} LSE max-abs {el:.3e}")


def test_gqa_equals_repeated_kv_on_gpu():
    inp = make_inputs(1, 256, 256, 8, 2, 64, seed=91)
    g = _dev(inp)
    o1, l1 = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    kr = g["k"].repeat_interleave(4, dim=2).contiguous()
    vr = g["v"].repeat_interleave(4, dim=2).contiguous()
    o2, l2 = ea.fwd(g["q"], kr, vr, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_deterministic_main_without_preprocess_stays_in_bounds():
    """Regression: a MAIN phase launched again without PREPROCESS used to draw
    tickets past the grid. It must now terminate in bounds; a later full
    backward (which clears the state) is again bit-identical to the first."""
    s, hq, hkv, d = 512, 2, 2, 128
    inp = make_inputs(1, s, s, hq, hkv, d, seed=111)
    g = _dev(inp)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    fused = dict(bwd_design=ea.BWD_FUSED_DQ)   # the ticket / semaphore path
    p = ea.make_params(1, s, s, hq, hkv, d, 1.0 / math.sqrt(d), True, True, options=fused)
    ws = torch.empty(ea.bwd_workspace_size(p), dtype=torch.uint8, device=DEV)
    first = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=True, deterministic=True,
                   workspace=ws, options=fused)
    dq, dk, dv = (torch.empty_like(x) for x in (g["q"], g["k"], g["v"]))
    short = ea.make_params(1, s, s, hq, hkv, d, 1.0 / math.sqrt(d), True, True,
                           options=dict(fused, spin_limit=1 << 14))
    ea.bwd_phases(short, ea.BWD_PREPROCESS | ea.BWD_MAIN | ea.BWD_POSTPROCESS, g["q"], g["k"],
                  g["v"], o, g["do"], lse, dq, dk, dv, ws)
    ea.bwd_phases(short, ea.BWD_MAIN, g["q"], g["k"], g["v"], o, g["do"], lse, dq, dk, dv, ws)
    torch.cuda.synchronize()
    again = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=True, deterministic=True,
                   workspace=ws, options=fused)
    torch.cuda.synchronize()
    assert ea.bwd_status(p, ws) == 0
    for a, b in zip(first, again):
        assert torch.equal(a, b)


@pytest.mark.parametrize("varlen", [False, True])
def test_persistent_and_one_shot_launches_agree(varlen, bwd_mode):
    """Resident workgroups looping over tiles compute every tile exactly as a
    one-workgroup-per-tile grid does: same bits for O, LSE, dQ, dK, dV."""
    d = 128
    if varlen:
        inp = make_inputs(0, 0, 0, 4, 2, d, seed=121, lengths=[3000, 17, 1200, 640, 2500, 1])
    else:
        inp = make_inputs(2, 3000, 3000, 8, 4, d, seed=122)
    g = _dev(inp)

    def run(opts):
        if varlen:
            mx = 3000
            o, lse = ea.fwd_varlen(g["q"], g["k"], g["v"], g["cu_seqlens_q"], g["cu_seqlens_k"],
                                   mx, mx, causal=True, options=opts)
            grads = ea.bwd_varlen(g["q"], g["k"], g["v"], o, g["do"], lse, g["cu_seqlens_q"],
                                  g["cu_seqlens_k"], mx, mx, causal=True, options=opts)
        else:
            o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True, options=opts)
            grads = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=True, options=opts)
        torch.cuda.synchronize()
        return (o, lse) + tuple(grads)

    a = run(bwd_mode)
    b = run(dict(bwd_mode, one_shot_grid=1))
    fused = bwd_mode["bwd_design"] == ea.BWD_FUSED_DQ
    for i, (x, y) in enumerate(zip(a, b)):
        if fused and i == 2:   # dQ of the fused design: unordered fp32 atomics
            continue
        assert torch.equal(x, y), i


def test_designs_back_to_back_without_global_state():
    """Designs are per-call options: interleaved calls with different designs on
    the same inputs each meet the oracle bar, and the two split designs (same
    dK/dV kernel arithmetic) give bit-equal dK, dV."""
    s, hq, hkv, d = 700, 4, 2, 128
    inp = make_inputs(1, s, s, hq, hkv, d, seed=131)
    g = _dev(inp)
    scale = 1.0 / math.sqrt(d)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True, softmax_scale=scale)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True)
    seq = [ea.BWD_RECOMPUTE, ea.BWD_STORED_DS, ea.BWD_FUSED_DQ, ea.BWD_RECOMPUTE, ea.BWD_STORED_DS]
    out = [ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=True, softmax_scale=scale,
                  options=dict(bwd_design=b)) for b in seq]
    torch.cuda.synchronize()
    for b, r in zip(seq, out):
        check_grads(r, ref, f"design {b}")
    for a, b in ((0, 3), (1, 4), (0, 1)):
        assert torch.equal(out[a][1], out[b][1]) and torch.equal(out[a][2], out[b][2])
    assert torch.equal(out[0][0], out[3][0]) and torch.equal(out[1][0], out[4][0])


@pytest.mark.parametrize("hq,hkv", [(4, 1), (6, 2)])
def test_stored_ds_lengths_beyond_declared_maximum_stay_in_the_workspace(hq, hkv):
    """Packed lengths longer than the declared maxima (a caller error the
    device cannot see before it runs): the stored-dS bound is computed from the
    declared maxima, and every query head's stores must stay inside the
    workspace. The workspace is a slice of a larger buffer filled with a
    canary; the canary must survive. dK and dV do not depend on the stored dS
    and must still meet the oracle bar."""
    lengths = [512, 300, 700]
    declared = 256
    d = 128
    inp = make_inputs(0, 0, 0, hq, hkv, d, seed=141, lengths=lengths)
    g = _dev(inp)
    scale = 1.0 / math.sqrt(d)
    mx = max(lengths)
    o, lse = ea.fwd_varlen(g["q"], g["k"], g["v"], g["cu_seqlens_q"], g["cu_seqlens_k"], mx, mx,
                           causal=True, softmax_scale=scale)
    opts = dict(bwd_design=ea.BWD_STORED_DS)
    p = ea.make_params(len(lengths), declared, declared, hq, hkv, d, scale, True, False,
                       total_q=sum(lengths), total_k=sum(lengths), options=opts)
    need = ea.bwd_workspace_size(p, varlen=True)
    pad = 1 << 20
    buf = torch.full((pad + need + pad,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = buf[pad:pad + need]
    print(f"[canary] hq{hq} hkv{hkv} lengths {lengths} declared {declared} ws {need}", flush=True)
    dq, dk, dv = ea.bwd_varlen(g["q"], g["k"], g["v"], o, g["do"], lse, g["cu_seqlens_q"],
                               g["cu_seqlens_k"], declared, declared, causal=True,
                               softmax_scale=scale, workspace=ws, options=opts)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 0xA5) and torch.all(buf[pad + need:] == 0xA5)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True,
                                    inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    from parity import rel_l2
    assert rel_l2(dk, ref[1]) <= 2e-2 and rel_l2(dv, ref[2]) <= 2e-2


@pytest.mark.parametrize("varlen", [False, True])
def test_head_split_matches_oracle_and_is_reproducible(varlen, bwd_mode):
    """The query heads of an MQA group split over 1, 2 and 8 key-block
    workgroups: every split matches the oracle, and a split run gives the same
    dK, dV bits twice (its fp32 partials are added in part order)."""
    hq, hkv, d = 8, 1, 128
    scale = 1.0 / math.sqrt(d)
    if varlen:
        lengths = [300, 0, 700, 129]
        inp = make_inputs(0, 0, 0, hq, hkv, d, seed=801, lengths=lengths)
    else:
        inp = make_inputs(1, 700, 700, hq, hkv, d, seed=802)
    g = _dev(inp)
    if varlen:
        mx = max(lengths)
        cu = (g["cu_seqlens_q"], g["cu_seqlens_k"])
        o, lse = ea.fwd_varlen(g["q"], g["k"], g["v"], *cu, mx, mx, causal=True,
                               softmax_scale=scale)
        ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True,
                                        inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    else:
        o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True, softmax_scale=scale)
        ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True)

    def run(split):
        opts = dict(bwd_design_opts, head_split=split)
        if varlen:
            out = ea.bwd_varlen(g["q"], g["k"], g["v"], o, g["do"], lse, *cu, mx, mx, causal=True,
                                softmax_scale=scale, options=opts)
        else:
            out = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=True,
                         softmax_scale=scale, options=opts)
        torch.cuda.synchronize()
        return out

    bwd_design_opts = bwd_mode
    for split in (1, 2, 8):
        print(f"[head split] varlen={varlen} {bwd_mode} split={split}", flush=True)
        grads = run(split)
        check_grads(grads, ref, f"head split {split} varlen {varlen}")
        if split == 8:
            again = run(split)
            assert torch.equal(grads[1], again[1]) and torch.equal(grads[2], again[2])


def test_head_split_leaves_packed_rows_past_the_last_sequence_alone():
    """Packed K / V with rows past the last sequence (total_k above
    cu_seqlens_k[batch]): the split backward's reduction writes dK, dV of the
    sequences' rows only (a canary survives in the rest), and those rows
    match the unsplit run."""
    lengths = [300, 129]
    hq, hkv, d, pad = 8, 1, 128, 64
    scale = 1.0 / math.sqrt(d)
    inp = make_inputs(0, 0, 0, hq, hkv, d, seed=811, lengths=lengths)
    g = _dev(inp)
    tk = g["k"].shape[0]
    zeros = torch.zeros((pad, hkv, d), dtype=g["k"].dtype, device=DEV)
    k = torch.cat([g["k"], zeros]).contiguous()
    v = torch.cat([g["v"], zeros]).contiguous()
    cu_q, cu_k = g["cu_seqlens_q"], g["cu_seqlens_k"]
    mx = max(lengths)
    o, lse = ea.fwd_varlen(g["q"], k, v, cu_q, cu_k, mx, mx, causal=True, softmax_scale=scale)
    results = {}
    for split in (1, 2):
        p = ea.make_params(len(lengths), mx, mx, hq, hkv, d, scale, True, total_q=g["q"].shape[0],
                           total_k=tk + pad, options=dict(head_split=split))
        assert ea.bwd_head_split(p, True) == split
        ws = torch.empty(ea.bwd_workspace_size(p, True), dtype=torch.uint8, device=DEV)
        dq = torch.empty_like(g["q"])
        dk = torch.full_like(k, 7.0)
        dv = torch.full_like(v, 7.0)
        ea.bwd_phases(p, ea.BWD_ALL, g["q"], k, v, o, g["do"], lse, dq, dk, dv, ws, cu_q, cu_k)
        torch.cuda.synchronize()
        assert torch.all(dk[tk:] == 7.0) and torch.all(dv[tk:] == 7.0), split
        results[split] = (dk[:tk].float(), dv[:tk].float())
    for a_, b_ in zip(results[1], results[2]):
        assert torch.linalg.vector_norm(a_ - b_) <= 1e-2 * torch.linalg.vector_norm(a_)


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_plan_gives_the_same_bits(causal, bwd_mode):
    """A cached varlen plan (one schedule launch, reused by every call) gives
    the bits of the calls that compute their own schedule, over three reuses
    of the plan (its tile counters stay valid across launches); deterministic
    mode so that every design's dQ is bitwise comparable."""
    lengths = [3000, 17, 1200, 640, 2500, 1, 0, 777]
    hq, hkv, d = 4, 2, 128
    inp = make_inputs(0, 0, 0, hq, hkv, d, seed=151, lengths=lengths)
    g = _dev(inp)
    mx = max(lengths)
    cq, ck = g["cu_seqlens_q"], g["cu_seqlens_k"]
    plan = ea.varlen_plan(cq, ck, mx, mx, sum(lengths), sum(lengths), hq, hkv, d, causal)

    def run(pl):
        o, lse = ea.fwd_varlen(g["q"], g["k"], g["v"], cq, ck, mx, mx, causal=causal, plan=pl)
        grads = ea.bwd_varlen(g["q"], g["k"], g["v"], o, g["do"], lse, cq, ck, mx, mx,
                              causal=causal, deterministic=True, options=bwd_mode, plan=pl)
        torch.cuda.synchronize()
        return (o, lse) + tuple(grads)

    ref = run(None)
    for _ in range(3):
        got = run(plan)
        for i, (x, y) in enumerate(zip(ref, got)):
            assert torch.equal(x, y), i
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], 1 / math.sqrt(d),
                                              causal, inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    check_o(got[0], o_ref, "plan")
    check_lse(got[1], lse_ref, "plan")
