"""Block-sparse masks on the HIP path, against the float64 oracle.

One byte per 128 x 128 block of (query, key) pairs per (batch, query head),
ANDed with the causal rule; rows that see no key get O = 0, LSE = -inf and
zero gradients. Every backward design that takes a mask is compared with the
oracle; the stored-dS design refuses one.
"""
import math

import pytest
import torch

import exact_attention_71_amd as ea
import oracle
from parity import check_grads, check_lse, check_o
from workloads import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DESIGNS = {"auto": {}, "recompute": dict(bwd_design=ea.BWD_RECOMPUTE),
           "fused": dict(bwd_design=ea.BWD_FUSED_DQ)}


def _mask(b, h, sq, sk, seed, density=0.5):
    nqb, nkb = -(-sq // 128), -(-sk // 128)
    g = torch.Generator().manual_seed(seed)
    return torch.rand((b, h, nqb, nkb), generator=g) < density


@pytest.mark.parametrize("design", list(DESIGNS))
@pytest.mark.parametrize("b,sq,sk,hq,hkv,d,causal", [
    (1, 700, 700, 2, 2, 128, True), (2, 300, 520, 4, 2, 64, False),
    (1, 1100, 1100, 4, 1, 128, False), (1, 513, 513, 2, 2, 256, True),
    (1, 400, 900, 2, 2, 128, True)])
def test_block_mask_matches_oracle(b, sq, sk, hq, hkv, d, causal, design):
    inp = make_inputs(b, sq, sk, hq, hkv, d, seed=600 + sq + sk + d)
    m = _mask(b, hq, sq, sk, seed=sq + d)
    g = {k: v.to(DEV) for k, v in inp.items()}
    md = m.to(DEV)
    scale = 1.0 / math.sqrt(d)
    what = f"mask b{b} s{sq}/{sk} hq{hq} hkv{hkv} d{d} causal{causal} {design}"
    print(f"[block mask] {what}", flush=True)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=causal, softmax_scale=scale, block_mask=md)
    dq, dk, dv = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=causal,
                        softmax_scale=scale, options=DESIGNS[design], block_mask=md)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal,
                                              block_mask=m)
    check_o(o, o_ref, what)
    check_lse(lse, lse_ref, what)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal,
                                    block_mask=m)
    check_grads((dq, dk, dv), ref, what)
    # rows whose every block is cleared (or above a causal diagonal) see no key
    dead = torch.from_numpy(lse_ref == float("-inf"))
    if dead.any():
        od = o.cpu().transpose(1, 2)[dead]
        assert torch.all(od == 0)
        assert torch.all(dq.cpu().transpose(1, 2)[dead] == 0)


@pytest.mark.parametrize("design", ["recompute", "fused"])
@pytest.mark.parametrize("sq,sk,hkv,d,causal,window", [
    (300, 9000, 2, 128, False, None), (300, 9000, 1, 256, False, None),
    (600, 12000, 2, 64, False, None), (4096, 4096, 2, 128, True, 3)])
def test_block_mask_over_many_key_tiles(sq, sk, hkv, d, causal, window, design):
    """More key tiles than a wavefront has lanes (the kernels list the visible
    ones 64 at a time), a sparse random mask or a band of blocks around the
    diagonal (sliding window)."""
    b, hq = 1, 2
    inp = make_inputs(b, sq, sk, hq, hkv, d, seed=700 + sk + d)
    if window is None:
        m = _mask(b, hq, sq, sk, seed=sk + d, density=0.3)
    else:
        i = torch.arange(-(-sq // 128))[:, None]
        j = torch.arange(-(-sk // 128))[None, :]
        m = ((i - j).abs() <= window).expand(b, hq, -1, -1).contiguous()
    g = {k: v.to(DEV) for k, v in inp.items()}
    scale = 1.0 / math.sqrt(d)
    what = f"mask s{sq}/{sk} hkv{hkv} d{d} causal{causal} window{window} {design}"
    print(f"[block mask] {what}", flush=True)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=causal, softmax_scale=scale,
                    block_mask=m.to(DEV))
    dq, dk, dv = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=causal,
                        softmax_scale=scale, options=DESIGNS[design], block_mask=m.to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal,
                                              block_mask=m)
    check_o(o, o_ref, what)
    check_lse(lse, lse_ref, what)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal,
                                    block_mask=m)
    check_grads((dq, dk, dv), ref, what)


def _masked_case(b, sq, sk, hq, hkv, d, causal, m, what, deterministic=False, options=None):
    inp = make_inputs(b, sq, sk, hq, hkv, d, seed=800 + sq + sk + d)
    g = {k: v.to(DEV) for k, v in inp.items()}
    md = m.to(DEV)
    scale = 1.0 / math.sqrt(d)
    print(f"[block mask] {what}", flush=True)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=causal, softmax_scale=scale, block_mask=md)
    grads = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=causal, softmax_scale=scale,
                   deterministic=deterministic, options=options, block_mask=md)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal,
                                              block_mask=m)
    check_o(o, o_ref, what)
    check_lse(lse, lse_ref, what)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal,
                                    block_mask=m)
    check_grads(grads, ref, what)


@pytest.mark.parametrize("design", ["recompute", "fused", "deterministic"])
@pytest.mark.parametrize("sq,sk,hq,hkv,d", [
    (650, 700, 4, 2, 128), (550, 700, 2, 1, 64), (450, 520, 2, 2, 256)])
def test_block_mask_rows_cut_by_the_causal_diagonal(sq, sk, hq, hkv, d, design):
    """Causal, with lengths whose diagonal makes a key block's first visible
    query block fall inside a 128-row mask row, and whose last mask row is
    partial: the dK/dV walk over the listed mask rows starts and ends inside
    a row. The deterministic design walks every step (its semaphore chain
    counts each key block at each query block)."""
    m = _mask(1, hq, sq, sk, seed=sq + sk + d, density=0.4)
    det = design == "deterministic"
    opts = DESIGNS["fused" if det else design]
    _masked_case(1, sq, sk, hq, hkv, d, True, m,
                 f"mask cut s{sq}/{sk} hq{hq} hkv{hkv} d{d} {design}", det, opts)


@pytest.mark.parametrize("design", ["recompute", "fused"])
def test_block_mask_with_more_mask_rows_than_a_workgroup_lists(design):
    """16 query heads per KV head (no head split) over 131 mask rows: 2096
    (head, row) pairs per key block, more than the dK/dV kernel lists, so it
    walks every step and skips none; the result is still the oracle's."""
    b, sq, sk, hq, hkv, d = 1, 16700, 300, 16, 1, 64
    m = _mask(b, hq, sq, sk, seed=31, density=0.3)
    _masked_case(b, sq, sk, hq, hkv, d, False, m, f"mask dense walk {design}",
                 options=dict(DESIGNS[design], head_split=1))


def test_shared_mask_broadcasts_over_batches_and_heads():
    """A [1, 1, nqb, nkb] mask applies to every (batch, head) (strides 0)."""
    b, s, hq, d = 2, 640, 4, 128
    inp = make_inputs(b, s, s, hq, hq, d, seed=611)
    m1 = _mask(1, 1, s, s, seed=612)
    full = m1.expand(b, hq, -1, -1).contiguous()
    g = {k: v.to(DEV) for k, v in inp.items()}
    o1, l1 = ea.fwd(g["q"], g["k"], g["v"], causal=True, block_mask=m1.to(DEV))
    o2, l2 = ea.fwd(g["q"], g["k"], g["v"], causal=True, block_mask=full.to(DEV))
    g1 = ea.bwd(g["q"], g["k"], g["v"], o1, g["do"], l1, causal=True, block_mask=m1.to(DEV))
    g2 = ea.bwd(g["q"], g["k"], g["v"], o2, g["do"], l2, causal=True, block_mask=full.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)
    o_ref, _ = oracle.attention_forward(inp["q"], inp["k"], inp["v"], 1 / math.sqrt(d), True,
                                        block_mask=full)
    check_o(o1, o_ref, "shared mask")


@pytest.mark.parametrize("design", list(DESIGNS))
def test_all_set_mask_gives_the_bits_of_no_mask(design):
    """The masked kernels with every block set compute exactly what the
    unmasked ones do."""
    b, s, hq, hkv, d = 1, 1000, 4, 2, 128
    inp = make_inputs(b, s, s, hq, hkv, d, seed=621)
    g = {k: v.to(DEV) for k, v in inp.items()}
    ones = torch.ones((1, 1, 8, 8), dtype=torch.bool, device=DEV)
    o1, l1 = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    o2, l2 = ea.fwd(g["q"], g["k"], g["v"], causal=True, block_mask=ones)
    det = DESIGNS[design].get("bwd_design") == ea.BWD_FUSED_DQ
    opts = dict(DESIGNS[design], bwd_design=ea.BWD_RECOMPUTE) if design == "auto" else DESIGNS[design]
    g1 = ea.bwd(g["q"], g["k"], g["v"], o1, g["do"], l1, causal=True, deterministic=det,
                options=opts)
    g2 = ea.bwd(g["q"], g["k"], g["v"], o1, g["do"], l1, causal=True, deterministic=det,
                options=opts, block_mask=ones)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


def test_stored_ds_and_varlen_refuse_a_mask():
    b, s, hq, d = 1, 256, 2, 128
    inp = make_inputs(b, s, s, hq, hq, d, seed=631)
    g = {k: v.to(DEV) for k, v in inp.items()}
    m = torch.ones((1, 1, 2, 2), dtype=torch.bool, device=DEV)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True, block_mask=m)
    with pytest.raises(ea.AttnError) as e:
        ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=True, block_mask=m,
               options=dict(bwd_design=ea.BWD_STORED_DS))
    assert e.value.status in (1, 2)
    with pytest.raises(ea.AttnError):
        ea.fwd(g["q"], g["k"], g["v"], causal=True, block_mask=m, options=dict(exp_emulation=2))
