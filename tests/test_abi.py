"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/attn71.h declares, validates arguments before touching
the device, sizes workspaces, and produces the documented tile orders."""
import collections
import ctypes
import os
import re

import pytest

import exact_attention_71_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn71.h")

INVALID, UNSUPPORTED, WS_SMALL = 1, 2, 3
SIZE_MAX = ctypes.c_size_t(-1).value


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = ea.load()
    names = _declared()
    assert "attn_fwd" in names and "attn_bwd_varlen" in names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(ea.EXPORTS)


def test_version_and_status_strings():
    lib = ea.load()
    assert ea.version() == 100
    assert lib.attn_status_string(0) == b"OK"
    assert lib.attn_status_string(3) == b"workspace too small"
    assert lib.attn_status_string(99) == b"unknown status"


def _p(**kw):
    base = dict(batch=2, seqlen_q=300, seqlen_k=300, heads_q=4, heads_kv=2, head_dim=128,
                scale=0.088, causal=False, deterministic=False)
    base.update(kw)
    return ea.make_params(base["batch"], base["seqlen_q"], base["seqlen_k"], base["heads_q"],
                          base["heads_kv"], base["head_dim"], base["scale"], base["causal"],
                          base["deterministic"], base.get("total_q", 0), base.get("total_k", 0))


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), UNSUPPORTED), (dict(head_dim=32), UNSUPPORTED),
    (dict(heads_q=3, heads_kv=2), INVALID), (dict(heads_kv=0), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=float("nan")), INVALID), (dict(scale=-1.0), INVALID),
    (dict(seqlen_k=-1), INVALID), (dict(batch=-1), INVALID),
    (dict(seqlen_q=1 << 24, heads_q=64, heads_kv=64), UNSUPPORTED),
])
def test_forward_rejects_bad_parameters(kw, status):
    lib = ea.load()
    p = _p(**kw)
    st = lib.attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == status
    st = lib.attn_bwd(ctypes.byref(p), *([FAKE] * 9), FAKE, 1 << 30, None)
    assert st == status


def test_causal_with_unequal_lengths_passes_validation():
    """Causal with Sq != Sk (bottom-right diagonal) is accepted: with a null
    q pointer the call must fail on the pointer, not on the shape."""
    lib = ea.load()
    for sq, sk in ((300, 299), (17, 4096), (4096, 17)):
        p = _p(causal=True, seqlen_q=sq, seqlen_k=sk)
        assert lib.attn_fwd(ctypes.byref(p), None, FAKE, FAKE, FAKE, None, None, 0, None) == INVALID
        assert lib.attn_fwd_workspace_size(ctypes.byref(p), 0) == 0
        assert 0 < lib.attn_bwd_workspace_size(ctypes.byref(p), 0) < (1 << 40)


def test_forward_rejects_null_and_misaligned_pointers():
    lib = ea.load()
    p = _p()
    assert lib.attn_fwd(ctypes.byref(p), None, FAKE, FAKE, FAKE, None, None, 0, None) == INVALID
    assert lib.attn_fwd(ctypes.byref(p), FAKE + 2, FAKE, FAKE, FAKE, None, None, 0, None) == INVALID
    assert lib.attn_fwd(None, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == INVALID
    assert lib.attn_fwd_varlen(ctypes.byref(p), None, None, FAKE, FAKE, FAKE, FAKE, None, None,
                               0, None) == INVALID


def test_backward_requires_lse_and_workspace():
    lib = ea.load()
    p = _p()
    need = ea.bwd_workspace_size(p)
    args = [FAKE] * 9   # q k v o dout lse dq dk dv
    args[5] = None      # lse
    assert lib.attn_bwd(ctypes.byref(p), *args, FAKE, need, None) == INVALID
    assert lib.attn_bwd(ctypes.byref(p), *([FAKE] * 9), FAKE, need - 1, None) == WS_SMALL
    assert lib.attn_bwd(ctypes.byref(p), *([FAKE] * 9), None, need, None) == INVALID
    assert lib.attn_bwd_phases(ctypes.byref(p), None, None, 0, *([FAKE] * 9), FAKE, need,
                               None) == INVALID
    assert lib.attn_bwd_phases(ctypes.byref(p), FAKE, None, 15, *([FAKE] * 9), FAKE, need,
                               None) == INVALID
    assert lib.attn_bwd_phases(ctypes.byref(p), None, None, 16, *([FAKE] * 9), FAKE, need,
                               None) == INVALID


def test_empty_batch_is_a_no_op():
    lib = ea.load()
    p = _p(batch=0)
    assert lib.attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 0


def test_workspace_sizes():
    p = _p()
    assert ea.fwd_workspace_size(p) == 0
    rows, hq, d = 2 * 300, 4, 128
    need = ea.bwd_workspace_size(p)
    assert need >= rows * hq * 4 + rows * hq * d * 4          # D and the dQ accumulator
    pd = _p(deterministic=True)
    assert ea.bwd_workspace_size(pd) > need                     # + semaphores
    pv = _p(total_q=1000, total_k=1000, batch=5)
    assert ea.fwd_workspace_size(pv, True) > 0
    assert ea.fwd_workspace_size(_p(head_dim=80)) == SIZE_MAX
    assert ea.bwd_workspace_size(_p(heads_q=5)) == SIZE_MAX


def test_tuning_knobs():
    ea.set_tuning("tile_order", 1)
    ea.set_tuning("tile_order", 0)
    for e in (1, 2, 4, 0, -1):
        ea.set_tuning("exp_emulation", e)
    for t in (0, 64, 8):
        ea.set_tuning("tau", t)
    with pytest.raises(ea.AttnError):
        ea.set_tuning("no_such_knob", 1)
    for bad in (3, 5, 8, -2):
        with pytest.raises(ea.AttnError):
            ea.set_tuning("exp_emulation", bad)
    for bad in (-1, 65):
        with pytest.raises(ea.AttnError):
            ea.set_tuning("tau", bad)
    assert ea.get_tuning("tau") == 8 and ea.get_tuning("exp_emulation") == -1


# ------------------------------------------------------------------ tile order
def _bm(d):
    return 256 if d <= 128 else 128


@pytest.mark.parametrize("b,s,hq,hkv,d,causal", [
    (2, 8192, 16, 16, 128, True), (4, 4096, 16, 16, 128, False), (1, 16384, 8, 8, 64, True),
    (1, 1000, 3, 1, 256, True), (3, 777, 2, 2, 128, False)])
def test_forward_tile_order_is_a_permutation_longest_first(b, s, hq, hkv, d, causal):
    p = _p(batch=b, seqlen_q=s, seqlen_k=s, heads_q=hq, heads_kv=hkv, head_dim=d, causal=causal)
    order = ea.tile_order(p, 0)
    nm = -(-s // _bm(d))
    assert len(order) == b * hq * nm
    assert sorted(order) == sorted((bb, h, m) for bb in range(b) for h in range(hq) for m in range(nm))
    # per XCD (workgroup i runs on XCD i % 8) and per batch-head, blocks are longest first
    seen = collections.defaultdict(list)
    for i, (bb, h, m) in enumerate(order):
        seen[(i % 8, bb, h)].append(m)
    for ms in seen.values():
        assert ms == sorted(ms, reverse=True)
    if (b * hq) % 8 == 0:
        # each XCD gets whole batch-heads
        owner = {}
        for i, (bb, h, m) in enumerate(order):
            assert owner.setdefault((bb, h), i % 8) == i % 8


@pytest.mark.parametrize("b,s,hq,hkv,d", [(2, 8192, 16, 16, 128), (1, 16384, 8, 8, 256),
                                         (1, 3000, 8, 2, 64)])
def test_backward_tile_orders(b, s, hq, hkv, d):
    p = _p(batch=b, seqlen_q=s, seqlen_k=s, heads_q=hq, heads_kv=hkv, head_dim=d, causal=True)
    nn_dkdv = -(-s // (256 if d <= 128 else 128))
    lpt = ea.tile_order(p, 1)
    assert sorted(lpt) == sorted((bb, h, n) for bb in range(b) for h in range(hkv)
                                 for n in range(nn_dkdv))
    nn = -(-s // 128)
    full = sorted((bb, h, n) for bb in range(b) for h in range(hkv) for n in range(nn))
    det = ea.tile_order(p, 2)
    assert sorted(det) == full
    # deterministic order: for each (batch, KV head) key blocks strictly descending, so every
    # workgroup only ever waits on workgroups that took earlier tickets
    pos = {}
    for i, t in enumerate(det):
        pos[t] = i
    for bb in range(b):
        for h in range(hkv):
            idx = [pos[(bb, h, n)] for n in range(nn)]
            assert all(idx[n] > idx[n + 1] for n in range(nn - 1))


def test_natural_tile_order_knob():
    p = _p(batch=1, seqlen_q=1024, seqlen_k=1024, heads_q=2, heads_kv=2, causal=True)
    ea.set_tuning("tile_order", 1)
    try:
        nat = ea.tile_order(p, 0)
    finally:
        ea.set_tuning("tile_order", 0)
    assert nat == [(0, h, m) for h in range(2) for m in range(4)]


@pytest.mark.parametrize("n,grid,nx", [(1024, 256, 8), (1000, 256, 8), (300, 256, 8), (7, 7, 8),
                                       (5000, 250, 8), (64, 13, 8), (100, 8, 8), (9, 3, 1),
                                       (2048, 512, 8), (33, 10, 4)])
def test_persistent_schedule_covers_every_tile_once(n, grid, nx):
    """Every tile position is taken by exactly one (workgroup, round), and a
    workgroup only takes positions of its own XCD residue class."""
    seen = []
    for g in range(grid):
        r = 0
        while True:
            i = ea.persistent_tile(g, r, grid, n, nx)
            if i < 0:
                break
            assert i % nx == g % nx
            seen.append(i)
            r += 1
    assert sorted(seen) == list(range(n))


def test_persistent_schedule_with_one_workgroup_per_tile_is_the_one_shot_grid():
    for n in (1, 8, 100, 1024):
        for g in range(n):
            assert ea.persistent_tile(g, 0, n, n, 8) == g
            assert ea.persistent_tile(g, 1, n, n, 8) == -1
    assert ea.persistent_tile(0, 0, 3, 100, 8) == -1      # fewer workgroups than XCDs: refused


def test_persistent_schedule_balances_causal_key_blocks():
    """B2 H16 S8192 d128 causal, dK/dV: key block n walks 256 - 8n query steps.
    256 resident workgroups get equal totals (the one-shot grid of 1024 would
    need every CU to pick the right successor at the right time)."""
    p = _p(batch=2, seqlen_q=8192, seqlen_k=8192, heads_q=16, heads_kv=16, head_dim=128,
           causal=True)
    order = ea.tile_order(p, 1)
    steps = [256 - 8 * blk for (_, _, blk) in order]
    tot = []
    for g in range(256):
        s, r = 0, 0
        while (i := ea.persistent_tile(g, r, 256, len(order), 8)) >= 0:
            s += steps[i]
            r += 1
        tot.append(s)
    assert max(tot) == min(tot) == sum(steps) // 256


def test_persistent_knob():
    for v in (0, 1):
        ea.set_tuning("persistent", v)
    with pytest.raises(ea.AttnError):
        ea.set_tuning("persistent", 2)
    ea.set_tuning("persistent", 1)


def test_stored_ds_selection_and_workspace():
    """Stored dS: automatic at head_dim 128 and 256, never with the fused
    design; its workspace holds 2 KiB per 32 x 32 sub-tile of every (sequence,
    query head) (packed lengths: a bound from the total and the longest, plus
    the per-sequence offsets)."""
    try:
        for d, auto in ((64, 0), (128, 1), (256, 1)):
            p = ea.make_params(2, 300, 700, 4, 2, d, 0.1, True, False)
            pv = ea.make_params(3, 300, 700, 4, 2, d, 0.1, True, False, total_q=500, total_k=1200)
            base_ws = base_vws = None
            for mode, want in ((-1, auto), (0, 0), (1, 1)):
                ea.set_tuning("bwd_store_ds", mode)
                assert ea.bwd_stores_ds(p) == want, (d, mode)
                assert ea.bwd_stores_ds(pv, varlen=True) == want, (d, mode)
                if mode == 0:
                    base_ws = ea.bwd_workspace_size(p)
                    base_vws = ea.bwd_workspace_size(pv, varlen=True)
            ea.set_tuning("bwd_store_ds", 1)
            nq32, nk32 = -(-300 // 64) * 2, -(-700 // 256) * 8
            extra = 2 * 4 * nq32 * nk32 * 2048
            assert ea.bwd_workspace_size(p) - base_ws >= extra
            assert ea.bwd_workspace_size(p) - base_ws < extra + 256
            # packed: 2 (cdiv(500, 64) + 3) 32-row blocks bound sum_s ds_nq32(Lq_s)
            vextra = 4 * 2 * (-(-500 // 64) + 3) * nk32 * 2048
            assert ea.bwd_workspace_size(pv, varlen=True) - base_vws >= vextra + 8 * 4
            assert ea.bwd_workspace_size(pv, varlen=True) - base_vws < vextra + 512
            ea.set_tuning("bwd_fused_dq", 1)
            assert ea.bwd_stores_ds(p) == 0
            ea.set_tuning("bwd_fused_dq", 0)
        # parameters the calls would reject (Hq not a multiple of Hkv; head_dim 96)
        assert ea.bwd_stores_ds(ea.make_params(1, 10, 10, 3, 2, 128, 0.1, False, False)) == -1
        assert ea.bwd_stores_ds(ea.make_params(1, 10, 10, 2, 2, 96, 0.1, False, False)) == -1
        # one head's sub-tiles beyond 32-bit buffer offsets: recomputation
        big = ea.make_params(1, 40000, 40000, 1, 1, 256, 0.1, True, False)
        assert ea.bwd_stores_ds(big) == 0
        with pytest.raises(ea.AttnError):
            ea.set_tuning("bwd_store_ds", 2)
    finally:
        ea.set_tuning("bwd_store_ds", -1)
        ea.set_tuning("bwd_fused_dq", 0)
