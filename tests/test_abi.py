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
    assert ea.version() == 202
    assert lib.attn_status_string(0) == b"OK"
    assert lib.attn_status_string(3) == b"workspace too small"
    assert lib.attn_status_string(99) == b"unknown status"


def _p(**kw):
    base = dict(batch=2, seqlen_q=300, seqlen_k=300, heads_q=4, heads_kv=2, head_dim=128,
                scale=0.088, causal=False, deterministic=False)
    base.update(kw)
    return ea.make_params(base["batch"], base["seqlen_q"], base["seqlen_k"], base["heads_q"],
                          base["heads_kv"], base["head_dim"], base["scale"], base["causal"],
                          base["deterministic"], base.get("total_q", 0), base.get("total_k", 0),
                          options=base.get("options"))


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


def test_tensors_with_no_elements_may_be_null():
    """No query rows and no keys: every data pointer may be null (PyTorch hands
    out null for tensors with no elements) and the calls are no-ops."""
    lib = ea.load()
    p = _p(seqlen_q=0, seqlen_k=0)
    ws = (ctypes.c_uint8 * 4096)()
    assert lib.attn_fwd(ctypes.byref(p), None, None, None, None, None, None, 0, None) == 0
    assert lib.attn_bwd(ctypes.byref(p), *([None] * 9), ws, 4096, None) == 0
    # query rows present: Q and O must be given
    q_only = _p(seqlen_k=0)
    assert lib.attn_fwd(ctypes.byref(q_only), None, None, None, None, None, None, 0,
                        None) == INVALID


def test_workspace_sizes():
    rows, hq, hkv, d = 2 * 300, 4, 2, 128
    p = _p(options=dict(bwd_design=ea.BWD_RECOMPUTE, head_split=1))
    assert ea.fwd_workspace_size(p) == 0
    need = ea.bwd_workspace_size(p)
    assert 2 * rows * hq * 4 <= need < 2 * rows * hq * 4 + 1024   # -D, LSE log2 e, counters
    # a head split adds the fp32 dK and dV partials of its parts
    split = ea.bwd_workspace_size(_p(options=dict(bwd_design=ea.BWD_RECOMPUTE, head_split=2)))
    assert need + 2 * 2 * rows * hkv * d * 4 <= split < need + 2 * 2 * rows * hkv * d * 4 + 256
    fused = ea.bwd_workspace_size(_p(options=dict(bwd_design=ea.BWD_FUSED_DQ, head_split=1)))
    assert fused >= need + rows * hq * d * 4                       # + the fp32 dQ accumulator
    fused_det = ea.bwd_workspace_size(_p(deterministic=True,
                                         options=dict(bwd_design=3, head_split=1)))
    assert fused_det > fused                                       # + semaphores
    # deterministic costs nothing outside the fused design
    assert ea.bwd_workspace_size(_p(deterministic=True,
                                    options=dict(bwd_design=1, head_split=1))) == need
    pv = _p(total_q=1000, total_k=1000, batch=5)
    assert ea.fwd_workspace_size(pv, True) > 0
    assert ea.fwd_workspace_size(_p(head_dim=80)) == SIZE_MAX
    assert ea.bwd_workspace_size(_p(heads_q=5)) == SIZE_MAX


@pytest.mark.parametrize("opt", [dict(bwd_design=4), dict(bwd_design=-1), dict(tile_order=2),
                                 dict(one_shot_grid=-1), dict(exp_emulation=3),
                                 dict(exp_emulation=8), dict(tau=-2.0), dict(tau=65.0),
                                 dict(tau=float("nan")), dict(spin_limit=-1),
                                 dict(ds_budget=-1), dict(head_split=-1), dict(head_split=3),
                                 dict(head_split=4), dict(reserved=1)])
def test_options_are_validated(opt):
    lib = ea.load()
    p = _p(options=opt)
    assert lib.attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == INVALID
    assert lib.attn_bwd(ctypes.byref(p), *([FAKE] * 9), FAKE, 1 << 30, None) == INVALID
    assert ea.fwd_workspace_size(p) == SIZE_MAX and ea.bwd_workspace_size(p) == SIZE_MAX
    assert ea.bwd_design(p) == -1


def test_valid_options_pass_validation():
    lib = ea.load()
    for opt in (dict(tau=-1.0), dict(tau=64.0), dict(tau=0.5), dict(exp_emulation=4),
                dict(tile_order=1, one_shot_grid=1), dict(spin_limit=5), dict(ds_budget=1)):
        p = _p(options=opt)
        # fails on the null q pointer, i.e. after the options were accepted
        assert lib.attn_fwd(ctypes.byref(p), None, FAKE, FAKE, FAKE, None, None, 0, None) == INVALID
        assert ea.bwd_workspace_size(p) != SIZE_MAX


def test_head_split_rule():
    """Automatic head split: the largest divisor of the KV group that keeps the
    key-block tiles within 512, only when the unsplit tiles fall below it."""
    def hs(b, s, hq, hkv, d, varlen=False, **opt):
        tot = b * s if varlen else 0
        p = ea.make_params(b, s, s, hq, hkv, d, 0.088, True, total_q=tot, total_k=tot,
                           options=opt or None)
        return ea.bwd_head_split(p, varlen)
    assert hs(2, 8192, 16, 1, 128) == 8        # MQA: 64 tiles -> 512
    assert hs(2, 8192, 16, 16, 128) == 1       # MHA: no group to split
    assert hs(1, 8192, 8, 2, 128) == 4         # 64 tiles, group 4 -> 256
    assert hs(16, 4352, 32, 4, 128, varlen=True) == 1   # packed GQA: 1152 tiles
    assert hs(1, 300, 8, 1, 64) == 8
    assert hs(2, 8192, 16, 1, 128, head_split=1) == 1
    assert hs(2, 8192, 16, 1, 128, head_split=4) == 4
    # the fused design at head_dim 256 (the 128-key kernel) walks whole groups
    assert hs(2, 8192, 16, 1, 256, bwd_design=ea.BWD_FUSED_DQ) == 1
    p = ea.make_params(1, 300, 300, 8, 1, 256, 0.088, True,
                       options=dict(bwd_design=ea.BWD_FUSED_DQ, head_split=2))
    assert ea.bwd_workspace_size(p) == SIZE_MAX and ea.bwd_head_split(p) == -1


def test_tile_counts_stay_within_int32():
    """Key-block tiles times the largest head split must fit the kernels' int32
    tile indices: 2^16 key blocks x 2^16 query heads is refused up front."""
    p = ea.make_params(1, 16, 1 << 23, 1 << 16, 1, 64, 0.125, False)
    assert ea.bwd_workspace_size(p) == SIZE_MAX and ea.bwd_head_split(p) == -1
    ok = ea.make_params(1, 16, 1 << 20, 1 << 10, 1, 64, 0.125, False)
    assert ea.bwd_workspace_size(ok) != SIZE_MAX


@pytest.mark.parametrize("d,causal", [(128, True), (64, True), (256, True), (128, False)])
def test_varlen_key_order_is_longest_first(d, causal):
    """Packed key-block tiles: one order over all sequences, by decreasing
    work (the query steps whose rows see some key of the block under the
    bottom-right causal mask, every step without it), ties by sequence then
    block. Brute force over the mask predicate itself."""
    import numpy as np
    rng = np.random.default_rng(7 + d)
    lq = [int(x) for x in rng.integers(0, 3000, 9)] + [0, 1, 257]
    # as many keys as queries, more keys, fewer keys (rows before the diagonal see none)
    lk = [x if i % 3 == 2 else max(0, x + (1 if i % 3 == 0 else -1) * int(rng.integers(0, 600)))
          for i, x in enumerate(lq)]
    cu_q = np.concatenate([[0], np.cumsum(lq)]).tolist()
    cu_k = np.concatenate([[0], np.cumsum(lk)]).tolist()
    bn = 256 if d <= 128 else 128
    bm = 64 if d == 64 else 32
    p = ea.make_params(len(lq), max(lq), max(lk), 8, 2, d, 0.1, causal,
                       total_q=cu_q[-1], total_k=cu_k[-1])

    def work(q, k, b):
        steps = 0
        for m in range(-(-q // bm)):
            rows = range(m * bm, min(q, (m + 1) * bm))
            keys = range(b * bn, min(k, (b + 1) * bn))
            steps += any(j <= i + (k - q) for i in rows for j in keys) if causal else 1
        return steps

    entries = [(s, b) for s in range(len(lq)) for b in range(-(-lk[s] // bn))]
    want = sorted(entries, key=lambda e: (-work(lq[e[0]], lk[e[0]], e[1]), e[0], e[1]))
    got = ea.varlen_key_order(p, cu_q, cu_k)
    assert got == want


def test_varlen_key_order_falls_back_for_many_sequences():
    """Ranking costs (key-block bound x batch) steps of one workgroup: past 2^17
    the kernel keeps the per-sequence order."""
    n = 1024
    cu = [i * 512 for i in range(n + 1)]
    p = ea.make_params(n, 512, 512, 8, 2, 128, 0.1, True, total_q=cu[-1], total_k=cu[-1])
    assert ea.varlen_key_order(p, cu, cu) is None
    small = ea.make_params(16, 512, 512, 8, 2, 128, 0.1, True, total_q=16 * 512, total_k=16 * 512)
    assert len(ea.varlen_key_order(small, cu[:17], cu[:17])) == 32


def test_workspace_size_is_a_pure_function_of_the_parameters():
    """No process-wide state: sizes and designs depend on the parameters
    (options included) alone, whatever other calls ran in between."""
    cases = [_p(head_dim=d, causal=c, options=dict(bwd_design=b))
             for d in (64, 128, 256) for c in (False, True) for b in range(4)]
    first = [(ea.bwd_workspace_size(p), ea.bwd_design(p), ea.fwd_workspace_size(p)) for p in cases]
    for p in reversed(cases):
        ea.bwd_workspace_size(p)
        ea.tile_order(p, 0)
    again = [(ea.bwd_workspace_size(p), ea.bwd_design(p), ea.fwd_workspace_size(p)) for p in cases]
    assert first == again
    assert not hasattr(ea.load(), "attn_set_tuning") or "attn_set_tuning" not in ea.EXPORTS


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
    # a head split of n makes (KV head, part) the scheduler's heads
    split = ea.bwd_head_split(p)
    assert split >= 1 and (hq // hkv) % split == 0
    if b * hkv * nn_dkdv >= 512:
        assert split == 1   # enough tiles: no split
    lpt = ea.tile_order(p, 1)
    assert sorted(lpt) == sorted((bb, h, n) for bb in range(b) for h in range(hkv * split)
                                 for n in range(nn_dkdv))
    # the fused design: 256-key blocks at head_dim 64 and 128 (the dK/dV kernel), 128 at 256
    nn = nn_dkdv
    full = sorted((bb, h, n) for bb in range(b) for h in range(hkv * split) for n in range(nn))
    det = ea.tile_order(p, 2)
    assert sorted(det) == full
    # deterministic order: for each (batch, KV head, part) key blocks strictly descending, so
    # every workgroup only ever waits on workgroups that took earlier tickets
    pos = {}
    for i, t in enumerate(det):
        pos[t] = i
    for bb in range(b):
        for h in range(hkv * split):
            idx = [pos[(bb, h, n)] for n in range(nn)]
            assert all(idx[n] > idx[n + 1] for n in range(nn - 1))


def test_natural_tile_order_option():
    p = _p(batch=1, seqlen_q=1024, seqlen_k=1024, heads_q=2, heads_kv=2, causal=True,
           options=dict(tile_order=1))
    assert ea.tile_order(p, 0) == [(0, h, m) for h in range(2) for m in range(4)]
    q = _p(batch=1, seqlen_q=1024, seqlen_k=1024, heads_q=2, heads_kv=2, causal=True)
    assert ea.tile_order(q, 0) != ea.tile_order(p, 0)


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


def test_stored_ds_selection_and_budget():
    """Stored dS: automatic at head_dim 128 and 256 when its area fits the
    budget, never at 64 or with another design requested; an explicit request
    over the budget is refused (size -1, design -1)."""
    for d, auto in ((64, 1), (128, 2), (256, 2)):
        for varlen in (False, True):
            kw = dict(batch=3, seqlen_q=300, seqlen_k=700, heads_q=4, heads_kv=2, head_dim=d,
                      causal=True)
            if varlen:
                kw.update(total_q=500, total_k=1200)
            assert ea.bwd_design(_p(**kw), varlen) == auto
            for b in (1, 2, 3):
                assert ea.bwd_design(_p(**kw, options=dict(bwd_design=b)), varlen) == b
            area = (ea.bwd_workspace_size(_p(**kw, options=dict(bwd_design=2)), varlen)
                    - ea.bwd_workspace_size(_p(**kw, options=dict(bwd_design=1)), varlen))
            assert area > 0
            tight = _p(**kw, options=dict(bwd_design=2, ds_budget=area - 1024))
            assert ea.bwd_design(tight, varlen) == -1
            assert ea.bwd_workspace_size(tight, varlen) == SIZE_MAX
            assert ea.bwd_design(_p(**kw, options=dict(ds_budget=area - 1024)), varlen) == 1
            assert ea.bwd_design(_p(**kw, options=dict(bwd_design=2, ds_budget=area)), varlen) == 2
    # parameters the calls would reject (Hq not a multiple of Hkv; head_dim 96)
    assert ea.bwd_design(ea.make_params(1, 10, 10, 3, 2, 128, 0.1, False, False)) == -1
    assert ea.bwd_design(ea.make_params(1, 10, 10, 2, 2, 96, 0.1, False, False)) == -1
    # no per-head size limit: S = 40000 causal d256 stores dS once the budget allows it
    big = ea.make_params(1, 40000, 40000, 1, 1, 256, 0.1, True, False,
                         options=dict(bwd_design=2, ds_budget=1 << 34))
    assert ea.bwd_design(big) == 2


# ------------------------------------------------------- stored-dS layout
def _dkdv_writes(lq, lk, d, causal):
    """(sub-row, sub-column) pairs the dK/dV kernel stores: key block n of
    256 keys (128 at head_dim 256) walks query steps of 32 rows (64 at head
    dim 64) from the first that sees its first key (bottom-right diagonal)
    to the end; every wave stores all of its sub-columns at every step."""
    bn, bm = (256, 64) if d == 64 else ((256, 32) if d == 128 else (128, 32))
    shift, nm = lk - lq, -(-lq // bm)
    out = set()
    for n in range(-(-lk // bn)):
        m_first = min(max(0, n * bn - shift) // bm, nm) if causal else 0
        for m in range(m_first, nm):
            for r in range(m * bm // 32, (m + 1) * bm // 32):
                for k in range(n * bn // 32, (n + 1) * bn // 32):
                    out.add((r, k))
    return out


def _dq_reads(lq, lk, d, causal):
    """(sub-row, sub-column) pairs the dQ kernel uses: wave rows 32 r (r with
    rows inside the sequence), key tiles of 32 keys (64 at head_dim 64), the
    sub-tiles with a visible pair for some row of the wave."""
    bn, bmq = (64 if d == 64 else 32), 256
    shift = lk - lq
    out = set()
    for r in range(-(-lq // 32)):
        m0 = (32 * r) // bmq * bmq
        kend = max(0, min(m0 + bmq + shift, lk)) if causal else lk
        for n in range(-(-kend // bn)):
            k0 = n * bn
            lim = 32 * r + 31 + shift - k0 if causal else bn - 1
            nv = 0 if lim < 0 else min(lim // 32 + 1, bn // 32)
            for j in range(nv):
                out.add((r, k0 // 32 + j))
    return out


@pytest.mark.parametrize("lq,lk", [(300, 300), (8192, 8192), (1000, 1000), (64, 64), (1, 1),
                                   (256, 257), (700, 300), (300, 700), (17, 4096), (4096, 17),
                                   (513, 1024), (1024, 513), (2000, 2000 + 255), (33, 33),
                                   (5000, 4000), (4000, 5000), (640, 7000)])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_stored_ds_layout_holds_every_write_and_read(lq, lk, d, causal):
    """The key-block-major layout (evaluated by the library on the host) gives
    every sub-tile the dK/dV kernel writes its own index inside the region,
    the dQ kernel reads only written sub-tiles, each key block's stored rows
    are contiguous (16 KiB per sub-row, so the dK/dV kernel advances by a
    constant per step), and the library's area for B x Hq regions equals the
    region size."""
    writes = _dkdv_writes(lq, lk, d, causal)
    reads = _dq_reads(lq, lk, d, causal)
    assert reads <= writes
    p = _p(batch=2, seqlen_q=lq, seqlen_k=lk, heads_q=3, heads_kv=1, head_dim=d, causal=causal)
    idx = {}
    region = None
    for r, k in sorted(writes):
        i, region = ea.ds_subtile(p, r, k)
        assert 0 <= i < region, (r, k, i, region)
        idx[(r, k)] = i
    assert len(set(idx.values())) == len(idx)               # one slot per written sub-tile
    # contiguity: within a key block, sub-row r + 1 sits 8 sub-tiles after r
    for (r, k), i in idx.items():
        if (r + 1, k) in idx:
            assert idx[(r + 1, k)] == i + 8
    # unstored neighbours of the written set return -1
    rows = -(-lq // 64) * 2
    for r, k in list(writes)[:50]:
        assert ea.ds_subtile(p, rows, k)[0] == -1 and ea.ds_subtile(p, r, -1)[0] == -1
    if writes:
        kw = dict(batch=2, seqlen_q=lq, seqlen_k=lk, heads_q=3, heads_kv=1, head_dim=d,
                  causal=causal)
        area = (ea.bwd_workspace_size(_p(**kw, options=dict(bwd_design=2, ds_budget=1 << 40)))
                - ea.bwd_workspace_size(_p(**kw, options=dict(bwd_design=1))))
        assert 2 * 3 * region * 2048 <= area < 2 * 3 * region * 2048 + 256
        # the region is exactly the written set, rounded to whole 256-key
        # blocks and to the 64-query rows of the longest dK/dV step
        blocks = {}
        for r, k in writes:
            blocks.setdefault(k // 8, set()).add(r)
        want = sum(8 * (rows - min(rs) // 2 * 2) for rs in blocks.values())
        assert region == want


def test_varlen_plan_validation():
    """Plans are sized by the sequence count alone, shrink the varlen
    workspaces (no tables there), and a call whose parameters differ from the
    plan's in any recorded field is rejected before anything is enqueued."""
    lib = ea.load()
    kw = dict(batch=5, seqlen_q=700, seqlen_k=700, heads_q=4, heads_kv=2, head_dim=128,
              causal=True, total_q=2000, total_k=2000)
    p = _p(**kw)
    n = lib.attn_varlen_plan_size(ctypes.byref(p))
    assert 0 < n < 1 << 16
    assert lib.attn_varlen_plan_size(ctypes.byref(_p(**dict(kw, batch=50)))) > n
    plan = ea.AttnVarlenPlan()
    # argument checks (no GPU needed): null cu, null data, small buffer
    assert lib.attn_varlen_plan_build(ctypes.byref(p), None, FAKE, FAKE, n, ctypes.byref(plan),
                                      None) == INVALID
    assert lib.attn_varlen_plan_build(ctypes.byref(p), FAKE, FAKE, None, n, ctypes.byref(plan),
                                      None) == INVALID
    assert lib.attn_varlen_plan_build(ctypes.byref(p), FAKE, FAKE, FAKE, n - 1,
                                      ctypes.byref(plan), None) == WS_SMALL
    # a plan as the builder fills it (zero sequences: filled without a launch)
    p0 = _p(**dict(kw, batch=0))
    plan0 = ea.AttnVarlenPlan()
    assert lib.attn_varlen_plan_build(ctypes.byref(p0), FAKE, FAKE, FAKE, 1 << 20,
                                      ctypes.byref(plan0), None) == 0
    assert (plan0.batch, plan0.num_heads_q, plan0.head_dim, plan0.causal) == (0, 4, 128, 1)
    # a plan built for p: fields as recorded
    good = ea.AttnVarlenPlan(FAKE, n, 5, 700, 700, 2000, 2000, 4, 2, 128, 1)
    pp = _p(**kw)
    pp.varlen_plan = ctypes.pointer(good)
    assert ea.fwd_workspace_size(pp, True) == 0
    assert ea.bwd_workspace_size(pp, True) < ea.bwd_workspace_size(p, True)
    # a valid plan passes validation (the call then fails on the null q)
    assert lib.attn_fwd_varlen(ctypes.byref(pp), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None,
                               0, None) == INVALID
    for field, val in (("batch", 4), ("seqlen_k", 701), ("total_q", 1999), ("num_heads_q", 8),
                       ("num_heads_kv", 1), ("head_dim", 64), ("causal", 0), ("bytes", n - 1)):
        bad = ea.AttnVarlenPlan(FAKE, n, 5, 700, 700, 2000, 2000, 4, 2, 128, 1)
        setattr(bad, field, val)
        q = _p(**kw)
        q.varlen_plan = ctypes.pointer(bad)
        args = [FAKE] * 7 + [None, FAKE, 1 << 20, None]
        assert lib.attn_fwd_varlen(ctypes.byref(q), *args) == INVALID, field
        bargs = [FAKE] * 11 + [FAKE, 1 << 30, None]
        assert lib.attn_bwd_varlen(ctypes.byref(q), *bargs) == INVALID, field
    # a plan on a fixed-length call
    f = _p(batch=5, seqlen_q=700, seqlen_k=700, heads_q=4, heads_kv=2, head_dim=128, causal=True)
    f.varlen_plan = ctypes.pointer(good)
    assert lib.attn_fwd(ctypes.byref(f), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == INVALID


def test_block_mask_validation():
    """Block masks: 4-byte aligned, non-negative strides, fixed length only,
    no exp emulation, and no stored dS (the automatic design recomputes dQ)."""
    lib = ea.load()
    kw = dict(batch=2, seqlen_q=300, seqlen_k=300, heads_q=4, heads_kv=2, head_dim=128,
              causal=True)

    def pm(ptr=FAKE, sb=9, sh=9, **extra):
        p = _p(**dict(kw, **extra))
        p.block_mask, p.block_mask_stride_b, p.block_mask_stride_h = ptr, sb, sh
        return p

    args = [None, FAKE, FAKE, FAKE, None, None, 0, None]     # null q: fails after validation
    assert lib.attn_fwd(ctypes.byref(pm()), *args) == INVALID
    assert ea.bwd_design(pm()) == ea.BWD_RECOMPUTE                       # automatic: recompute
    assert ea.bwd_design(_p(**kw)) == ea.BWD_STORED_DS                   # without a mask
    assert ea.bwd_design(pm(options=dict(bwd_design=ea.BWD_STORED_DS))) == -1
    assert ea.bwd_design(pm(options=dict(bwd_design=ea.BWD_FUSED_DQ))) == ea.BWD_FUSED_DQ
    full = [FAKE] * 4 + [None, None, 0, None]
    assert lib.attn_fwd(ctypes.byref(pm(ptr=FAKE + 2)), *full) == INVALID       # misaligned
    assert lib.attn_fwd(ctypes.byref(pm(sb=-1)), *full) == INVALID
    assert lib.attn_fwd(ctypes.byref(pm(options=dict(exp_emulation=2))), *full) == UNSUPPORTED
    assert lib.attn_fwd(ctypes.byref(pm(sh=1 << 30)), *full) == UNSUPPORTED     # > 2^31 bytes
    pv = pm(total_q=600, total_k=600)
    assert lib.attn_fwd_varlen(ctypes.byref(pv), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                               1 << 20, None) == UNSUPPORTED
    # the kernels list up to 4096 visible 64-key tiles per workgroup
    # (null q: the first case passes the mask checks and fails on the pointer)
    assert lib.attn_fwd(ctypes.byref(pm(seqlen_k=4096 * 64, sb=0, sh=0)), *args) == INVALID
    assert lib.attn_fwd(ctypes.byref(pm(seqlen_k=4096 * 64 + 1, sb=0, sh=0)), *args) == UNSUPPORTED
