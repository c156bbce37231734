"""Python binding of libattn71 (fused exact attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libattn71.so``. PyTorch provides device memory and the current
stream. If the library is missing the import fails loudly; there is no
fallback implementation.

Entry points mirror the C ABI in ``include/attn71.h``:

    fwd(q, k, v, causal=False, softmax_scale=None, return_lse=True, options=None)
    fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, ...)
    bwd(q, k, v, o, do, lse, causal=False, softmax_scale=None, deterministic=False, options=None)
    bwd_varlen(q, k, v, o, do, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, ...)
    bwd_phases(...)          the backward split into its launches
    bwd_design(params)       the backward design a call with these parameters runs
    tile_order(...)          the fixed-length tile schedule, evaluated on the host
    varlen_key_order(...)    the packed-length key-block order, evaluated on the host

Design and tuning choices are per call: ``options`` is a dict of
``attn_options`` fields (bwd_design, tile_order, one_shot_grid,
exp_emulation, tau, spin_limit, ds_budget, head_split); missing fields take
the library's defaults. Nothing is process-global. A packed batch's
schedule can be built once with ``varlen_plan`` and passed to every varlen
call (``plan=``); ``bwd_noalloc`` runs the backward on the library's own
device scratch for callers that cannot allocate.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn71.so")

ATTN_OK = 0
ATTN_ERR_UNSUPPORTED = 2
BWD_PREPROCESS, BWD_MAIN, BWD_POSTPROCESS, BWD_DQ, BWD_ALL = 1, 2, 4, 8, 15


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib().attn_status_string(status).decode()} (status {status})")


BWD_AUTO, BWD_RECOMPUTE, BWD_STORED_DS, BWD_FUSED_DQ = 0, 1, 2, 3


class AttnOptions(ctypes.Structure):
    _fields_ = [("bwd_design", ctypes.c_int32), ("tile_order", ctypes.c_int32),
                ("one_shot_grid", ctypes.c_int32), ("exp_emulation", ctypes.c_int32),
                ("tau", ctypes.c_float), ("spin_limit", ctypes.c_int32),
                ("ds_budget", ctypes.c_int64), ("head_split", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class AttnVarlenPlan(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("bytes", ctypes.c_size_t),
                ("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32),
                ("seqlen_k", ctypes.c_int32), ("total_q", ctypes.c_int32),
                ("total_k", ctypes.c_int32), ("num_heads_q", ctypes.c_int32),
                ("num_heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("causal", ctypes.c_int32)]


class AttnParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32),
                ("seqlen_k", ctypes.c_int32), ("total_q", ctypes.c_int32),
                ("total_k", ctypes.c_int32), ("num_heads_q", ctypes.c_int32),
                ("num_heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32),
                ("deterministic", ctypes.c_int32), ("opt", AttnOptions),
                ("varlen_plan", ctypes.POINTER(AttnVarlenPlan)),
                ("block_mask", ctypes.c_void_p), ("block_mask_stride_b", ctypes.c_int64),
                ("block_mask_stride_h", ctypes.c_int64)]


MASK_BLOCK = 128   # queries and keys per block-mask entry


class VarlenPlan:
    """A built varlen plan: the C struct plus the torch buffer that holds its
    tables (kept alive here)."""

    def __init__(self, struct: AttnVarlenPlan, buf: torch.Tensor):
        self.struct = struct
        self.buf = buf


_LIB = None
_P = ctypes.POINTER(AttnParams)
_vp = ctypes.c_void_p

EXPORTS = ["attn_status_string", "attn_version", "attn_fwd_workspace_size",
           "attn_bwd_workspace_size", "attn_fwd", "attn_fwd_varlen", "attn_bwd",
           "attn_bwd_varlen", "attn_bwd_phases", "attn_bwd_status", "attn_tile_order",
           "attn_persistent_tile", "attn_bwd_design", "attn_bwd_noalloc",
           "attn_bwd_ds_subtile", "attn_varlen_plan_size", "attn_varlen_plan_build",
           "attn_bwd_head_split", "attn_varlen_key_order"]


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m exact_attention_71_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_version.restype = ctypes.c_int
    for n in ("attn_fwd_workspace_size", "attn_bwd_workspace_size"):
        getattr(lib, n).restype = ctypes.c_size_t
        getattr(lib, n).argtypes = [_P, ctypes.c_int32]
    lib.attn_fwd.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.attn_fwd_varlen.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.attn_bwd.argtypes = [_P] + [_vp] * 10 + [ctypes.c_size_t, _vp]
    lib.attn_bwd_noalloc.argtypes = [_P] + [_vp] * 10
    lib.attn_bwd_varlen.argtypes = [_P] + [_vp] * 12 + [ctypes.c_size_t, _vp]
    lib.attn_bwd_phases.argtypes = [_P, _vp, _vp, ctypes.c_int32] + [_vp] * 10 + [ctypes.c_size_t, _vp]
    lib.attn_bwd_status.argtypes = [_P, ctypes.c_int32, _vp, ctypes.POINTER(ctypes.c_int32), _vp]
    lib.attn_tile_order.argtypes = [_P, ctypes.c_int32, _vp, ctypes.c_int64,
                                    ctypes.POINTER(ctypes.c_int64)]
    lib.attn_varlen_key_order.argtypes = [_P, _vp, _vp, _vp, ctypes.c_int64,
                                          ctypes.POINTER(ctypes.c_int64)]
    lib.attn_persistent_tile.argtypes = [ctypes.c_int32] * 5
    lib.attn_persistent_tile.restype = ctypes.c_int32
    lib.attn_bwd_design.argtypes = [_P, ctypes.c_int32]
    lib.attn_bwd_head_split.argtypes = [_P, ctypes.c_int32]
    lib.attn_bwd_head_split.restype = ctypes.c_int32
    lib.attn_varlen_plan_size.argtypes = [_P]
    lib.attn_varlen_plan_size.restype = ctypes.c_size_t
    lib.attn_varlen_plan_build.argtypes = [_P, _vp, _vp, _vp, ctypes.c_size_t,
                                           ctypes.POINTER(AttnVarlenPlan), _vp]
    lib.attn_bwd_ds_subtile.argtypes = [_P, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_int64)]
    lib.attn_bwd_ds_subtile.restype = ctypes.c_int64
    for n in EXPORTS:
        if n not in ("attn_status_string", "attn_version", "attn_fwd_workspace_size",
                     "attn_bwd_workspace_size", "attn_bwd_ds_subtile", "attn_varlen_plan_size"):
            getattr(lib, n).restype = ctypes.c_int
    _LIB = lib
    return lib


def load() -> ctypes.CDLL:
    """Load the library (raises ImportError if it is not built)."""
    return _lib()


def _check(status: int, where: str) -> None:
    if status != ATTN_OK:
        raise AttnError(status, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _expect(t: torch.Tensor, name: str, dtype=torch.bfloat16) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_options(options: Optional[dict] = None) -> AttnOptions:
    """attn_options from a dict of its fields (missing fields: 0 = default)."""
    o = AttnOptions()
    for k, v in (options or {}).items():
        if k not in dict(AttnOptions._fields_):
            raise ValueError(f"unknown option {k!r}")
        setattr(o, k, float(v) if k == "tau" else int(v))
    return o


def make_params(batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim, scale, causal,
                deterministic=False, total_q=0, total_k=0,
                options: Optional[dict] = None, plan: Optional["VarlenPlan"] = None) -> AttnParams:
    p = AttnParams(int(batch), int(seqlen_q), int(seqlen_k), int(total_q), int(total_k),
                   int(heads_q), int(heads_kv), int(head_dim), float(scale), int(bool(causal)),
                   int(bool(deterministic)), make_options(options))
    if plan is not None:
        p.varlen_plan = ctypes.pointer(plan.struct)
    return p


def prepare_block_mask(mask: Optional[torch.Tensor], batch: int, heads_q: int, seqlen_q: int,
                       seqlen_k: int) -> Optional[torch.Tensor]:
    """A block mask as the library reads it: uint8 (bool accepted), shape
    [batch or 1, heads_q or 1, ceil(seqlen_q / 128), ceil(seqlen_k / 128)],
    contiguous and 4-byte aligned on the GPU (copied if needed)."""
    if mask is None:
        return None
    nqb, nkb = -(-seqlen_q // MASK_BLOCK), -(-seqlen_k // MASK_BLOCK)
    if mask.dim() != 4 or tuple(mask.shape[2:]) != (nqb, nkb) or \
            mask.shape[0] not in (1, batch) or mask.shape[1] not in (1, heads_q):
        raise ValueError(f"block mask must be [{batch} or 1, {heads_q} or 1, {nqb}, {nkb}], "
                         f"got {tuple(mask.shape)}")
    if not mask.is_cuda:
        raise ValueError("block mask must be on the GPU")
    # the library reads whole 4-byte words: a 4-byte aligned buffer padded to a
    # multiple of 4 bytes
    m = mask.to(torch.uint8).contiguous()
    n = m.numel()
    buf = torch.zeros((n + 3) // 4 * 4, dtype=torch.uint8, device=m.device)
    buf[:n].copy_(m.reshape(-1))
    return buf[:n].view(m.shape)


def set_block_mask(p: AttnParams, m: Optional[torch.Tensor]) -> None:
    """Point the parameters at a prepared block mask (size-1 dims broadcast)."""
    if m is None:
        return
    p.block_mask = m.data_ptr()
    p.block_mask_stride_b = m.stride(0) if m.shape[0] > 1 else 0
    p.block_mask_stride_h = m.stride(1) if m.shape[1] > 1 else 0


def varlen_plan(cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                total_q: int, total_k: int, heads_q: int, heads_kv: int, head_dim: int,
                causal: bool) -> VarlenPlan:
    """attn_varlen_plan_build: the schedule of one packed batch, computed once
    on the current stream for every later varlen call with these parameters."""
    _expect(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _expect(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    nseq = cu_seqlens_q.numel() - 1
    p = make_params(nseq, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, head_dim, 1.0, causal,
                    total_q=total_q, total_k=total_k)
    n = _lib().attn_varlen_plan_size(ctypes.byref(p))
    buf = _workspace(n, cu_seqlens_q.device)
    st = AttnVarlenPlan()
    _check(_lib().attn_varlen_plan_build(ctypes.byref(p), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                         _ptr(buf), buf.numel(), ctypes.byref(st), _stream()),
           "attn_varlen_plan_build")
    return VarlenPlan(st, buf)


def _workspace(nbytes: int, device) -> torch.Tensor:
    if nbytes == ctypes.c_size_t(-1).value:
        raise AttnError(1, "workspace size")
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def fwd_workspace_size(p: AttnParams, varlen: bool = False) -> int:
    return _lib().attn_fwd_workspace_size(ctypes.byref(p), int(varlen))


def bwd_workspace_size(p: AttnParams, varlen: bool = False) -> int:
    return _lib().attn_bwd_workspace_size(ctypes.byref(p), int(varlen))


def bwd_design(p: AttnParams, varlen: bool = False) -> int:
    """BWD_RECOMPUTE, BWD_STORED_DS or BWD_FUSED_DQ: the design a backward call
    with these parameters runs; -1: parameters the calls would reject."""
    return _lib().attn_bwd_design(ctypes.byref(p), int(varlen))


def bwd_head_split(p: AttnParams, varlen: bool = False) -> int:
    """Query-head parts per KV group of the backward's key-block kernel
    (1: unsplit); -1: parameters the calls would reject."""
    return _lib().attn_bwd_head_split(ctypes.byref(p), int(varlen))


# --------------------------------------------------------------------- forward
def fwd(q, k, v, causal: bool = False, softmax_scale: Optional[float] = None,
        return_lse: bool = True, out: Optional[torch.Tensor] = None,
        lse_out: Optional[torch.Tensor] = None, options: Optional[dict] = None,
        block_mask: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q [B, Sq, Hq, d], k/v [B, Sk, Hkv, d] bf16 -> (o [B, Sq, Hq, d], lse [B, Hq, Sq] fp32)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, n)
    b, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    p = make_params(b, sq, sk, hq, hkv, d, scale, causal, options=options)
    bm = prepare_block_mask(block_mask, b, hq, sq, sk)
    set_block_mask(p, bm)
    o = torch.empty_like(q) if out is None else out
    lse = None
    if return_lse:
        lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device) if lse_out is None else lse_out
    ws = _workspace(fwd_workspace_size(p), q.device)
    _check(_lib().attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                           _ptr(ws), ws.numel(), _stream()), "attn_fwd")
    return o, lse


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
               causal: bool = False, softmax_scale: Optional[float] = None,
               return_lse: bool = True, options: Optional[dict] = None,
               plan: Optional[VarlenPlan] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q [Tq, Hq, d], k/v [Tk, Hkv, d], cu_seqlens int32 [n+1] -> (o, lse [Hq, Tq])."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, n)
    _expect(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _expect(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    nseq = cu_seqlens_q.numel() - 1
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    p = make_params(nseq, max_seqlen_q, max_seqlen_k, hq, hkv, d, scale, causal, total_q=tq,
                    total_k=tk, options=options, plan=plan)
    o = torch.empty_like(q)
    lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device) if return_lse else None
    ws = _workspace(fwd_workspace_size(p, True), q.device)
    _check(_lib().attn_fwd_varlen(ctypes.byref(p), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                  _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws),
                                  ws.numel(), _stream()), "attn_fwd_varlen")
    return o, lse


# -------------------------------------------------------------------- backward
def bwd(q, k, v, o, do, lse, causal: bool = False, softmax_scale: Optional[float] = None,
        deterministic: bool = False, workspace: Optional[torch.Tensor] = None,
        options: Optional[dict] = None, block_mask: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) of sum(do * o) for fixed-length BSHD inputs."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _expect(t, n)
    _expect(lse, "lse", torch.float32)
    b, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    p = make_params(b, sq, sk, hq, hkv, d, scale, causal, deterministic, options=options)
    bm = prepare_block_mask(block_mask, b, hq, sq, sk)
    set_block_mask(p, bm)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = workspace if workspace is not None else _workspace(bwd_workspace_size(p), q.device)
    _check(_lib().attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                           _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
                           _stream()), "attn_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, do, lse, causal: bool = False, softmax_scale: Optional[float] = None,
                deterministic: bool = False, options: Optional[dict] = None):
    """attn_bwd_noalloc: the recomputing backward on the library's static device
    scratch (no workspace; the C call allocates nothing; dq, dk, dv are
    allocated here by torch)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _expect(t, n)
    _expect(lse, "lse", torch.float32)
    b, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    p = make_params(b, sq, sk, hq, hkv, d, scale, causal, deterministic, options=options)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(_lib().attn_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                                   _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _stream()),
           "attn_bwd_noalloc")
    return dq, dk, dv


def bwd_varlen(q, k, v, o, do, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
               max_seqlen_k: int, causal: bool = False, softmax_scale: Optional[float] = None,
               deterministic: bool = False, workspace: Optional[torch.Tensor] = None,
               options: Optional[dict] = None, plan: Optional[VarlenPlan] = None):
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _expect(t, n)
    _expect(lse, "lse", torch.float32)
    _expect(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _expect(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    nseq = cu_seqlens_q.numel() - 1
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    p = make_params(nseq, max_seqlen_q, max_seqlen_k, hq, hkv, d, scale, causal, deterministic,
                    total_q=tq, total_k=tk, options=options, plan=plan)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = workspace if workspace is not None else _workspace(bwd_workspace_size(p, True), q.device)
    _check(_lib().attn_bwd_varlen(ctypes.byref(p), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                  _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                  _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _stream()),
           "attn_bwd_varlen")
    return dq, dk, dv


def bwd_phases(p: AttnParams, phases: int, q, k, v, o, do, lse, dq, dk, dv,
               workspace: torch.Tensor, cu_seqlens_q=None, cu_seqlens_k=None) -> None:
    """Run selected backward phases (mask of BWD_*) on the current stream."""
    _check(_lib().attn_bwd_phases(ctypes.byref(p), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                  int(phases), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                                  _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                  workspace.numel(), _stream()), "attn_bwd_phases")


def bwd_status(p: AttnParams, workspace: torch.Tensor, varlen: bool = False) -> int:
    val = ctypes.c_int32(0)
    _check(_lib().attn_bwd_status(ctypes.byref(p), int(varlen), _ptr(workspace),
                                  ctypes.byref(val), _stream()), "attn_bwd_status")
    return val.value


def varlen_key_order(p: AttnParams, cu_q, cu_k):
    """[(sequence, key block)] in the order the packed-length dK/dV kernel takes
    its key-block tiles (KV heads innermost), or None where it keeps the
    per-sequence order. cu_q / cu_k: host int sequences of batch + 1 offsets."""
    lib = _lib()
    cq = (ctypes.c_int32 * len(cu_q))(*[int(x) for x in cu_q])
    ck = (ctypes.c_int32 * len(cu_k))(*[int(x) for x in cu_k])
    count = ctypes.c_int64(0)
    st = lib.attn_varlen_key_order(ctypes.byref(p), cq, ck, None, 0, ctypes.byref(count))
    if st == ATTN_ERR_UNSUPPORTED:
        return None
    _check(st, "attn_varlen_key_order")
    buf = (ctypes.c_int32 * (2 * count.value))()
    _check(lib.attn_varlen_key_order(ctypes.byref(p), cq, ck, buf, count.value,
                                     ctypes.byref(count)), "attn_varlen_key_order")
    return [tuple(buf[2 * i:2 * i + 2]) for i in range(count.value)]


def tile_order(p: AttnParams, which: int):
    """[(batch, head, block)] per workgroup for which = 0 fwd, 1 bwd, 2 deterministic bwd."""
    lib = _lib()
    count = ctypes.c_int64(0)
    _check(lib.attn_tile_order(ctypes.byref(p), which, None, 0, ctypes.byref(count)), "attn_tile_order")
    buf = (ctypes.c_int32 * (3 * count.value))()
    _check(lib.attn_tile_order(ctypes.byref(p), which, buf, count.value, ctypes.byref(count)),
           "attn_tile_order")
    return [tuple(buf[3 * i:3 * i + 3]) for i in range(count.value)]


def ds_subtile(p: AttnParams, row32: int, col32: int):
    """(index of the stored-dS sub-tile (row32, col32) in a (sequence, head)
    region or -1, sub-tiles in the region), host evaluation."""
    n = ctypes.c_int64(0)
    i = _lib().attn_bwd_ds_subtile(ctypes.byref(p), int(row32), int(col32), ctypes.byref(n))
    return int(i), int(n.value)


def persistent_tile(g: int, r: int, grid: int, ntiles: int, nx: int = 8) -> int:
    """Tile position taken by persistent workgroup g in round r (-1: none)."""
    return int(_lib().attn_persistent_tile(g, r, grid, ntiles, nx))


def version() -> int:
    return _lib().attn_version()
