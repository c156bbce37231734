"""Exact attention written out from its definition, in float64.

Test infrastructure: see ``oracle/__init__.py``.

Definition followed (FlashAttention-4 pages: digest page, notation table, which
fixes alpha = 1/sqrt(d); roofline paragraph, two forward GEMMs S = Q K^T and
O = P V; blog page, introduction and "correction warpgroup" list, softmax
between the GEMMs and an optional stored LSE; blog page, backward section, the
recomputation of S and P and the gradient GEMMs for dQ, dK, dP, dV and the
elementwise P and dS):

    s_ij  = alpha * q_i . k_j                      j visible to i
    LSE_i = log sum_{j visible} exp(s_ij)          (natural log)
    P_ij  = exp(s_ij - LSE_i), 0 where j is hidden
    O_i   = sum_j P_ij v_j
    D_i   = dO_i . O_i
    dP_ij = dO_i . v_j
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = alpha * sum_j dS_ij k_j
    dK_j  = alpha * sum_{h in group} sum_i dS_ij q_i
    dV_j  =         sum_{h in group} sum_i P_ij dO_i

Visibility: non-causal, every key of the same sequence; causal (lower
triangular, query i sees key j iff j <= i; the pages only use equal query and
key lengths). With Sq != Sk the diagonal is aligned to the last query and the
last key (bottom-right): query i sees key j iff j <= i + Sk - Sq, so the last
query sees every key, and with Sq > Sk the first Sq - Sk queries see none.
Grouped heads: query head h reads KV head h // (Hq / Hkv). A query row that
sees no key (an empty key sequence, or a row above a bottom-right diagonal)
gets O = 0 and LSE = -inf, and its gradients are 0.

Block-sparse masks (the synthesis page's block-sparse attention built on the
FA4 framework; the pages give no format, so this is a reading): an optional
boolean mask per (batch, query head) with one entry per BLOCK x BLOCK block of
(query, key) pairs, BLOCK = 128 (the tile of the pages' cycle table,
M = N = 128). Query i sees key j iff the causal rule allows it and the entry of
block (i // BLOCK, j // BLOCK) is set; a cleared entry hides every pair of its
block. Fixed length only.

Layouts: fixed length BSHD [B, S, H, d], LSE [B, Hq, Sq]; packed variable
length THD [T, H, d] with cu_seqlens [n + 1], LSE [Hq, T].

The only library step is the float64 matrix product (numpy); rows are processed
in chunks so that memory stays bounded at long sequence lengths.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

_CHUNK = 512
BLOCK = 128   # block-sparse mask granularity (queries and keys per entry)


def _f64(x) -> np.ndarray:
    """bf16/fp32 torch tensor or numpy array -> float64 numpy (exact upcast)."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64, copy=False)
    import torch  # local: the oracle only needs torch to read tensors
    return x.detach().to("cpu", torch.float64).numpy()


def _visible(rows: np.ndarray, nk: int, causal: bool, nq: int,
             bmask: Optional[np.ndarray] = None,
             cols: Optional[np.ndarray] = None) -> Optional[np.ndarray]:
    """Visibility of keys ``cols`` (all ``nk`` keys by default) to query rows
    ``rows`` of a sequence of ``nq`` queries and ``nk`` keys, or None when
    every key is visible. Causal: key j is visible iff j <= i + (nk - nq)
    (bottom-right aligned; plain lower triangular when nq == nk). bmask
    [ceil(nq / BLOCK), ceil(nk / BLOCK)]: key j is visible to row i only if
    the entry of block (i // BLOCK, j // BLOCK) is set."""
    cols = np.arange(nk) if cols is None else np.asarray(cols)
    vis = None
    if causal:
        vis = cols[None, :] <= rows[:, None] + (nk - nq)
    if bmask is not None:
        b = np.asarray(bmask, dtype=bool)[rows[:, None] // BLOCK, cols[None, :] // BLOCK]
        vis = b if vis is None else (vis & b)
    return vis


def head_forward(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float, causal: bool,
                 rows: Optional[np.ndarray] = None,
                 bmask: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One (sequence, head): qh [Sq, d], kh/vh [Sk, d] -> O [n, d], LSE [n].

    ``rows`` selects query rows (absolute indices, for the masks); all rows by
    default. ``bmask``: this head's block mask (see the module docstring).
    """
    sq, d = qh.shape
    sk = kh.shape[0]
    rows = np.arange(sq) if rows is None else np.asarray(rows)
    o = np.zeros((rows.size, vh.shape[1]), dtype=np.float64)
    lse = np.full(rows.size, -np.inf, dtype=np.float64)
    if sk == 0:
        return o, lse
    for c0 in range(0, rows.size, _CHUNK):
        r = rows[c0:c0 + _CHUNK]
        s = scale * (qh[r] @ kh.T)
        vis = _visible(r, sk, causal, sq, bmask)
        if vis is not None:
            s = np.where(vis, s, -np.inf)
        # rows that see no key keep O = 0 and LSE = -inf
        seen = vis.any(axis=1) if vis is not None else np.ones(r.size, dtype=bool)
        if not seen.any():
            continue
        idx = np.nonzero(seen)[0]
        s = s[idx]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        o[c0 + idx] = (e @ vh) / l
        lse[c0 + idx] = (m + np.log(l))[:, 0]
    return o, lse


def head_probs(qh, kh, scale, causal, lse, rows=None, bmask=None) -> np.ndarray:
    """P_ij = exp(s_ij - LSE_i) with hidden entries 0 (small inputs only)."""
    sq = qh.shape[0]
    rows = np.arange(sq) if rows is None else np.asarray(rows)
    s = scale * (qh[rows] @ kh.T)
    vis = _visible(rows, kh.shape[0], causal, sq, bmask)
    with np.errstate(over="ignore"):   # rows with LSE = -inf see no key: P = 0
        p = np.exp(s - lse[:, None])
    if vis is not None:
        p = np.where(vis, p, 0.0)
    return p


def head_backward(qh, kh, vh, doh, scale, causal, bmask=None):
    """One (sequence, query head): returns dQ [Sq, d], dK [Sk, d], dV [Sk, d]
    (dK, dV are this query head's share; grouped heads are summed by the caller)."""
    sq, d = qh.shape
    sk = kh.shape[0]
    dq = np.zeros_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros((sk, vh.shape[1]), dtype=np.float64)
    if sk == 0 or sq == 0:
        return dq, dk, dv
    _, lse_all = head_forward(qh, kh, vh, scale, causal, bmask=bmask)
    for c0 in range(0, sq, _CHUNK):
        r = np.arange(c0, min(sq, c0 + _CHUNK))
        lse = lse_all[r]
        p = head_probs(qh, kh, scale, causal, lse, rows=r, bmask=bmask)   # P
        o = p @ vh                                           # O
        dD = np.sum(doh[r] * o, axis=1)                      # D = rowsum(dO o O)
        dp = doh[r] @ vh.T                                   # dP = dO V^T
        ds = p * (dp - dD[:, None])                          # dS = P o (dP - D)
        dq[r] = scale * (ds @ kh)                            # dQ = alpha dS K
        dk += scale * (ds.T @ qh[r])                         # dK = alpha dS^T Q
        dv += p.T @ doh[r]                                   # dV = P^T dO
    return dq, dk, dv


def head_dq_rows(qh, kh, vh, doh, scale, causal, rows, bmask=None):
    """dQ for selected query rows of one (sequence, head), from the definition
    row by row: P_i from LSE_i, O_i = P_i V, D_i = dO_i . O_i,
    dS_i = P_i (dO_i V^T - D_i), dQ_i = alpha dS_i K."""
    rows = np.asarray(rows)
    _, lse = head_forward(qh, kh, vh, scale, causal, rows=rows, bmask=bmask)
    p = head_probs(qh, kh, scale, causal, lse, rows=rows, bmask=bmask)
    o = p @ vh
    dd = np.sum(doh[rows] * o, axis=1)
    ds = p * (doh[rows] @ vh.T - dd[:, None])
    return scale * (ds @ kh)


def head_dkdv_cols(qh, kh, vh, doh, scale, causal, cols, bmask=None):
    """This query head's share of dK, dV for selected key rows (columns of P):
    needs LSE_i and D_i of every query row, then dK_j = alpha sum_i dS_ij q_i,
    dV_j = sum_i P_ij dO_i."""
    cols = np.asarray(cols)
    sq, sk = qh.shape[0], kh.shape[0]
    o, lse = head_forward(qh, kh, vh, scale, causal, bmask=bmask)
    dd = np.sum(doh * o, axis=1)
    s = scale * (qh @ kh[cols].T)                          # [Sq, n]
    with np.errstate(over="ignore"):
        p = np.exp(s - lse[:, None])
    vis = _visible(np.arange(sq), sk, causal, sq, bmask, cols=cols)
    if vis is not None:
        p = np.where(vis, p, 0.0)
    ds = p * (doh @ vh[cols].T - dd[:, None])
    return scale * (ds.T @ qh), p.T @ doh


def _sequences(q, cu_q, cu_k, k):
    """Yield (seq index, q row slice, k row slice) for BSHD or THD inputs."""
    if cu_q is None:
        for b in range(q.shape[0]):
            yield b, (b, slice(None)), (b, slice(None))
    else:
        cq = [int(x) for x in _f64(cu_q)]
        ck = cq if cu_k is None else [int(x) for x in _f64(cu_k)]
        for s in range(len(cq) - 1):
            yield s, (slice(cq[s], cq[s + 1]),), (slice(ck[s], ck[s + 1]),)


def _head_slice(x, sl, h):
    return x[sl[0], h] if len(sl) == 1 else x[sl[0], sl[1], h]


def _block_mask(block_mask, varlen):
    """[B, Hq, nqb, nkb] boolean block mask (None: no mask); fixed length only."""
    if block_mask is None:
        return None
    if varlen:
        raise ValueError("block masks are defined for fixed-length inputs only")
    return _f64(block_mask) != 0


def attention_forward(q, k, v, scale: float, causal: bool, cu_seqlens_q=None,
                      cu_seqlens_k=None, block_mask=None):
    """Full forward. Returns (O float64 in q's layout, LSE float64)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    varlen = cu_seqlens_q is not None
    bm = _block_mask(block_mask, varlen)
    hq = q.shape[-2]
    hkv = k.shape[-2]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    grp = hq // hkv
    o = np.zeros(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    if varlen:
        lse = np.full((hq, q.shape[0]), -np.inf)
    else:
        lse = np.full((q.shape[0], hq, q.shape[1]), -np.inf)
    for s, qs, ks in _sequences(q, cu_seqlens_q, cu_seqlens_k, k):
        for h in range(hq):
            oh, lh = head_forward(_head_slice(q, qs, h), _head_slice(k, ks, h // grp),
                                  _head_slice(v, ks, h // grp), scale, causal,
                                  bmask=None if bm is None else bm[s, h])
            if varlen:
                o[qs[0], h] = oh
                lse[h, qs[0]] = lh
            else:
                o[s, :, h] = oh
                lse[s, h] = lh
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool, cu_seqlens_q=None,
                       cu_seqlens_k=None, block_mask=None):
    """Exact gradient of sum(dO o O). Returns (dQ, dK, dV) float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    varlen = cu_seqlens_q is not None
    bm = _block_mask(block_mask, varlen)
    hq, hkv = q.shape[-2], k.shape[-2]
    grp = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for s, qs, ks in _sequences(q, cu_seqlens_q, cu_seqlens_k, k):
        for h in range(hq):
            g = h // grp
            dqh, dkh, dvh = head_backward(_head_slice(q, qs, h), _head_slice(k, ks, g),
                                          _head_slice(v, ks, g), _head_slice(do, qs, h),
                                          scale, causal, bmask=None if bm is None else bm[s, h])
            if varlen:
                dq[qs[0], h] = dqh
                dk[ks[0], g] += dkh
                dv[ks[0], g] += dvh
            else:
                dq[s, :, h] = dqh
                dk[s, :, g] += dkh
                dv[s, :, g] += dvh
    return dq, dk, dv


def attention_probs(q, k, scale, causal, lse):
    """P for fixed-length inputs [B, Hq, Sq, Sk] (small inputs only)."""
    q, k = _f64(q), _f64(k)
    hq, hkv = q.shape[2], k.shape[2]
    grp = hq // hkv
    out = np.zeros((q.shape[0], hq, q.shape[1], k.shape[1]))
    for b in range(q.shape[0]):
        for h in range(hq):
            out[b, h] = head_probs(q[b, :, h], k[b, :, h // grp], scale, causal, lse[b, h])
    return out


def rowsum_do_o(do, o) -> np.ndarray:
    """D = rowsum(dO o O) over the head dimension, in float64."""
    return np.sum(_f64(do) * _f64(o), axis=-1)


def repeat_kv(x, groups: int) -> np.ndarray:
    """[.., Hkv, d] -> [.., Hkv*groups, d], KV head g repeated for heads g*G..g*G+G-1."""
    return np.repeat(_f64(x), groups, axis=-2)
