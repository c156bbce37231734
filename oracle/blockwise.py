"""Tiled online-softmax forward with conditional rescaling (algorithm model).

Test infrastructure: see ``oracle/__init__.py``.

This model runs the forward the way the FlashAttention-4 pages describe it, in
their order, so that tests can show the method reaches the exact result of
``attention.head_forward``:

* S_j = Q K_j^T for one key tile j, turned into base-2 units
  s' = alpha * log2(e) * s (the threshold is given as tau = log2(256) = 8.0,
  digest page, item 3 "conditional softmax rescaling"; blog page, forward
  section, rescaling equation);
* running row max m_j = max(m_{j-1}, rowmax S_j) (digest page, item 3);
* the rescale of the output accumulator and of the row sum happens only when
  the jump m_j - m_{j-1} exceeds tau; otherwise the old reference max is kept
  and P_j = 2^(S_j - m_{j-1}) is accumulated against it (blog page, forward
  section, the two-case equation for O_j);
* the decision is taken once per group of rows that execute together (a warp on
  the pages, a wavefront here) so that they do not diverge (blog page, end of
  the correction-warpgroup paragraph).  Reading used: the group rescales when
  ANY of its rows jumps by more than tau, and each row then moves to its own
  new max;
* the final output is divided by the true accumulated statistics,
  O = O_acc / l, and LSE = ln(2) * (m + log2 l) (blog page, the final
  normalisation and "optionally compute and store LSE").

Readings for points the pages leave open: the reference max starts at -inf, so
the first tile always rescales, with factor 0 for the empty accumulator; a row
whose reference max is still -inf uses 0 as the exponent offset; the row sum is
taken over the unrounded p, and only the copy of P that feeds the P V product
may be rounded (``round_p``).
"""
from __future__ import annotations

import math
from typing import Callable, Optional

import numpy as np

from .attention import _f64

LOG2E = 1.0 / math.log(2.0)


def _group_forward(qg, kh, vh, rows, scale, causal, block_n, tau, exp2, dt, round_p, stats,
                   off=0):
    """One decision group of query rows (absolute indices ``rows``); under the
    causal mask row i sees keys j <= i + ``off``."""
    n_rows = rows.size
    sk = kh.shape[0]
    m_ref = np.full(n_rows, -np.inf, dtype=dt)
    l = np.zeros(n_rows, dtype=dt)
    acc = np.zeros((n_rows, vh.shape[1]), dtype=dt)
    last_key = max(0, int(rows.max()) + 1 + off) if causal else sk
    n_tiles = -(-min(last_key, sk) // block_n)
    c = dt(scale * LOG2E)
    for t in range(n_tiles):
        cols = np.arange(t * block_n, min(sk, (t + 1) * block_n))
        s = (qg @ kh[cols].T).astype(dt) * c                     # S_j in log2 units
        if causal:
            s = np.where(cols[None, :] <= rows[:, None] + off, s, dt(-np.inf))
        m_new = np.maximum(m_ref, s.max(axis=1))                   # m_j
        with np.errstate(invalid="ignore"):
            jump = m_new - m_ref
        if np.any(jump > tau):                                     # one decision per group
            with np.errstate(invalid="ignore"):                    # rows that saw no key yet
                fac = np.where(np.isneginf(m_ref), dt(0.0),
                               exp2((np.where(np.isneginf(m_ref), m_new, m_ref) - m_new).astype(dt)))
            acc = acc * fac[:, None].astype(dt)
            l = l * fac.astype(dt)
            m_ref = m_new
            stats["rescaled"] += 1
        else:
            stats["skipped"] += 1
        m_use = np.where(np.isneginf(m_ref), dt(0.0), m_ref).astype(dt)
        p = exp2((s - m_use[:, None]).astype(dt)).astype(dt)       # P_j = 2^(S_j - m_ref)
        stats["max_p"] = max(stats["max_p"], float(p.max()) if p.size else 0.0)
        l = (l + p.sum(axis=1, dtype=dt)).astype(dt)               # row sum of unrounded p
        pv = p if round_p is None else round_p(p).astype(dt)
        acc = (acc + (pv @ vh[cols]).astype(dt)).astype(dt)       # O_j
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(l[:, None] > 0, acc / l[:, None], 0.0)
        lse = np.where(l > 0, math.log(2.0) * (m_ref.astype(np.float64)
                                               + np.log2(l.astype(np.float64))), -np.inf)
    return o.astype(np.float64), lse


def blockwise_forward(q, k, v, scale: float, causal: bool, block_m: int = 128,
                      block_n: int = 64, group_rows: int = 32, tau: float = 8.0,
                      exp2: Optional[Callable] = None, dtype=np.float64,
                      round_p: Optional[Callable] = None, stats: Optional[dict] = None):
    """Fixed-length BSHD forward through the tiled algorithm.

    ``block_m`` rows form one workgroup tile, split into decision groups of
    ``group_rows`` rows; ``block_n`` keys per tile; ``tau`` in log2 units
    (``tau = 0`` rescales whenever the max grows, ``tau = inf`` never after the
    first tile).  ``dtype`` float32 simulates single-precision arithmetic.
    Returns (O, LSE) in the layouts of ``attention.attention_forward``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    dt = np.dtype(dtype).type
    exp2 = exp2 if exp2 is not None else (lambda x: np.exp2(x))
    if stats is None:
        stats = {}
    stats.setdefault("rescaled", 0)
    stats.setdefault("skipped", 0)
    stats.setdefault("max_p", 0.0)
    bsz, sq, hq, d = q.shape
    hkv, sk = k.shape[2], k.shape[1]
    grp = hq // hkv
    o = np.zeros(q.shape[:-1] + (v.shape[-1],))
    lse = np.full((bsz, hq, sq), -np.inf)
    for b in range(bsz):
        for h in range(hq):
            qh = q[b, :, h].astype(dt)
            kh = k[b, :, h // grp].astype(dt)
            vh = v[b, :, h // grp].astype(dt)
            for m0 in range(0, sq, block_m):
                for r0 in range(m0, min(sq, m0 + block_m), group_rows):
                    rows = np.arange(r0, min(sq, r0 + group_rows, m0 + block_m))
                    og, lg = _group_forward(qh[rows], kh, vh, rows, scale, causal, block_n,
                                            tau, exp2, dt, round_p, stats, off=sk - sq)
                    o[b, rows, h] = og
                    lse[b, h, rows] = lg
    return o, lse
