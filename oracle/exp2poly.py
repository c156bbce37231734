"""Software 2^x: Cody-Waite range reduction + degree-3 Horner polynomial.

Test infrastructure: see ``oracle/__init__.py``.

Method (FlashAttention-4 blog page, section on the faster exponential; digest
page, item 2 "software-emulated exp"):

1. range reduction 2^x = 2^floor(x) * 2^(x - floor(x)), n = floor(x),
   f = x - n in [0, 1);
2. 2^f ~= p0 + p1 f + p2 f^2 + p3 f^3 evaluated in Horner form, with p0 = 1
   and the other coefficients chosen to minimise the maximum RELATIVE error on
   [0, 1) (the pages print p1 ~ 0.6951, p2 ~ 0.2276, p3 ~ 0.0771 and a float32
   maximum relative error of 8.77e-5);
3. multiplication by 2^n is an integer add of n into the float32 exponent
   field (2^f lies in [1, 2), whose biased exponent is 127).

Reading for an edge the pages leave open: inputs below -126 flush to 0, which
keeps step 3 inside the normal range (the attention path only ever asks for
x <= tau = 8, so there is no overflow side).
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

# Coefficients as printed (blog page, faster-exponential section).
PAGE_COEFFS: Tuple[float, float, float, float] = (1.0, 0.6951, 0.2276, 0.0771)


def exp2_cody_waite(x, coeffs: Sequence[float] = PAGE_COEFFS) -> np.ndarray:
    """2^x in float32 arithmetic (each Horner step rounded to float32)."""
    x = np.asarray(x, dtype=np.float32)
    flush = ~(x >= np.float32(-126.0))          # also catches -inf and NaN
    xs = np.where(flush, np.float32(0.0), x).astype(np.float32)
    n = np.floor(xs).astype(np.float32)
    f = (xs - n).astype(np.float32)              # exact: |x| < 2^23
    p0, p1, p2, p3 = (np.float32(c) for c in coeffs)
    p = (p3 * f + p2).astype(np.float32)
    p = (p * f + p1).astype(np.float32)
    p = (p * f + p0).astype(np.float32)          # ~2^f in [1, 2)
    bits = p.view(np.int32) + (n.astype(np.int32) << 23)
    out = bits.view(np.float32)
    return np.where(flush, np.float32(0.0), out).astype(np.float32)


def max_rel_error(coeffs: Sequence[float], f: np.ndarray) -> float:
    """max |poly(f) - 2^f| / 2^f on the given points, in float64."""
    p0, p1, p2, p3 = (float(c) for c in coeffs)
    f = np.asarray(f, dtype=np.float64)
    poly = ((p3 * f + p2) * f + p1) * f + p0
    return float(np.max(np.abs(poly / np.exp2(f) - 1.0)))


def fit_exp2_minimax(n_points: int = 4001, p0: float = 1.0) -> Tuple[Tuple[float, ...], float]:
    """Minimax relative-error fit of p1..p3 with p0 fixed, as a linear program.

    minimise t  subject to  |p0 + p1 f + p2 f^2 + p3 f^3 - 2^f| <= t * 2^f
    on a grid of [0, 1]; returns ((p0, p1, p2, p3), t).
    """
    from scipy.optimize import linprog

    f = np.linspace(0.0, 1.0, n_points)
    w = np.exp2(f)
    basis = np.stack([f, f * f, f ** 3], axis=1)          # columns for p1..p3
    rhs = w - p0
    # poly - w <= t w  ->  basis.p - t w <= w - p0 ; -(poly - w) <= t w -> -basis.p - t w <= p0 - w
    a_ub = np.concatenate([np.concatenate([basis, -w[:, None]], axis=1),
                           np.concatenate([-basis, -w[:, None]], axis=1)])
    b_ub = np.concatenate([rhs, -rhs])
    res = linprog(c=[0, 0, 0, 1], A_ub=a_ub, b_ub=b_ub,
                  bounds=[(None, None)] * 3 + [(0, None)], method="highs")
    if not res.success:
        raise RuntimeError(res.message)
    p1, p2, p3, t = res.x
    return (p0, float(p1), float(p2), float(p3)), float(t)
