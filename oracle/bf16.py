"""bfloat16 rounding and spacing, from the format's definition.

Test infrastructure: see ``oracle/__init__.py``.

bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and float32's
exponent range.  Rounding is to nearest, ties to even.  The largest relative
error of that rounding, 2^-8 / (1 + 2^-8) = 3.891e-3, is the "BF16
quantisation error 3.89e-3" the FlashAttention-4 digest page compares the exp2
polynomial against (item 2).
"""
from __future__ import annotations

import numpy as np

_MIN_EXP = -126          # smallest normal exponent (x = m * 2^e, 1 <= m < 2)
_SIG = 8                 # significant bits


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    Works directly on float64 (no intermediate float32 rounding).  Values past
    the largest finite bfloat16 become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    ax = np.abs(x[fin])
    e = np.floor(np.log2(ax))
    # guard the log2 rounding at exact powers of two
    e = np.where(np.exp2(e) > ax, e - 1, e)
    e = np.where(np.exp2(e + 1) <= ax, e + 1, e)
    e = np.maximum(e, _MIN_EXP)                   # subnormals share the min spacing
    spacing = np.exp2(e - (_SIG - 1))
    r = np.rint(ax / spacing) * spacing            # rint: ties to even
    r = np.where(r > 3.3895313892515355e38, np.inf, r)
    out[fin] = np.sign(x[fin]) * r
    return out


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (distance to the next larger magnitude)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    safe = np.where(ax > 0, ax, 1.0)
    e = np.floor(np.log2(safe))
    e = np.where(np.exp2(e) > safe, e - 1, e)
    e = np.where(np.exp2(e + 1) <= safe, e + 1, e)
    e = np.where(ax > 0, np.maximum(e, _MIN_EXP), _MIN_EXP)
    return np.exp2(e - (_SIG - 1))
