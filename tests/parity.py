"""Comparison helpers for the GPU parity tests (HIP path vs the float64 oracle).

Criteria, from the stated pass bar for bf16 inputs:
  O    max-abs <= 1e-2 beyond the output's own bf16 rounding (half a bf16 ulp
       of the oracle value, which no bf16 output can avoid), mean-abs <= 1e-3;
       and, where the bf16 spacing allows it (|O| < 2, spacing <= 2^-7), the
       error against the oracle rounded to bf16 is <= 1e-2 as well (the
       survey's proposal for the tolerance conflict of large outputs);
  LSE  max-abs <= 1e-3;
  dQ, dK, dV  relative L2 <= 2e-2.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

O_MAX, O_MEAN, LSE_MAX, GRAD_REL = 1e-2, 1e-3, 1e-3, 2e-2


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def o_errors(o_gpu, o_ref: np.ndarray) -> dict:
    g = to64(o_gpu) if isinstance(o_gpu, torch.Tensor) else o_gpu
    err = np.abs(g - o_ref)
    half_ulp = 0.5 * oracle.bf16_ulp(o_ref)
    floor = np.abs(oracle.round_bf16(o_ref) - o_ref)
    vs_rounded = np.abs(g - oracle.round_bf16(o_ref))
    small = np.abs(o_ref) < 2.0
    return {"max_abs": float(err.max(initial=0.0)),
            "max_excess": float(np.max(err - half_ulp, initial=0.0)),
            "mean_abs": float(err.mean()) if err.size else 0.0,
            "max_vs_rounded_ref": float(vs_rounded.max(initial=0.0)),
            "max_vs_rounded_ref_below2": float(vs_rounded[small].max(initial=0.0)),
            "bf16_floor": float(floor.max(initial=0.0))}


def check_o(o_gpu, o_ref, what=""):
    e = o_errors(o_gpu, o_ref)
    assert e["max_excess"] <= O_MAX and e["mean_abs"] <= O_MEAN, (what, e)
    assert e["max_vs_rounded_ref_below2"] <= O_MAX, (what, e)
    return e


def check_lse(lse_gpu, lse_ref, what=""):
    g = to64(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(g), fin), (what, "non-finite pattern differs")
    err = float(np.abs(g[fin] - lse_ref[fin]).max(initial=0.0))
    assert err <= LSE_MAX, (what, err)
    return err


def rel_l2(a, ref) -> float:
    a = to64(a) if isinstance(a, torch.Tensor) else a
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / (den if den > 0 else 1.0))


def check_grads(got, ref, what=""):
    out = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        out[name] = rel_l2(g, r)
        assert out[name] <= GRAD_REL, (what, name, out)
    return out
