"""Float64 CPU oracle for the fused exact-attention hot path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here. The HIP
library never calls, links or falls back to this code, and this code imports
nothing from the HIP package: the two share no kernels, helpers, tables or
constants. Inputs come from ``workloads.py`` (random numbers only).

Contents
--------
attention.py   the definition of exact attention, its LSE and its gradient,
               written out in float64 (numpy matmul is the only library step).
blockwise.py   the tiled online-softmax forward with conditional rescaling,
               following the steps of the FlashAttention-4 pages in their order;
               used to show that skipping small rescales reaches the definition.
exp2poly.py    the Cody-Waite + degree-3 Horner exp2 and a minimax refit of its
               coefficients.
bf16.py        round-to-nearest-even to bfloat16 and bf16 spacing (ulp).

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (a library routine, finite differences, closed forms, invariants or
a number printed on the pages); see ``tests/test_oracle_*.py``.
"""
from .attention import (attention_forward, attention_backward, attention_probs,
                        rowsum_do_o, repeat_kv, head_forward, head_backward, head_dq_rows,
                        head_dkdv_cols)
from .blockwise import blockwise_forward
from .exp2poly import exp2_cody_waite, fit_exp2_minimax, PAGE_COEFFS
from .bf16 import round_bf16, bf16_ulp

__all__ = ["attention_forward", "attention_backward", "attention_probs", "rowsum_do_o",
           "repeat_kv", "head_forward", "head_backward", "head_dq_rows", "head_dkdv_cols", "blockwise_forward", "exp2_cody_waite", "fit_exp2_minimax",
           "PAGE_COEFFS", "round_bf16", "bf16_ulp"]
