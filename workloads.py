"""Seeded synthetic workloads for the exact-attention hot path.

This module only draws random inputs and counts algorithmic work. It holds none
of the attention arithmetic, so both the float64 oracle (``oracle/``) and the
HIP path (``exact_attention_71_amd``) can be fed from it without sharing code.

Recipe (the same for every workload): a ``torch.Generator`` seeded with
``71000 + workload number`` draws, in this order, the sequence lengths (varlen
only), then Q, K, V and dO as float32 N(0, 1); where a workload asks for it the
first half of the query heads of Q and K (and the matching KV heads of K) are
multiplied by 3; every tensor is then rounded once, round-to-nearest-even, to
bfloat16. Layout is BSHD ``[B, S, H, d]`` for fixed length and THD ``[T, H, d]``
for packed variable-length batches, with ``cu_seqlens`` int32 ``[n + 1]``.

Work counting follows the roofline convention of the FlashAttention-4 pages
(digest page, roofline paragraph under the notation table): a forward pass does
two GEMMs of 2*M*N*d flops each, i.e. 4*M*N*d per (query, key) block, and the
backward pass does five, 2.5x the forward; causal masking halves both.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    number: int
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int            # fixed length Sq = Sk (ignored for varlen)
    head_dim: int
    causal: bool
    passes: str            # "fwd" or "fwd+bwd"
    scaled_heads: bool = False     # x3 on Q and K of the first half of the heads
    varlen: bool = False
    num_seqs: int = 0
    len_lo: int = 0
    len_hi: int = 0
    deterministic: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / (self.head_dim ** 0.5)


WORKLOADS: Dict[str, Workload] = {
    "small": Workload("small", 1, 1, 2, 2, 256, 64, False, "fwd+bwd"),
    "fwd4k": Workload("fwd4k", 2, 4, 16, 16, 4096, 128, False, "fwd"),
    "causal8k": Workload("causal8k", 3, 2, 16, 16, 8192, 128, True, "fwd+bwd",
                         scaled_heads=True),
    "varlen_gqa": Workload("varlen_gqa", 4, 16, 32, 4, 0, 128, True, "fwd+bwd",
                           varlen=True, num_seqs=16, len_lo=512, len_hi=8192),
    "det16k_d64": Workload("det16k_d64", 5, 1, 8, 8, 16384, 64, True, "fwd+bwd",
                           deterministic=True),
    "det16k_d128": Workload("det16k_d128", 5, 1, 8, 8, 16384, 128, True, "fwd+bwd",
                            deterministic=True),
    "det16k_d256": Workload("det16k_d256", 5, 1, 8, 8, 16384, 256, True, "fwd+bwd",
                            deterministic=True),
}


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def draw_lengths(num_seqs: int, lo: int, hi: int, seed: int) -> List[int]:
    """Integer sequence lengths uniform on [lo, hi] inclusive (CPU generator)."""
    g = _gen(seed, "cpu")
    return torch.randint(lo, hi + 1, (num_seqs,), generator=g).tolist()


def cu_from_lengths(lengths: List[int]) -> torch.Tensor:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def make_inputs(batch: int, seqlen_q: int, seqlen_k: int, heads_q: int, heads_kv: int,
                head_dim: int, seed: int, device: str = "cpu", scaled_heads: bool = False,
                lengths: Optional[List[int]] = None, lengths_k: Optional[List[int]] = None,
                with_grad: bool = True) -> Dict[str, torch.Tensor]:
    """Draw bf16 Q, K, V (and dO) from N(0, 1).

    Fixed length: BSHD tensors. When ``lengths`` is given the batch is packed
    THD with ``cu_seqlens_q``/``cu_seqlens_k`` (``lengths_k`` defaults to
    ``lengths``).
    """
    g = _gen(seed, device)
    out: Dict[str, torch.Tensor] = {}
    if lengths is not None:
        lk = lengths if lengths_k is None else lengths_k
        tq, tk = int(sum(lengths)), int(sum(lk))
        shp_q, shp_k = (tq, heads_q, head_dim), (tk, heads_kv, head_dim)
        out["cu_seqlens_q"] = cu_from_lengths(lengths)
        out["cu_seqlens_k"] = cu_from_lengths(lk)
    else:
        shp_q = (batch, seqlen_q, heads_q, head_dim)
        shp_k = (batch, seqlen_k, heads_kv, head_dim)
    q = torch.randn(shp_q, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(shp_k, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shp_k, generator=g, device=device, dtype=torch.float32)
    if scaled_heads:
        q[..., : heads_q // 2, :] *= 3.0
        k[..., : max(1, heads_kv // 2), :] *= 3.0
    out["q"] = q.to(torch.bfloat16)
    out["k"] = k.to(torch.bfloat16)
    out["v"] = v.to(torch.bfloat16)
    del q, k, v
    if with_grad:
        do = torch.randn(shp_q, generator=g, device=device, dtype=torch.float32)
        out["do"] = do.to(torch.bfloat16)
    return out


def workload_inputs(w: Workload, device: str = "cpu", with_grad: bool = True,
                    seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    seed = 71000 + w.number if seed is None else seed
    if w.varlen:
        lengths = draw_lengths(w.num_seqs, w.len_lo, w.len_hi, seed)
        return make_inputs(w.num_seqs, 0, 0, w.heads_q, w.heads_kv, w.head_dim, seed + 1,
                           device=device, lengths=lengths, with_grad=with_grad,
                           scaled_heads=w.scaled_heads)
    return make_inputs(w.batch, w.seqlen, w.seqlen, w.heads_q, w.heads_kv, w.head_dim, seed,
                       device=device, scaled_heads=w.scaled_heads, with_grad=with_grad)


# ---------------------------------------------------------------- work counting
def pair_count(lengths_q: List[int], lengths_k: List[int], causal: bool) -> float:
    """Number of (query, key) pairs the flop convention counts.

    Non-causal: Lq * Lk per sequence.  Causal: half of it, as in the pages'
    convention (not the exact triangle count Lq*(Lq+1)/2).
    """
    tot = 0.0
    for lq, lk in zip(lengths_q, lengths_k):
        tot += float(lq) * float(lk) * (0.5 if causal else 1.0)
    return tot


def attention_flops(lengths_q: List[int], lengths_k: List[int], heads_q: int, head_dim: int,
                    causal: bool) -> Dict[str, float]:
    """Algorithmic flops: forward 4*pairs*d per head, backward 2.5x forward."""
    fwd = 4.0 * pair_count(lengths_q, lengths_k, causal) * heads_q * head_dim
    return {"fwd": fwd, "bwd": 2.5 * fwd, "fwd+bwd": 3.5 * fwd}


def tile_cycles(m: int, n: int, d: int, mma_ops_per_clk: float, exp_ops_per_clk: float) -> Dict[str, float]:
    """Per-tile cycle model of the pages: T_MMA fwd = 4MNd/rate, bwd = 10MNd/rate,
    T_exp = MN/rate (independent of d)."""
    return {"mma_fwd": 4.0 * m * n * d / mma_ops_per_clk,
            "mma_bwd": 10.0 * m * n * d / mma_ops_per_clk,
            "exp": float(m * n) / exp_ops_per_clk}


def workload_flops(w: Workload, lengths: Optional[List[int]] = None) -> Dict[str, float]:
    if w.varlen:
        assert lengths is not None
        return attention_flops(lengths, lengths, w.heads_q, w.head_dim, w.causal)
    return attention_flops([w.seqlen] * w.batch, [w.seqlen] * w.batch, w.heads_q, w.head_dim,
                           w.causal)
