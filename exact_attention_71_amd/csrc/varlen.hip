// Varlen pre-pass (FlashAttention-4 blog page, scheduling section: a
// preprocessing kernel sorts the batches by their longest tile and writes a
// virtual-to-actual batch map that the attention kernel walks; the metadata
// can be cached). One workgroup computes one or more schedule tables, one
// after the other: for each, every thread ranks some sequences (rank =
// number of longer sequences, ties broken by index, so the map is a
// permutation), then single threads write the prefix sums over the sorted
// order (tiles), over the natural order (query blocks for the deterministic
// chain; stored-dS regions) and clear the table's tile-ticket counter. Key-block
// tables may also rank every key block of every sequence in one
// longest-first list (the pages' ordering applied to single tiles rather than
// whole sequences): with 16 sequences of 512 to 8192 tokens, a list
// scheduling model of the per-sequence order keeps the CUs 92 % busy, the
// global order 99 %.
#include "common.hpp"
#include "kernels.hpp"
#include "schedule.hpp"

namespace attn71 {

namespace {

// sequences whose lengths the key-block ranking stages in LDS (the host
// enables the ranking for at most 361: key blocks x sequences <= 2^17)
constexpr int kRankMaxSeq = 512;

__global__ __launch_bounds__(256) void varlen_schedule_kernel(SchedArgs a) {
  __shared__ int len_q[kRankMaxSeq], len_k[kRankMaxSeq];
  for (int i = 0; i < a.nsets; ++i) {
    const SchedSet& t = a.set[i];
    for (int s = threadIdx.x; s < a.nseq; s += blockDim.x)
      t.order[varlen_rank(t.key_cu, a.nseq, s)] = s;
    if (t.queue && threadIdx.x == 128) *t.queue = 0u;   // tile tickets of the launches that follow
    if (t.key_tiles) {
      // every key block of every sequence, ranked among all of them; the
      // lengths staged in LDS (the ranking reads each nseq times per block)
      const bool staged = a.nseq <= kRankMaxSeq;
      if (staged) {
        for (int s = threadIdx.x; s < a.nseq; s += blockDim.x) {
          len_q[s] = a.q_cu[s + 1] - a.q_cu[s];
          len_k[s] = t.count_cu[s + 1] - t.count_cu[s];
        }
      }
      __syncthreads();
      int nkb = 0;
      if (staged)
        for (int s = 0; s < a.nseq; ++s) nkb += imax(0, cdiv(len_k[s], t.blk));
      const bool fits = staged && nkb <= t.key_cap;
      if (threadIdx.x == 0) t.key_tiles[0] = fits ? 1 : 0;
      if (fits) {
        for (int e = threadIdx.x; e < nkb; e += blockDim.x) {
          int s, b;
          key_block_at(len_k, a.nseq, t.blk, e, &s, &b);
          const int r = key_block_rank(len_q, len_k, a.nseq, t.rank_bm, t.blk, t.causal != 0, s, b);
          if (s >= 0 && r >= 0 && r < nkb) {
            t.key_tiles[2 + 2 * r] = s;
            t.key_tiles[3 + 2 * r] = b;
          }
        }
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int acc = 0;
      t.tile_prefix[0] = 0;
      for (int vs = 0; vs < a.nseq; ++vs) {
        const int s = t.order[vs];
        acc += cdiv(t.count_cu[s + 1] - t.count_cu[s], t.blk) * t.heads;
        t.tile_prefix[vs + 1] = acc;
      }
    } else if (threadIdx.x == 64 && t.mb_prefix) {
      int acc = 0;
      t.mb_prefix[0] = 0;
      for (int s = 0; s < a.nseq; ++s) {
        acc += cdiv(a.q_cu[s + 1] - a.q_cu[s], t.mb_blk);
        t.mb_prefix[s + 1] = acc;
      }
    } else if (threadIdx.x == 192 && t.ds_prefix) {
      // stored-dS regions of the sequences in order; a sequence whose regions
      // would end past the area (lengths beyond the declared maxima), or whose
      // key-block columns exceed 32-bit offsets, gets -1
      int64_t acc = 0;
      for (int s = 0; s < a.nseq; ++s) {
        const DsGeom g = ds_geom(a.q_cu[s + 1] - a.q_cu[s], t.count_cu[s + 1] - t.count_cu[s],
                                 t.causal != 0);
        const int64_t reg = (int64_t)t.ds_heads * ds_region_tiles(g);
        t.ds_prefix[s] = acc + reg <= t.ds_tiles && g.rows < kDsMaxRows ? acc : -1;
        acc += reg;
      }
      t.ds_prefix[a.nseq] = acc;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_varlen_schedule(const SchedArgs& a, hipStream_t stream) {
  if (a.nsets <= 0) return hipSuccess;
  hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn71
