// Varlen pre-pass (FlashAttention-4 blog page, scheduling section: a
// preprocessing kernel sorts the batches by their longest tile and writes a
// virtual-to-actual batch map that the attention kernel walks; the metadata
// can be cached). One workgroup computes one or more schedule tables, one
// after the other: for each, every thread ranks some sequences (rank =
// number of longer sequences, ties broken by index, so the map is a
// permutation), then single threads write the prefix sums over the sorted
// order (tiles), over the natural order (query blocks for the deterministic
// chain; stored-dS regions) and clear the table's tile-ticket counter.
#include "common.hpp"
#include "kernels.hpp"
#include "schedule.hpp"

namespace attn71 {

namespace {

__global__ __launch_bounds__(256) void varlen_schedule_kernel(SchedArgs a) {
  for (int i = 0; i < a.nsets; ++i) {
    const SchedSet& t = a.set[i];
    for (int s = threadIdx.x; s < a.nseq; s += blockDim.x)
      t.order[varlen_rank(t.key_cu, a.nseq, s)] = s;
    if (t.queue && threadIdx.x == 128) *t.queue = 0u;   // tile tickets of the launches that follow
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
