// Varlen pre-pass (FlashAttention-4 blog page, scheduling section: a
// preprocessing kernel sorts the batches by their longest tile and writes a
// virtual-to-actual batch map that the attention kernel walks). One
// workgroup: each thread ranks some sequences (rank = number of longer
// sequences, ties broken by index, so the map is a permutation), then one
// thread writes the prefix sums of tiles over the sorted order.
#include "common.hpp"
#include "kernels.hpp"
#include "schedule.hpp"

namespace attn71 {

namespace {

__global__ __launch_bounds__(256) void varlen_schedule_kernel(const int* __restrict__ key_cu,
                                                              const int* __restrict__ count_cu,
                                                              const int* __restrict__ q_cu,
                                                              int nseq, int heads, int blk,
                                                              int* order, int* tile_prefix,
                                                              int* mb_prefix, int mb_blk,
                                                              unsigned* queue,
                                                              int64_t* ds_prefix, int ds_heads,
                                                              int causal) {
  for (int s = threadIdx.x; s < nseq; s += blockDim.x) order[varlen_rank(key_cu, nseq, s)] = s;
  if (queue && threadIdx.x == 128) *queue = 0u;   // tile tickets of the launch that follows
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    tile_prefix[0] = 0;
    for (int vs = 0; vs < nseq; ++vs) {
      const int s = order[vs];
      acc += cdiv(count_cu[s + 1] - count_cu[s], blk) * heads;
      tile_prefix[vs + 1] = acc;
    }
  } else if (threadIdx.x == 64 && mb_prefix) {
    int acc = 0;
    mb_prefix[0] = 0;
    for (int s = 0; s < nseq; ++s) {
      acc += cdiv(q_cu[s + 1] - q_cu[s], mb_blk);
      mb_prefix[s + 1] = acc;
    }
  } else if (threadIdx.x == 192 && ds_prefix) {
    int64_t acc = 0;
    ds_prefix[0] = 0;
    for (int s = 0; s < nseq; ++s) {
      acc += (int64_t)ds_heads *
             ds_region_tiles(ds_geom(q_cu[s + 1] - q_cu[s], count_cu[s + 1] - count_cu[s], causal != 0));
      ds_prefix[s + 1] = acc;
    }
  }
}

}  // namespace

hipError_t launch_varlen_schedule(const int* key_cu, const int* count_cu, const int* q_cu,
                                  int nseq, int heads, int blk, int* order, int* tile_prefix,
                                  int* mb_prefix, int mb_blk, unsigned* queue,
                                  int64_t* ds_prefix, int ds_heads, int causal,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(256), 0, stream, key_cu, count_cu,
                     q_cu, nseq, heads, blk, order, tile_prefix, mb_prefix, mb_blk, queue,
                     ds_prefix, ds_heads, causal);
  return hipGetLastError();
}

}  // namespace attn71
