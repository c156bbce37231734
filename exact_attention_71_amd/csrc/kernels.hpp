// Kernel argument blocks and launchers shared by the host API and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn71 {

// Softmax rescale threshold in base-2 units: tau = log2(256) = 8.0
// (FlashAttention-4 digest page, item 3; blog page, forward rescaling equation).
constexpr float kTau = 8.0f;   // default rescale threshold, log2 units (log2 256)

struct SeqView {
  const int* cu_q;        // packed varlen offsets (device), null for fixed length
  const int* cu_k;
  int batch;              // fixed: B; varlen: number of sequences
  int seqlen_q, seqlen_k; // fixed length only
  int total_q;            // rows of the packed q (varlen LSE stride)
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;             // may be null
  SeqView sv;
  const int* order;       // varlen: virtual -> actual sequence
  const int* tile_prefix; // varlen: first tile of each virtual sequence
  int hq, hkv, group;
  int nm;                 // fixed: query blocks per sequence
  int sec, nxcd;
  int natural;            // 1: plain tile order (tuning / ablation)
  int ntiles;             // tiles of the launch (varlen: upper bound)
  unsigned* queue;        // varlen: tile ticket counter (null: static walk)
  int causal;
  float alpha;            // softmax scale
  float scale_log2;       // alpha * log2(e)
  float tau;              // rescale threshold on the running-max jump, log2 units
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;            // -D = -rowsum(dO o O), same layout as LSE (negated: the
                          // dK/dV kernel starts its dP accumulators from it)
  float* lse2;            // LSE * log2(e), same layout as LSE
  float* dq_acc;          // fp32 [rows][Hq][d]
  int* sem;               // deterministic: one counter per (query block, query head)
  int* ticket;            // deterministic: workgroup ticket counter
  int* status;            // error word (non-zero: a bounded wait expired)
  SeqView sv;
  const int* order;       // varlen: virtual -> actual sequence (by key length)
  const int* tile_prefix; // varlen: first tile of each virtual sequence
  const int* mb_prefix;   // varlen: query-block prefix per actual sequence
  int hq, hkv, group;
  int nn;                 // fixed: key blocks per sequence
  int nm;                 // fixed: query blocks per sequence
  int sec, nxcd;
  int natural;            // 1: plain tile order (non-deterministic only)
  int ntiles;             // dK/dV (or fused) tiles of the launch (varlen: upper bound)
  int ntiles_dq;          // dQ kernel tiles (varlen: upper bound)
  unsigned* queue;        // varlen: dK/dV tile ticket counter (null: static walk)
  unsigned* queue_dq;     // varlen: dQ tile ticket counter
  int causal, deterministic;
  float alpha;
  float scale_log2;
  const int* order_dq;    // varlen: dQ kernel schedule (by key length)
  const int* tile_prefix_dq;
  int nm_dq;              // fixed: query blocks of the dQ kernel per sequence
  int sec_dq;
  int zero_acc;           // preprocess clears the fp32 dQ accumulator (fused path)
  int64_t rows_q;         // total query rows (B*Sq or total_q)
  int64_t n_sem;          // semaphore words to clear (deterministic)
  int spin_limit;         // bounded wait for the deterministic chain
  // Stored dS (null: the dQ kernel recomputes S and dP). Per (sequence,
  // query head): ds_nq32_of(Lq) x ds_nk32_of(Lk) sub-tiles of 32 queries x 32
  // keys, bf16, 2 KiB each, in the register order of the dK/dV kernel; the
  // regions of the heads of a sequence follow each other, sequences in order.
  char* ds;
  const int64_t* ds_prefix;  // varlen: first sub-tile of each sequence (null: fixed length)
  int64_t ds_bytes;          // size of the dS area (regions are clamped to it)
};

// Stored-dS geometry: query blocks of 32 rounded to the dK/dV step (64 rows
// at most), key blocks of 32 rounded to the dK/dV workgroup (256 keys at
// most), so every sub-tile the dK/dV kernel writes lies inside its head.
__host__ __device__ inline int ds_nq32_of(int seqlen_q) { return (seqlen_q + 63) / 64 * 2; }
__host__ __device__ inline int ds_nk32_of(int seqlen_k) { return (seqlen_k + 255) / 256 * 8; }

// Byte offset from p.ds of the stored-dS region of (sequence s, query head h)
// with lq queries and lk keys; *bh_bytes = the region's size, clamped to the
// dS area (packed lengths beyond the maximum the caller declared would
// otherwise place a region past it; the buffer range then drops the stores).
__device__ inline int64_t ds_region(const BwdParams& p, int s, int h, int lq, int lk,
                                    int* bh_bytes) {
  const int nq = ds_nq32_of(lq), nk = ds_nk32_of(lk);
  const int64_t first = p.ds_prefix ? p.ds_prefix[s] : (int64_t)s * p.hq * nq * nk;
  const int64_t off = (first + (int64_t)h * nq * nk) * 2048;
  const int64_t room = p.ds_bytes - off;
  const int64_t size = (int64_t)nq * nk * 2048;
  // wave-uniform by construction (the tile is); made explicit for SGPRs
  *bh_bytes = __builtin_amdgcn_readfirstlane(room <= 0 ? 0 : static_cast<int>(size < room ? size : room));
  const int64_t r = room <= 0 ? 0 : off;
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(r));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(r >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Tile sizes (rows of the query block and keys of the key block) per head dim.
#ifndef ATTN71_FWD_NW
#define ATTN71_FWD_NW 8
#endif
#ifndef ATTN71_FWD_QB
#define ATTN71_FWD_QB 1
#endif
#ifndef ATTN71_FWD_BN
#define ATTN71_FWD_BN 128
#endif
template <int D> struct FwdCfg {
  static constexpr int NW = (D <= 128) ? ATTN71_FWD_NW : 4; // wavefronts per workgroup
  static constexpr int QB = (D <= 128) ? ATTN71_FWD_QB : 1; // 32-row query blocks per wave
  static constexpr int BM = NW * 32 * QB;
  static constexpr int BN = (D == 64) ? 128 : (D == 256 ? 64 : ATTN71_FWD_BN);  // keys per tile
};
template <int D> struct BwdCfg {
  static constexpr int BN = 128;                  // keys per workgroup (32 per wave)
  static constexpr int BM = (D <= 128) ? 64 : 32; // queries per inner step
};

template <int D> struct DqCfg {
  static constexpr int NW = (D <= 128) ? 8 : 4;   // wavefronts, 32 query rows each
  static constexpr int BM = NW * 32;
  static constexpr int BN = (D <= 128) ? 64 : 32; // keys per tile
};
inline int dq_block_m(int d) { return d <= 128 ? DqCfg<128>::BM : DqCfg<256>::BM; }

template <int D> struct DqDsCfg {
  static constexpr int NW = 8;                    // wavefronts, 32 query rows each
  static constexpr int BM = NW * 32;
  static constexpr int BN = (D == 64) ? 64 : 32;  // keys per tile (a K tile covers 8 KiB at least)
  static constexpr int NSD = (D == 64) ? 4 : (D == 128 ? 8 : 6);  // dS ring depth (K ring: 3)
};

template <int D> struct DkdvCfg {
  static constexpr int KB = (D <= 128) ? 2 : 1;   // 32-key blocks per wavefront
  static constexpr int BN = 4 * 32 * KB;          // keys per workgroup (four wavefronts)
  static constexpr int BM = (D == 64) ? 64 : 32;  // queries per step
};
inline int dkdv_block_n(int d) { return d <= 128 ? DkdvCfg<128>::BN : DkdvCfg<256>::BN; }

inline int fwd_block_m(int d) {
  return d == 64 ? FwdCfg<64>::BM : d == 128 ? FwdCfg<128>::BM : FwdCfg<256>::BM;
}
inline int bwd_block_n(int) { return 128; }
inline int bwd_block_m(int d) { return d <= 128 ? 64 : 32; }

// Workgroups of `kernel` (block of `threads`) that fit on one CU at once.
template <typename K>
int resident_per_cu(K kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1)
    n = 1;
  return n;
}
// Grid of a persistent launch over `ntiles` tiles: every resident slot
// (resident <= 0: a one-shot grid of ntiles), never fewer than min(ntiles, nx)
// so that every XCD residue class of tiles has a workgroup.
inline int persistent_grid(int ntiles, int resident, int nx) {
  if (resident <= 0 || resident >= ntiles) return ntiles;
  const int lo = ntiles < nx ? ntiles : nx;
  return resident < lo ? lo : resident;
}

// Launchers. `cus` is the device's CU count for persistent launches, or 0 for
// a one-shot grid of one workgroup per tile (p.ntiles).
hipError_t launch_fwd(const FwdParams& p, int d, int cus, int exp_emulation, bool pingpong,
                      hipStream_t stream);
hipError_t launch_bwd_pre(const BwdParams& p, int d, hipStream_t stream);
// fused = true: dQ accumulated with fp32 atomics (or the deterministic
// semaphore chain) inside the dK/dV kernel; false: dK/dV only.
hipError_t launch_bwd_main(const BwdParams& p, int d, int grid, bool fused, hipStream_t stream);
// dK, dV only: one workgroup per DkdvCfg<d>::BN keys (see bwd_dkdv.hip).
hipError_t launch_bwd_dkdv(const BwdParams& p, int d, int cus, hipStream_t stream);
// dQ without atomics: one workgroup per query block (see bwd_dq.hip).
hipError_t launch_bwd_dq(const BwdParams& p, int d, int cus, hipStream_t stream);
// dQ = alpha dS K from the dS the dK/dV kernel stored (p.ds; see bwd_dq_ds.hip).
hipError_t launch_bwd_dq_ds(const BwdParams& p, int d, int cus, hipStream_t stream);
hipError_t launch_bwd_post(const BwdParams& p, int d, hipStream_t stream);
// Varlen pre-pass: order[] = sequences by decreasing length of key_cu (ties
// by index), tile_prefix[vs] = first tile of virtual sequence vs with
// cdiv(len of count_cu, blk) * heads tiles each, and (optional) mb_prefix[s]
// = first query block of actual sequence s with cdiv(len of q_cu, mb_blk);
// clears *queue (optional) for the tile tickets of the launch that follows.
// Optional ds_prefix[s] = first stored-dS sub-tile of sequence s (lengths
// from q_cu and count_cu, ds_heads query heads each; see ds_region).
hipError_t launch_varlen_schedule(const int* key_cu, const int* count_cu, const int* q_cu,
                                  int nseq, int heads, int blk, int* order, int* tile_prefix,
                                  int* mb_prefix, int mb_blk, unsigned* queue,
                                  int64_t* ds_prefix, int ds_heads, hipStream_t stream);

}  // namespace attn71
