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
  // Stored dS (null: the dQ kernel recomputes S and dP): per (sequence,
  // query head) a region of 32-query x 32-key bf16 sub-tiles, 2 KiB each, in
  // the register order of the dK/dV kernel, holding only the sub-tiles that
  // kernel writes (DsGeom below); the regions of the heads of a sequence follow
  // each other, sequences in order.
  char* ds;
  const int64_t* ds_prefix;  // varlen: first sub-tile of each sequence (null: fixed length)
  int64_t ds_bytes;          // size of the dS area (every range is clamped to it)
};

// Stored-dS geometry of one (sequence, query head) with lq queries and lk
// keys. Sub-row r holds queries 32r .. 32r+31 (rows = 2 ceil(lq / 64): whole
// dK/dV steps of up to 64 queries); it stores sub-columns 0 .. width(r) - 1,
// 32 keys each. Widths are whole key blocks of 256 keys (the dK/dV workgroup)
// and constant over groups of 8 sub-rows (256 queries): group G stores the
// key blocks that reach into it, all kb of them without a causal mask, and
// blocks [0, G + c) with c = 1 + ceil((lk - lq) / 256) under the bottom-right
// causal diagonal (key block n writes the rows from its first visible one on,
// and 256 n - (lk - lq) >= 256 (G + 1) keeps it out of group G). A row's
// sub-tiles are contiguous; rows follow each other.
struct DsGeom {
  int rows;       // stored sub-rows
  int kb;         // key blocks of 256 keys
  int c;          // causal: group G holds min(max(G + c, 0), kb) blocks
  int causal;
  int64_t p0;     // causal: ds_psum(max(c, 0))
};

__host__ __device__ inline int64_t ds_clampi(int64_t a, int64_t lo, int64_t hi) {
  return a < lo ? lo : (a > hi ? hi : a);
}
// sum over a = 0 .. n-1 of min(a, kb) (n >= 0)
__host__ __device__ inline int64_t ds_psum(int64_t n, int64_t kb) {
  const int64_t n1 = n < kb + 1 ? n : kb + 1;
  return n1 * (n1 - 1) / 2 + (n - n1) * kb;
}
__host__ __device__ inline DsGeom ds_geom(int lq, int lk, bool causal) {
  DsGeom g;
  g.rows = (lq + 63) / 64 * 2;
  g.kb = (lk + 255) / 256;
  g.causal = causal ? 1 : 0;
  const int shift = lk - lq;
  // ceil(shift / 256) for either sign
  const int cdv = shift >= 0 ? (shift + 255) / 256 : -((-shift) / 256);
  g.c = 1 + cdv;
  g.p0 = causal ? ds_psum(g.c > 0 ? g.c : 0, g.kb) : 0;
  return g;
}
// key blocks (of 256) stored for the rows of group G
__host__ __device__ inline int ds_group_blocks(const DsGeom& g, int G) {
  return g.causal ? (int)ds_clampi((int64_t)G + g.c, 0, g.kb) : g.kb;
}
// sub-tiles stored in sub-row r
__host__ __device__ inline int ds_width(const DsGeom& g, int r) { return 8 * ds_group_blocks(g, r >> 3); }
// sub-tiles stored before sub-row r (0 <= r <= rows)
__host__ __device__ inline int64_t ds_row_start(const DsGeom& g, int r) {
  if (!g.causal) return (int64_t)r * 8 * g.kb;
  const int G = r >> 3;
  const int64_t a = (int64_t)G + g.c;
  const int64_t full = ds_psum(a > 0 ? a : 0, g.kb) - g.p0;   // blocks of groups 0 .. G-1
  return 64 * full + (int64_t)(r - 8 * G) * 8 * ds_group_blocks(g, G);
}
// sub-tiles of the whole region
__host__ __device__ inline int64_t ds_region_tiles(const DsGeom& g) { return ds_row_start(g, g.rows); }

// Byte offset from p.ds of sub-row r of the region of (sequence s, query head
// h) and, in *range, the bytes of the nr rows from there that lie inside the
// dS area (a region past the area, from packed lengths beyond the maximum the
// caller declared, gets range 0: its stores are dropped and its reads give
// zero). Rows past the region get range 0 too. Wave-uniform.
__device__ inline int64_t ds_rows_at(const BwdParams& p, const DsGeom& g, int s, int h, int r,
                                     int nr, int* range) {
  const int64_t reg = ds_region_tiles(g);
  const int64_t first = p.ds_prefix ? p.ds_prefix[s] : (int64_t)s * p.hq * reg;
  const int64_t off = (first + (int64_t)h * reg + ds_row_start(g, r)) * 2048;
  int64_t n = r < g.rows ? (ds_row_start(g, r + nr < g.rows ? r + nr : g.rows) - ds_row_start(g, r)) * 2048 : 0;
  const int64_t room = p.ds_bytes - off;
  if (n > room) n = room;
  *range = __builtin_amdgcn_readfirstlane(n <= 0 ? 0 : static_cast<int>(n > 0x7fffffffLL ? 0x7fffffffLL : n));
  const int64_t o = n <= 0 ? 0 : off;
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(o));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(o >> 32));
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
hipError_t launch_fwd(const FwdParams& p, int d, int cus, int exp_emulation, hipStream_t stream);
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
// from q_cu and count_cu, ds_heads query heads each; see DsGeom).
hipError_t launch_varlen_schedule(const int* key_cu, const int* count_cu, const int* q_cu,
                                  int nseq, int heads, int blk, int* order, int* tile_prefix,
                                  int* mb_prefix, int mb_blk, unsigned* queue,
                                  int64_t* ds_prefix, int ds_heads, int causal,
                                  hipStream_t stream);

}  // namespace attn71
