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

// Block-sparse mask (fixed length): byte (b, h, i, j) at
// b * sb + h * sh + i * nkb + j, one per 128 x 128 block of (query, key)
// pairs; zero hides the block. mask == null: no mask.
constexpr int kMaskBlock = 128;
// key tiles a masked forward or dQ workgroup lists (its visible ones): the
// host refuses masks over more than kMaxMaskTiles 64-key tiles
constexpr int kMaxMaskTiles = 4096;
// (query head, 128-row mask row) pairs a masked dK/dV workgroup lists (its
// visible ones); a workgroup with more pairs walks every step instead
constexpr int kMaxMaskRows = 2048;
struct MaskView {
  const uint8_t* mask;
  int64_t sb, sh;       // bytes between batches / query heads (0: shared)
  int nkb;              // entries per mask row: ceil(Sk / 128)
  int range;            // bytes of the mask buffer
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
  MaskView mask;
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
  const int* key_tiles;   // varlen, optional: a SchedSet key-tile list (used when its
                          // first word is set; else the per-sequence order)
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
  MaskView mask;
  char* ds;
  const int64_t* ds_prefix;  // varlen: first sub-tile of each sequence, -1 for a
                             // sequence whose regions do not fit the area (its
                             // stores are dropped); null: fixed length
  int64_t ds_bytes;          // size of the dS area
  // dQ inside the 256-key dK/dV kernel (fused design): 0 off, 1 fp32 atomics
  // into dq_acc, 2 the same in the deterministic order (sem, in turns of
  // four wavefront adds per key block)
  int dq_mode;
  // Head split (hsplit > 1): tile head t.head = KV head * hsplit + part (fixed
  // length) or ticket i = base tile * hsplit + part (packed lengths); part j
  // walks query heads j group/hsplit .. of the group and writes fp32 dK
  // (unscaled) and dV partials [part][row][KV head][d] of rows_k rows each,
  // which launch_bwd_dkdv_reduce adds in part order.
  int hsplit;
  float* dk_part;
  float* dv_part;
  int64_t rows_k;
};

// Stored-dS layout of one (sequence, query head) with lq queries and lk
// keys, key-block major. Sub-tiles are 32 queries x 32 keys of bf16 (2 KiB).
// The keys form kb = ceil(lk / 256) blocks of 256 (8 sub-columns: the dK/dV
// workgroup, or two of them at head_dim 256); block n keeps the sub-rows
// r0(n) .. rows - 1 (rows = 2 ceil(lq / 64): whole dK/dV steps of up to 64
// queries), 16 KiB per sub-row with its 8 sub-tiles in column order, and the
// blocks follow each other. r0(n) is where the dK/dV kernel's first step for
// the block begins: 0 without a causal mask; under the bottom-right diagonal
// (query i sees key j iff j <= i + lk - lq) the first 64-query step that sees
// key 256 n, r0(n) = min(rows, 2 max(0, 4n + f)) with f = floor((lq - lk) / 64).
// The dK/dV kernel then advances by a constant 16 KiB per step; the dQ
// kernel, which reads one sub-row across the blocks, moves to a new column
// base every 8 sub-tiles.
// A key-block column of 16 KiB per sub-row is addressed with 32-bit offsets.
constexpr int kDsMaxRows = (1 << 17) - 1;   // sub-rows: queries < 4194240
struct DsGeom {
  int rows;       // sub-rows of a block that starts at row 0
  int kb;         // key blocks
  int f;          // causal: r0(n) = min(rows, 2 max(0, 4n + f))
  int causal;
};

__host__ __device__ inline int64_t ds_floordiv(int64_t a, int64_t b) {
  return a >= 0 ? a / b : -((-a + b - 1) / b);
}
__host__ __device__ inline DsGeom ds_geom(int lq, int lk, bool causal) {
  DsGeom g;
  g.rows = (lq + 63) / 64 * 2;
  g.kb = (lk + 255) / 256;
  g.f = (int)ds_floordiv((int64_t)lq - lk, 64);
  g.causal = causal ? 1 : 0;
  return g;
}
// first stored sub-row of key block n
__host__ __device__ inline int ds_r0(const DsGeom& g, int n) {
  if (!g.causal) return 0;
  const int64_t a = 4ll * n + g.f;
  const int64_t r = a > 0 ? 2 * a : 0;
  return (int)(r < g.rows ? r : g.rows);
}
// sub-tiles of blocks 0 .. n-1 (0 <= n <= kb): 8 sum_j (rows - r0(j)). Under
// the causal mask r0(j) is 0 for j < j1 (4j + f <= 0), 8j + 2f for
// j1 <= j < j2 and rows from j2 on (8j + 2f >= rows).
__host__ __device__ inline int64_t ds_col_start(const DsGeom& g, int n) {
  if (!g.causal) return 8ll * n * g.rows;
  const int64_t j1 = ds_floordiv(-(int64_t)g.f, 4) + 1 > 0 ? ds_floordiv(-(int64_t)g.f, 4) + 1 : 0;
  int64_t j2 = ds_floordiv((int64_t)g.rows - 2ll * g.f + 7, 8);
  if (j2 < j1) j2 = j1;
  const int64_t a = j1 < n ? j1 : n, b = j2 < n ? j2 : n;
  int64_t r0sum = 8 * (b * (b - 1) / 2 - a * (a - 1) / 2) + 2ll * g.f * (b - a);
  if (n > j2) r0sum += (int64_t)g.rows * (n - j2);
  return 8 * ((int64_t)n * g.rows - r0sum);
}
// sub-tiles of the whole region
__host__ __device__ inline int64_t ds_region_tiles(const DsGeom& g) { return ds_col_start(g, g.kb); }
// sub-tile index of (sub-row r, sub-column k) in the region, -1 if not stored
__host__ __device__ inline int64_t ds_subtile(const DsGeom& g, int r, int k) {
  const int n = k >> 3;
  if (r < 0 || k < 0 || n >= g.kb || r >= g.rows || r < ds_r0(g, n)) return -1;
  return ds_col_start(g, n) + 8ll * (r - ds_r0(g, n)) + (k & 7);
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
// The fused design (dQ reduced across key blocks by atomics or the
// deterministic chain): at head_dim 64 and 128 inside the 256-key dK/dV
// kernel (one global reduction per 256 keys); at 256, whose Q / dO ring
// leaves no LDS for the K tile, in the 128-key kernel of bwd.hip.
inline bool fused_in_dkdv(int d) { return d <= 128; }
inline int fused_block_n(int d) { return fused_in_dkdv(d) ? dkdv_block_n(d) : BwdCfg<256>::BN; }
inline int fused_block_m(int d) {
  return d == 64 ? DkdvCfg<64>::BM : d == 128 ? DkdvCfg<128>::BM : BwdCfg<256>::BM;
}

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
// Fused design at head_dim 256: dK, dV and the dQ atomics (or the
// deterministic chain) in one 128-key kernel; one workgroup per tile.
hipError_t launch_bwd_main(const BwdParams& p, int d, int grid, hipStream_t stream);
// dK, dV: one workgroup per DkdvCfg<d>::BN keys (see bwd_dkdv.hip); with
// p.dq_mode set (head_dim 64, 128) also dQ into p.dq_acc.
hipError_t launch_bwd_dkdv(const BwdParams& p, int d, int cus, hipStream_t stream);
// dK = bf16(alpha sum of the dK partials), dV = bf16(sum of the dV
// partials), parts in order (p.hsplit > 1).
hipError_t launch_bwd_dkdv_reduce(const BwdParams& p, int d, hipStream_t stream);
// dQ without atomics: one workgroup per query block (see bwd_dq.hip).
hipError_t launch_bwd_dq(const BwdParams& p, int d, int cus, hipStream_t stream);
// dQ = alpha dS K from the dS the dK/dV kernel stored (p.ds; see bwd_dq_ds.hip).
hipError_t launch_bwd_dq_ds(const BwdParams& p, int d, int cus, hipStream_t stream);
hipError_t launch_bwd_post(const BwdParams& p, int d, hipStream_t stream);
// Varlen pre-pass tables. One set: order[] = sequences by decreasing length
// of key_cu (ties by index), tile_prefix[vs] = first tile of virtual sequence
// vs with cdiv(len of count_cu, blk) * heads tiles each; optional
// mb_prefix[s] = first query block of actual sequence s with
// cdiv(len of q_cu, mb_blk); optional ds_prefix[s] = first stored-dS
// sub-tile of sequence s (lengths from q_cu and count_cu, ds_heads query
// heads each; see DsGeom), or -1 when its regions would end past ds_tiles
// sub-tiles; clears *queue (optional) for the tile tickets of the launches
// that follow.
struct SchedSet {
  const int* key_cu;
  const int* count_cu;
  int heads, blk;
  int* order;
  int* tile_prefix;
  int* mb_prefix;
  int mb_blk;
  // optional (key-block kinds): key_tiles[0] = 1 when the list below is
  // written (0 when the blocks exceed key_cap), key_tiles[2 + 2 r], [3 + 2 r]
  // = (sequence, key block) of rank r in the longest-first order of all key
  // blocks (schedule.hpp: key_block_rank, steps of rank_bm query rows)
  int* key_tiles;
  int key_cap, rank_bm;
  unsigned* queue;
  int64_t* ds_prefix;
  int ds_heads, causal;
  int64_t ds_tiles;
};
constexpr int kMaxSchedSets = 5;
struct SchedArgs {
  const int* q_cu;
  int nseq, nsets;
  SchedSet set[kMaxSchedSets];
};
// One launch (a single workgroup) computes every set of `a`.
hipError_t launch_varlen_schedule(const SchedArgs& a, hipStream_t stream);

}  // namespace attn71
