// C ABI of the attention library: validation, workspace layout, dispatch.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing (and the argument checks run without a GPU).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "attn71.h"
#include "kernels.hpp"
#include "schedule.hpp"

using namespace attn71;

namespace {

constexpr int kNxcd = 8;                        // MI355X: 8 XCDs of 32 CUs
constexpr int64_t kL2Bytes = 4ll << 20;         // L2 per XCD
constexpr int64_t kMaxExtent = (1ll << 31) - 1; // 32-bit buffer offsets
constexpr size_t kAlign = 256;

// Options of one call with defaults resolved (attn_options; all-zero = defaults).
struct Opts {
  int bwd_design;     // ATTN_BWD_* as requested (AUTO resolved by bwd_design_of)
  bool natural;       // plain tile order
  bool persistent;    // resident workgroups loop over the tiles
  int exp_emulation;  // FMA-path exponentials of every 8
  float tau;          // rescale threshold, log2 units
  int spin_limit;
  int64_t ds_budget;
};
Opts opts_of(const attn_params* p) {
  const attn_options& o = p->opt;
  Opts r;
  r.bwd_design = o.bwd_design;
  r.natural = o.tile_order != 0;
  r.persistent = o.one_shot_grid == 0;
  r.exp_emulation = o.exp_emulation;
  r.tau = o.tau == 0.0f ? kTau : (o.tau < 0.0f ? 0.0f : o.tau);
  r.spin_limit = o.spin_limit > 0 ? o.spin_limit : (1 << 26);
  r.ds_budget = o.ds_budget > 0 ? o.ds_budget : ATTN_DS_BUDGET_DEFAULT;
  return r;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------- validation
// Bytes of a block-mask buffer: the span of the last (batch, head) block
// table plus the strides, rounded up to whole 4-byte words (the kernels read
// the mask a word at a time, and a word that ends past the buffer range reads
// as zero).
int64_t mask_bytes(const attn_params* p) {
  const int64_t nqb = cdiv(p->seqlen_q, kMaskBlock), nkb = cdiv(p->seqlen_k, kMaskBlock);
  if (p->batch <= 0 || nqb * nkb == 0) return 0;
  const int64_t span = (int64_t)(p->batch - 1) * p->block_mask_stride_b +
                       (int64_t)(p->num_heads_q - 1) * p->block_mask_stride_h + nqb * nkb;
  return (span + 3) / 4 * 4;
}
MaskView mask_view(const attn_params* p) {
  MaskView m;
  std::memset(&m, 0, sizeof(m));
  if (!p->block_mask) return m;
  m.mask = p->block_mask;
  m.sb = p->block_mask_stride_b;
  m.sh = p->block_mask_stride_h;
  m.nkb = cdiv(p->seqlen_k, kMaskBlock);
  m.range = static_cast<int>(mask_bytes(p));
  return m;
}

attn_status check_params(const attn_params* p, bool varlen) {
  if (!p) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256) return ATTN_ERR_UNSUPPORTED;
  if (p->batch < 0 || p->seqlen_q < 0 || p->seqlen_k < 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->num_heads_q < 1 || p->num_heads_kv < 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->num_heads_q % p->num_heads_kv) return ATTN_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(p->softmax_scale) || !(p->softmax_scale > 0.0f)) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->causal != 0 && p->causal != 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->deterministic != 0 && p->deterministic != 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (varlen && (p->total_q < 0 || p->total_k < 0)) return ATTN_ERR_INVALID_ARGUMENT;
  const attn_options& o = p->opt;
  if (o.bwd_design < ATTN_BWD_AUTO || o.bwd_design > ATTN_BWD_FUSED_DQ) return ATTN_ERR_INVALID_ARGUMENT;
  if ((o.tile_order != 0 && o.tile_order != 1) || (o.one_shot_grid != 0 && o.one_shot_grid != 1))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (o.exp_emulation != 0 && o.exp_emulation != 1 && o.exp_emulation != 2 && o.exp_emulation != 4)
    return ATTN_ERR_INVALID_ARGUMENT;
  if (!(o.tau == 0.0f || o.tau == -1.0f || (o.tau > 0.0f && o.tau <= 64.0f)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (o.spin_limit < 0 || o.ds_budget < 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (o.reserved != 0 || o.head_split < 0 ||
      (o.head_split > 1 && ((p->num_heads_q / p->num_heads_kv) % o.head_split != 0 ||
                            (o.bwd_design == ATTN_BWD_FUSED_DQ && !fused_in_dkdv(p->head_dim)))))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (p->block_mask) {
    if (p->block_mask_stride_b < 0 || p->block_mask_stride_h < 0 ||
        (reinterpret_cast<uintptr_t>(p->block_mask) & 3u))
      return ATTN_ERR_INVALID_ARGUMENT;
    if (varlen || o.exp_emulation != 0 || mask_bytes(p) > kMaxExtent ||
        cdiv(p->seqlen_k, 64) > kMaxMaskTiles)   // the kernels' visible-tile lists
      return ATTN_ERR_UNSUPPORTED;
  }
  // one (sequence, head) slab must stay within 32-bit byte offsets
  const int64_t d = p->head_dim;
  const int64_t ext_q = (int64_t)p->seqlen_q * p->num_heads_q * d * 4;  // fp32 dQ accumulator
  const int64_t ext_k = (int64_t)p->seqlen_k * p->num_heads_kv * d * 2;
  if (ext_q > kMaxExtent || ext_k > kMaxExtent) return ATTN_ERR_UNSUPPORTED;
  const int64_t rows_q = varlen ? p->total_q : (int64_t)p->batch * p->seqlen_q;
  const int64_t rows_k = varlen ? p->total_k : (int64_t)p->batch * p->seqlen_k;
  // grids stay below 2^31 workgroups and row indices in int32
  if (rows_q * p->num_heads_q > (1ll << 30) || rows_k > (1ll << 30)) return ATTN_ERR_UNSUPPORTED;
  // key-block tiles (128-key blocks bound every backward design) times the
  // largest head split (the group size) within int32
  const int64_t kblocks = varlen ? rows_k / 128 + 1 + p->batch
                                 : (int64_t)p->batch * ((p->seqlen_k + 127) / 128);
  if (kblocks * p->num_heads_q > (1ll << 30)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

int64_t rows_q_of(const attn_params* p, bool varlen) {
  return varlen ? p->total_q : (int64_t)p->batch * p->seqlen_q;
}

// ------------------------------------------------------------ workspace maps
// Varlen schedule tables of one kernel (see SchedSet): offsets in a buffer.
enum SetKind { kSetFwd = 0, kSetDkdv = 1, kSetFused = 2, kSetDq = 3, kSetDqDs = 4, kNumSets = 5 };
struct SetMap {
  size_t order = 0, tile_prefix = 0, mb_prefix = 0, ds_prefix = 0, key_tiles = 0, queue = 0;
  bool mb = false, ds = false;
  int key_cap = 0;        // entries of the key-tile list (0: none)
};
// The key-tile list (one longest-first order of all key blocks) of the
// key-block kernels that run in the dK/dV kernel: entries bounded by
// total_k / block + batch; ranking costs entries x batch steps of one
// workgroup, so only up to 2^17 of them.
int key_list_cap(const attn_params* p, int kind) {
  const int d = p->head_dim;
  if (kind != kSetDkdv && !(kind == kSetFused && fused_in_dkdv(d))) return 0;
  const int64_t cap = (int64_t)p->total_k / dkdv_block_n(d) + 1 + p->batch;
  return cap * p->batch <= (1ll << 17) ? (int)cap : 0;
}
size_t map_set(size_t off, const attn_params* p, int kind, SetMap* m) {
  const int64_t nseq = p->batch;
  m->mb = kind == kSetDkdv || kind == kSetFused;
  m->ds = kind == kSetDkdv;
  m->key_cap = key_list_cap(p, kind);
  m->order = off; off = align_up(off + sizeof(int) * (size_t)nseq);
  m->tile_prefix = off; off = align_up(off + sizeof(int) * ((size_t)nseq + 1));
  if (m->mb) { m->mb_prefix = off; off = align_up(off + sizeof(int) * ((size_t)nseq + 1)); }
  if (m->ds) { m->ds_prefix = off; off = align_up(off + sizeof(int64_t) * ((size_t)nseq + 1)); }
  if (m->key_cap) {
    m->key_tiles = off;
    off = align_up(off + 2 * sizeof(int) * ((size_t)m->key_cap + 1));
  }
  m->queue = off; off = align_up(off + sizeof(unsigned));
  return off;
}

struct FwdWs {
  SetMap set;
  size_t total = 0;
};
FwdWs fwd_ws(const attn_params* p, bool varlen) {
  FwdWs w;
  if (varlen && !p->varlen_plan) w.total = map_set(0, p, kSetFwd, &w.set);
  return w;
}

// A varlen plan: the tables of all five kernels.
struct PlanMap {
  SetMap set[kNumSets];
  size_t total = 0;
};
PlanMap plan_map(const attn_params* p) {
  PlanMap m;
  size_t off = 0;
  for (int k = 0; k < kNumSets; ++k) off = map_set(off, p, k, &m.set[k]);
  m.total = off;
  return m;
}

struct BwdWs {
  size_t dsum = 0, lse2 = 0, dq_acc = 0, sem = 0, misc = 0, ds = 0, part = 0;
  int split = 1;          // query-head parts per KV group (dK / dV partials when > 1)
  SetMap main, dq;        // varlen tables of the key-block and dQ kernels (no plan)
  bool tables = false;
  size_t total = 0;
  int64_t n_sem = 0;
  int design = ATTN_BWD_RECOMPUTE;
};
// schedule-table kinds of a backward design
int main_kind(int design) { return design == ATTN_BWD_FUSED_DQ ? kSetFused : kSetDkdv; }
int dq_kind(int design) { return design == ATTN_BWD_STORED_DS ? kSetDqDs : kSetDq; }
// Bytes of the stored-dS area: fixed length, B * Hq regions of the visible
// sub-tiles (DsGeom); packed lengths, a bound from the totals and the longest
// key length, 2 (ceil(total_q / 64) + batch) sub-rows of at most
// 8 ceil(seqlen_k / 256) sub-tiles per query head (the exact regions are laid
// out on the device by the varlen schedule pass).
int64_t ds_area_bytes(const attn_params* p, bool varlen) {
  if (varlen)
    return (int64_t)p->num_heads_q * 2 * ((int64_t)cdiv(p->total_q, 64) + p->batch) *
           (8ll * cdiv(p->seqlen_k, 256)) * 2048;
  const DsGeom g = ds_geom(p->seqlen_q, p->seqlen_k, p->causal != 0);
  return (int64_t)p->batch * p->num_heads_q * ds_region_tiles(g) * 2048;
}
// The backward design of a call (ATTN_BWD_AUTO resolved), -1 if the request
// cannot be met (stored dS over the budget). Automatic: stored dS at
// head_dim 128 and 256, where it measured 5 % and 11 % faster per fwd+bwd
// step than recomputing S and dP in the dQ kernel; at 64 the dK/dV kernel's
// extra writes cost more than the dQ kernel saves.
int bwd_design_of(const attn_params* p, bool varlen) {
  const Opts o = opts_of(p);
  if (o.bwd_design == ATTN_BWD_FUSED_DQ || o.bwd_design == ATTN_BWD_RECOMPUTE) return o.bwd_design;
  // stored dS needs the whole dS area within the budget (and no block mask)
  const bool fits = ds_area_bytes(p, varlen) <= o.ds_budget && !p->block_mask &&
                    ds_geom(p->seqlen_q, p->seqlen_k, p->causal != 0).rows < kDsMaxRows;
  if (o.bwd_design == ATTN_BWD_STORED_DS) return fits ? ATTN_BWD_STORED_DS : -1;
  return (p->head_dim >= 128 && fits) ? ATTN_BWD_STORED_DS : ATTN_BWD_RECOMPUTE;
}
int64_t bwd_mblocks(const attn_params* p, bool varlen) {
  const int bm = fused_block_m(p->head_dim);
  return varlen ? (int64_t)cdiv(p->total_q, bm) + p->batch
                : (int64_t)p->batch * cdiv(p->seqlen_q, bm);
}
// Key-block tiles of the backward before any head split: (sequence, KV
// head, block of fused_block_n or dkdv_block_n keys); for packed lengths the
// bound from the totals.
int bwd_base_tiles(const attn_params* p, bool varlen, bool fused) {
  const int bn = fused ? fused_block_n(p->head_dim) : dkdv_block_n(p->head_dim);
  if (varlen) return (cdiv(p->total_k, bn) + p->batch) * p->num_heads_kv;
  return p->batch * p->num_heads_kv * cdiv(p->seqlen_k, bn);
}
// Query-head parts per KV group (opt.head_split; automatic: the largest
// divisor of the group that keeps the tiles within ATTN_SPLIT_TARGET, when the
// unsplit tiles fall below it). The 128-key fused kernel (head_dim 256)
// walks whole groups.
int head_split_of(const attn_params* p, bool varlen, int design) {
  const int group = p->num_heads_q / p->num_heads_kv;
  const bool fused = design == ATTN_BWD_FUSED_DQ;
  if (fused && !fused_in_dkdv(p->head_dim)) return 1;
  const int req = p->opt.head_split;
  if (req >= 1) return req;
  const int64_t base = bwd_base_tiles(p, varlen, fused);
  int s = 1;
  for (int c = 2; c <= group; ++c)
    if (group % c == 0 && base * c <= ATTN_SPLIT_TARGET) s = c;
  return s;
}
int64_t rows_k_of(const attn_params* p, bool varlen) {
  return varlen ? p->total_k : (int64_t)p->batch * p->seqlen_k;
}

// Workspace regions (256-byte aligned): -D and LSE log2 e per (row, query
// head); the fp32 dQ accumulator and the semaphores only for the fused
// design; ticket / status / tile counters; the varlen schedule tables; the
// stored dS.
BwdWs bwd_ws(const attn_params* p, bool varlen) {
  BwdWs w;
  w.design = bwd_design_of(p, varlen);
  const bool fused = w.design == ATTN_BWD_FUSED_DQ;
  const int64_t rq = rows_q_of(p, varlen);
  size_t off = 0;
  w.dsum = off; off = align_up(off + sizeof(float) * (size_t)(rq * p->num_heads_q));
  w.lse2 = off; off = align_up(off + sizeof(float) * (size_t)(rq * p->num_heads_q));
  w.dq_acc = off;
  if (fused) off = align_up(off + sizeof(float) * (size_t)(rq * p->num_heads_q * p->head_dim));
  w.n_sem = fused && p->deterministic ? bwd_mblocks(p, varlen) * p->num_heads_q : 0;
  w.sem = off; off = align_up(off + sizeof(int) * (size_t)w.n_sem);
  w.misc = off; off = align_up(off + 64);
  w.split = w.design < 0 ? 1 : head_split_of(p, varlen, w.design);
  if (w.split > 1) {   // fp32 dK and dV partials, [part][row][KV head][d] each
    w.part = off;
    off = align_up(off + 2 * sizeof(float) * (size_t)w.split *
                             (size_t)(rows_k_of(p, varlen) * p->num_heads_kv * p->head_dim));
  }
  if (varlen && !p->varlen_plan && w.design > 0) {
    w.tables = true;
    off = map_set(off, p, main_kind(w.design), &w.main);
    if (!fused) off = map_set(off, p, dq_kind(w.design), &w.dq);
  }
  if (w.design == ATTN_BWD_STORED_DS) {
    w.ds = off;
    off = align_up(off + (size_t)ds_area_bytes(p, varlen));
  }
  w.total = off;
  return w;
}

// sections of batch-heads whose reused operands fit in one XCD's L2
int section_width(int64_t bytes_per_bh) {
  if (bytes_per_bh <= 0) return 1;
  const int64_t s = kL2Bytes / bytes_per_bh;
  return s < 1 ? 1 : (s > 64 ? 64 : (int)s);
}

int fwd_grid(const attn_params* p, bool varlen) {
  const int bm = fwd_block_m(p->head_dim);
  if (varlen) return (cdiv(p->total_q, bm) + p->batch) * p->num_heads_q;
  return p->batch * p->num_heads_q * cdiv(p->seqlen_q, bm);
}
int dq_grid(const attn_params* p, bool varlen) {
  const int bm = dq_block_m(p->head_dim);
  if (varlen) return (cdiv(p->total_q, bm) + p->batch) * p->num_heads_q;
  return p->batch * p->num_heads_q * cdiv(p->seqlen_q, bm);
}
int bwd_grid(const attn_params* p, bool varlen, bool fused, int split) {
  return bwd_base_tiles(p, varlen, fused) * split;
}

// ----------------------------------------------------------------- device
std::mutex g_dev_mu;
int g_dev_ok[64];  // 0 unknown, 1 gfx950, 2 other
int g_dev_cus[64]; // compute units per device

attn_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev < 0 || dev >= 64) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_HIP;
    g_dev_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_cus[dev] = prop.multiProcessorCount;
  }
  return g_dev_ok[dev] == 1 ? ATTN_OK : ATTN_ERR_UNSUPPORTED;
}

// CU count for persistent launches of the current device (after
// check_device), or 0 when the call asks for one workgroup per tile.
int launch_cus(bool persistent) {
  if (!persistent) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  return g_dev_cus[dev] > 0 ? g_dev_cus[dev] : 0;
}

SeqView make_sv(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k) {
  SeqView sv;
  sv.cu_q = cu_q;
  sv.cu_k = cu_k;
  sv.batch = p->batch;
  sv.seqlen_q = p->seqlen_q;
  sv.seqlen_k = p->seqlen_k;
  sv.total_q = cu_q ? p->total_q : p->batch * p->seqlen_q;
  return sv;
}

// Schedule-table descriptor of one kernel's varlen tables at `m` in `base`.
// Query-block kernels (forward, dQ) sort the sequences by key length and
// count query blocks; key-block kernels sort by query length and count key
// blocks.
SchedSet make_set(const attn_params* p, int kind, const int32_t* cu_q, const int32_t* cu_k,
                  char* base, const SetMap& m) {
  SchedSet s;
  std::memset(&s, 0, sizeof(s));
  const int d = p->head_dim;
  const bool qblocks = kind == kSetFwd || kind == kSetDq || kind == kSetDqDs;
  s.key_cu = qblocks ? cu_k : cu_q;
  s.count_cu = qblocks ? cu_q : cu_k;
  s.heads = qblocks ? p->num_heads_q : p->num_heads_kv;
  s.blk = kind == kSetFwd ? fwd_block_m(d)
        : kind == kSetDkdv ? dkdv_block_n(d)
        : kind == kSetFused ? fused_block_n(d)
        : kind == kSetDq ? dq_block_m(d) : DqDsCfg<128>::BM;
  s.order = reinterpret_cast<int*>(base + m.order);
  s.tile_prefix = reinterpret_cast<int*>(base + m.tile_prefix);
  s.mb_prefix = m.mb ? reinterpret_cast<int*>(base + m.mb_prefix) : nullptr;
  s.mb_blk = fused_block_m(d);
  if (m.key_cap) {
    s.key_tiles = reinterpret_cast<int*>(base + m.key_tiles);
    s.key_cap = m.key_cap;
    s.rank_bm = d == 64 ? DkdvCfg<64>::BM : DkdvCfg<128>::BM;   // query rows per dK/dV step
  }
  s.queue = reinterpret_cast<unsigned*>(base + m.queue);
  s.ds_prefix = m.ds ? reinterpret_cast<int64_t*>(base + m.ds_prefix) : nullptr;
  s.ds_heads = p->num_heads_q;
  s.causal = p->causal;
  s.ds_tiles = ds_area_bytes(p, true) / 2048;
  return s;
}

// A plan passed with the parameters must have been built for them.
attn_status check_plan(const attn_params* p, bool varlen) {
  const attn_varlen_plan* pl = p->varlen_plan;
  if (!pl) return ATTN_OK;
  if (!varlen || !pl->data || pl->bytes < plan_map(p).total) return ATTN_ERR_INVALID_ARGUMENT;
  if (pl->batch != p->batch || pl->seqlen_q != p->seqlen_q || pl->seqlen_k != p->seqlen_k ||
      pl->total_q != p->total_q || pl->total_k != p->total_k ||
      pl->num_heads_q != p->num_heads_q || pl->num_heads_kv != p->num_heads_kv ||
      pl->head_dim != p->head_dim || pl->causal != p->causal)
    return ATTN_ERR_INVALID_ARGUMENT;
  return ATTN_OK;
}

attn_status fwd_impl(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k,
                     const void* q, const void* k, const void* v, void* o, float* lse,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  const bool varlen = cu_q != nullptr;
  attn_status st = check_params(p, varlen);
  if (st != ATTN_OK) return st;
  if (varlen && !cu_k) return ATTN_ERR_INVALID_ARGUMENT;
  // a tensor with no elements may be a null pointer (no kernel touches it)
  const bool has_q = rows_q_of(p, varlen) > 0, has_k = rows_k_of(p, varlen) > 0;
  if (has_q && (!q || !o || (has_k && (!k || !v)))) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_INVALID_ARGUMENT;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_INVALID_ARGUMENT;
  st = check_plan(p, varlen);
  if (st != ATTN_OK) return st;
  const FwdWs wl = fwd_ws(p, varlen);
  if (ws_bytes < wl.total) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (wl.total && !ws) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->batch == 0 || rows_q_of(p, varlen) == 0) return ATTN_OK;
  st = check_device();
  if (st != ATTN_OK) return st;

  const int d = p->head_dim;
  FwdParams fp;
  fp.q = q; fp.k = k; fp.v = v; fp.o = o; fp.lse = lse;
  fp.sv = make_sv(p, cu_q, cu_k);
  fp.order = nullptr; fp.tile_prefix = nullptr; fp.queue = nullptr;
  fp.hq = p->num_heads_q; fp.hkv = p->num_heads_kv; fp.group = p->num_heads_q / p->num_heads_kv;
  const int bm = fwd_block_m(d);
  fp.nm = cdiv(p->seqlen_q, bm);
  fp.sec = section_width(2ll * p->seqlen_k * d * 2);
  fp.nxcd = kNxcd;
  const Opts op = opts_of(p);
  fp.natural = op.natural ? 1 : 0;
  fp.ntiles = fwd_grid(p, varlen);
  fp.causal = p->causal;
  fp.alpha = p->softmax_scale;
  fp.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  fp.tau = op.tau;
  fp.mask = mask_view(p);
  const int pcus = launch_cus(op.persistent);
  if (varlen) {
    // the tables from a plan, or from a schedule pass into the workspace
    char* tb = static_cast<char*>(p->varlen_plan ? p->varlen_plan->data : ws);
    const SetMap m = p->varlen_plan ? plan_map(p).set[kSetFwd] : wl.set;
    const SchedSet s = make_set(p, kSetFwd, cu_q, cu_k, tb, m);
    if (!p->varlen_plan) {
      SchedArgs a;
      std::memset(&a, 0, sizeof(a));
      a.q_cu = cu_q;
      a.nseq = p->batch;
      a.nsets = 1;
      a.set[0] = s;
      if (launch_varlen_schedule(a, stream) != hipSuccess) return ATTN_ERR_HIP;
    }
    fp.order = s.order;
    fp.tile_prefix = s.tile_prefix;
    fp.queue = pcus ? s.queue : nullptr;
  }
  // the FMA-path exp2 issues from the same VALU port as v_exp_f32 here, and
  // with the hand-scheduled forward step every share E > 0 measured slower at
  // head_dim 64, 128 and 256, so the default is none
  if (launch_fwd(fp, d, pcus, op.exp_emulation, stream) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

// launch = false: validate only (no HIP call at all).
attn_status bwd_impl(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k, int phases,
                     const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                     hipStream_t stream, bool launch = true) {
  const bool varlen = cu_q != nullptr;
  attn_status st = check_params(p, varlen);
  if (st != ATTN_OK) return st;
  if (varlen && !cu_k) return ATTN_ERR_INVALID_ARGUMENT;
  if (phases <= 0 || phases > ATTN_BWD_ALL) return ATTN_ERR_INVALID_ARGUMENT;
  st = check_plan(p, varlen);
  if (st != ATTN_OK) return st;
  const BwdWs wl = bwd_ws(p, varlen);
  if (wl.design < 0) return ATTN_ERR_UNSUPPORTED;   // stored dS requested over the budget
  const bool fused_mode = wl.design == ATTN_BWD_FUSED_DQ;
  const bool pre = phases & ATTN_BWD_PREPROCESS, main = phases & ATTN_BWD_MAIN,
             post = (phases & ATTN_BWD_POSTPROCESS) && fused_mode,
             dqk = (phases & ATTN_BWD_DQ) && !fused_mode;
  // a tensor with no elements may be a null pointer: with no query rows no
  // kernel reads Q, O, dO or LSE or writes dQ, with no keys none reads K, V
  // or writes dK, dV
  const bool has_q = rows_q_of(p, varlen) > 0, has_k = rows_k_of(p, varlen) > 0;
  if (pre && has_q && (!o || !dout)) return ATTN_ERR_INVALID_ARGUMENT;
  if (pre && (!aligned16(o) || !aligned16(dout))) return ATTN_ERR_INVALID_ARGUMENT;
  if ((main || dqk) && ((has_q && (!q || !dout || !lse)) || (has_k && (!k || !v))))
    return ATTN_ERR_INVALID_ARGUMENT;
  if ((main || dqk) && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) ||
                        (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (main && ((has_k && (!dk || !dv)) || !aligned16(dk) || !aligned16(dv)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if ((post || dqk) && ((has_q && !dq) || !aligned16(dq))) return ATTN_ERR_INVALID_ARGUMENT;
  if (ws_bytes < wl.total) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (!ws) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->batch == 0 || (!has_q && !has_k) || !launch) return ATTN_OK;
  st = check_device();
  if (st != ATTN_OK) return st;

  const int d = p->head_dim;
  char* base = static_cast<char*>(ws);
  BwdParams bp;
  std::memset(&bp, 0, sizeof(bp));
  bp.q = q; bp.k = k; bp.v = v; bp.o = o; bp.dout = dout; bp.lse = lse;
  bp.dq = dq; bp.dk = dk; bp.dv = dv;
  bp.dsum = reinterpret_cast<float*>(base + wl.dsum);
  bp.lse2 = reinterpret_cast<float*>(base + wl.lse2);
  bp.dq_acc = reinterpret_cast<float*>(base + wl.dq_acc);
  bp.sem = reinterpret_cast<int*>(base + wl.sem);
  bp.ticket = reinterpret_cast<int*>(base + wl.misc);
  bp.status = reinterpret_cast<int*>(base + wl.misc + 4);
  bp.sv = make_sv(p, cu_q, cu_k);
  bp.hq = p->num_heads_q; bp.hkv = p->num_heads_kv; bp.group = p->num_heads_q / p->num_heads_kv;
  const Opts op = opts_of(p);
  const bool fused = fused_mode;
  const bool use_ds = wl.design == ATTN_BWD_STORED_DS;
  const int bn = fused ? fused_block_n(d) : dkdv_block_n(d), bm = fused_block_m(d);
  bp.nn = cdiv(p->seqlen_k, bn);
  bp.nm = cdiv(p->seqlen_q, bm);
  bp.hsplit = wl.split;
  bp.sec = section_width(2ll * (bp.group / wl.split) * p->seqlen_q * d * 2);
  bp.nxcd = kNxcd;
  bp.natural = op.natural ? 1 : 0;
  bp.ntiles = bwd_grid(p, varlen, fused, wl.split);
  bp.ntiles_dq = dq_grid(p, varlen);
  bp.causal = p->causal;
  bp.deterministic = p->deterministic;
  bp.alpha = p->softmax_scale;
  bp.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  bp.rows_q = rows_q_of(p, varlen);
  bp.n_sem = fused ? wl.n_sem : 0;
  bp.zero_acc = fused ? 1 : 0;
  bp.spin_limit = op.spin_limit;
  bp.mask = mask_view(p);
  if (wl.split > 1) {
    bp.dk_part = reinterpret_cast<float*>(base + wl.part);
    bp.dv_part = bp.dk_part + (size_t)wl.split * rows_k_of(p, varlen) * p->num_heads_kv * d;
    bp.rows_k = rows_k_of(p, varlen);
  }
  // fused design at head_dim 64 / 128: dQ inside the 256-key dK/dV kernel
  const bool fused_dkdv = fused && fused_in_dkdv(d);
  bp.dq_mode = fused_dkdv ? (p->deterministic ? 2 : 1) : 0;
  const int bmq = use_ds ? DqDsCfg<128>::BM : dq_block_m(d);
  bp.nm_dq = cdiv(p->seqlen_q, bmq);
  if (use_ds) {
    bp.ds = base + wl.ds;
    bp.ds_bytes = static_cast<int64_t>(wl.total - wl.ds);

    bp.ntiles_dq = varlen ? (cdiv(p->total_q, bmq) + p->batch) * p->num_heads_q
                          : p->batch * p->num_heads_q * bp.nm_dq;
  }
  bp.sec_dq = section_width(2ll * p->seqlen_k * d * 2);
  // Packed sequences of very different lengths make tiles too unequal for a
  // static walk (measured 19 % slower dK/dV on 16 sequences of 512..8192):
  // there the persistent workgroups draw tiles from device counters, which
  // the varlen schedule pass clears.
  const int pcus = launch_cus(op.persistent);
  SchedArgs sched;
  std::memset(&sched, 0, sizeof(sched));
  if (varlen) {
    // the tables from a plan, or from the schedule pass of PREPROCESS into the
    // workspace (one launch for the key-block and the dQ kernel's tables)
    char* tb = p->varlen_plan ? static_cast<char*>(p->varlen_plan->data) : base;
    const PlanMap pm = p->varlen_plan ? plan_map(p) : PlanMap();
    const SetMap mm = p->varlen_plan ? pm.set[main_kind(wl.design)] : wl.main;
    const SetMap dm = p->varlen_plan ? pm.set[dq_kind(wl.design)] : wl.dq;
    sched.q_cu = cu_q;
    sched.nseq = p->batch;
    sched.set[sched.nsets++] = make_set(p, main_kind(wl.design), cu_q, cu_k, tb, mm);
    if (!fused) sched.set[sched.nsets++] = make_set(p, dq_kind(wl.design), cu_q, cu_k, tb, dm);
    const SchedSet& ms = sched.set[0];
    bp.order = ms.order;
    bp.tile_prefix = ms.tile_prefix;
    bp.mb_prefix = ms.mb_prefix;
    bp.key_tiles = ms.key_tiles;
    bp.queue = pcus ? ms.queue : nullptr;
    if (use_ds) bp.ds_prefix = ms.ds_prefix;
    if (!fused) {
      const SchedSet& qs = sched.set[1];
      bp.order_dq = qs.order;
      bp.tile_prefix_dq = qs.tile_prefix;
      bp.queue_dq = pcus ? qs.queue : nullptr;
    }
    if (p->varlen_plan) sched.nsets = 0;   // computed when the plan was built
  }
  // The deterministic chain needs tiles started in the order of its turns:
  // workgroups draw them from the ticket word the preprocess clears
  if (bp.dq_mode == 2) bp.queue = reinterpret_cast<unsigned*>(bp.ticket);
  if (pre) {
    if (varlen && launch_varlen_schedule(sched, stream) != hipSuccess) return ATTN_ERR_HIP;
    if (launch_bwd_pre(bp, d, stream) != hipSuccess) return ATTN_ERR_HIP;
  }
  if (main) {
    const hipError_t e = fused && !fused_dkdv ? launch_bwd_main(bp, d, bp.ntiles, stream)
                                              : launch_bwd_dkdv(bp, d, pcus, stream);
    if (e != hipSuccess) return ATTN_ERR_HIP;
    if (wl.split > 1 && launch_bwd_dkdv_reduce(bp, d, stream) != hipSuccess) return ATTN_ERR_HIP;
  }
  if (dqk) {
    const hipError_t e = use_ds ? launch_bwd_dq_ds(bp, d, pcus, stream)
                                   : launch_bwd_dq(bp, d, pcus, stream);
    if (e != hipSuccess) return ATTN_ERR_HIP;
  }
  if (post && launch_bwd_post(bp, d, stream) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

// ------------------------------------------------ allocation-free backward
// Device scratch of attn_bwd_noalloc, for callers that cannot allocate
// (graph capture, serving loops, harnesses that forbid allocation): the
// recomputing backward's workspace (-D and LSE log2 e per (row, query head),
// the ticket / status words) lives in this static array, which every GPU the
// library runs on holds until the process ends. In host code the name is a
// stand-in, not a device address: kernels and copies use the address
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept in g_scratch.
__device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch[64];

attn_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev < 0 || dev >= 64) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return ATTN_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "OK";
    case ATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported";
    case ATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int attn_version(void) { return ATTN71_VERSION; }

size_t attn_fwd_workspace_size(const attn_params* p, int32_t varlen) {
  if (check_params(p, varlen != 0) != ATTN_OK) return (size_t)-1;
  return fwd_ws(p, varlen != 0).total;
}

size_t attn_bwd_workspace_size(const attn_params* p, int32_t varlen) {
  if (check_params(p, varlen != 0) != ATTN_OK) return (size_t)-1;
  const BwdWs w = bwd_ws(p, varlen != 0);
  return w.design < 0 ? (size_t)-1 : w.total;
}

size_t attn_varlen_plan_size(const attn_params* p) {
  if (check_params(p, true) != ATTN_OK) return (size_t)-1;
  return plan_map(p).total;
}

attn_status attn_varlen_plan_build(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k,
                                   void* data, size_t bytes, attn_varlen_plan* plan,
                                   hipStream_t stream) {
  attn_status st = check_params(p, true);
  if (st != ATTN_OK) return st;
  if (!cu_q || !cu_k || !data || !plan) return ATTN_ERR_INVALID_ARGUMENT;
  const PlanMap m = plan_map(p);
  if (bytes < m.total) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  plan->data = data;
  plan->bytes = bytes;
  plan->batch = p->batch;
  plan->seqlen_q = p->seqlen_q;
  plan->seqlen_k = p->seqlen_k;
  plan->total_q = p->total_q;
  plan->total_k = p->total_k;
  plan->num_heads_q = p->num_heads_q;
  plan->num_heads_kv = p->num_heads_kv;
  plan->head_dim = p->head_dim;
  plan->causal = p->causal;
  if (p->batch == 0) return ATTN_OK;
  st = check_device();
  if (st != ATTN_OK) return st;
  SchedArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q_cu = cu_q;
  a.nseq = p->batch;
  for (int k = 0; k < kNumSets; ++k)
    a.set[a.nsets++] = make_set(p, k, cu_q, cu_k, static_cast<char*>(data), m.set[k]);
  return launch_varlen_schedule(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int32_t attn_bwd_design(const attn_params* p, int32_t varlen) {
  if (check_params(p, varlen != 0) != ATTN_OK) return -1;
  return bwd_design_of(p, varlen != 0);
}

attn_status attn_fwd(const attn_params* p, const void* q, const void* k, const void* v, void* o,
                     float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fwd_impl(p, nullptr, nullptr, q, k, v, o, lse, ws, ws_bytes, stream);
}

attn_status attn_fwd_varlen(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k,
                            const void* q, const void* k, const void* v, void* o, float* lse,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!cu_q || !cu_k) return ATTN_ERR_INVALID_ARGUMENT;
  return fwd_impl(p, cu_q, cu_k, q, k, v, o, lse, ws, ws_bytes, stream);
}

attn_status attn_bwd(const attn_params* p, const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse, void* dq, void* dk,
                     void* dv, void* ws, size_t ws_bytes, hipStream_t stream) {
  return bwd_impl(p, nullptr, nullptr, ATTN_BWD_ALL, q, k, v, o, dout, lse, dq, dk, dv, ws,
                  ws_bytes, stream);
}

attn_status attn_bwd_noalloc(const attn_params* p, const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse, void* dq,
                             void* dk, void* dv, hipStream_t stream) {
  attn_status st = check_params(p, false);
  if (st != ATTN_OK) return st;
  if (p->opt.bwd_design != ATTN_BWD_AUTO && p->opt.bwd_design != ATTN_BWD_RECOMPUTE)
    return ATTN_ERR_UNSUPPORTED;
  attn_params pr = *p;
  pr.opt.bwd_design = ATTN_BWD_RECOMPUTE;
  // an automatic head split whose dK / dV partials do not fit runs unsplit
  if (pr.opt.head_split == 0 && bwd_ws(&pr, false).total > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
    pr.opt.head_split = 1;
  if (bwd_ws(&pr, false).total > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_UNSUPPORTED;
  // every argument is checked before the first HIP call (the scratch lookup)
  void* const placeholder = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  st = bwd_impl(&pr, nullptr, nullptr, ATTN_BWD_ALL, q, k, v, o, dout, lse, dq, dk, dv, placeholder,
                ATTN_NOALLOC_SCRATCH_BYTES, stream, /*launch=*/false);
  if (st != ATTN_OK || p->batch == 0) return st;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != ATTN_OK) return st;
  return bwd_impl(&pr, nullptr, nullptr, ATTN_BWD_ALL, q, k, v, o, dout, lse, dq, dk, dv, ws,
                  ATTN_NOALLOC_SCRATCH_BYTES, stream);
}

attn_status attn_bwd_varlen(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k,
                            const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!cu_q || !cu_k) return ATTN_ERR_INVALID_ARGUMENT;
  return bwd_impl(p, cu_q, cu_k, ATTN_BWD_ALL, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes,
                  stream);
}

attn_status attn_bwd_phases(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k,
                            int32_t phases, const void* q, const void* k, const void* v,
                            const void* o, const void* dout, const float* lse, void* dq,
                            void* dk, void* dv, void* ws, size_t ws_bytes, hipStream_t stream) {
  if ((cu_q == nullptr) != (cu_k == nullptr)) return ATTN_ERR_INVALID_ARGUMENT;
  return bwd_impl(p, cu_q, cu_k, phases, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, stream);
}

attn_status attn_bwd_status(const attn_params* p, int32_t varlen, const void* ws,
                            int32_t* status_out, hipStream_t stream) {
  if (!status_out || !ws) return ATTN_ERR_INVALID_ARGUMENT;
  attn_status st = check_params(p, varlen != 0);
  if (st != ATTN_OK) return st;
  const BwdWs wl = bwd_ws(p, varlen != 0);
  int32_t val = 0;
  if (hipMemcpyAsync(&val, static_cast<const char*>(ws) + wl.misc + 4, sizeof(int32_t),
                     hipMemcpyDeviceToHost, stream) != hipSuccess)
    return ATTN_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return ATTN_ERR_HIP;
  *status_out = val;
  return ATTN_OK;
}

attn_status attn_tile_order(const attn_params* p, int32_t which, int32_t* out, int64_t capacity,
                            int64_t* count) {
  if (!count || which < 0 || which > 3 || capacity < 0 || (capacity > 0 && !out))
    return ATTN_ERR_INVALID_ARGUMENT;
  attn_status st = check_params(p, false);
  if (st != ATTN_OK) return st;
  const int d = p->head_dim;
  if (which == 0 || which == 3) {
    const int nm = cdiv(p->seqlen_q, which == 0 ? fwd_block_m(d) : dq_block_m(d));
    const int sec = section_width(2ll * p->seqlen_k * d * 2);
    const int n = which == 0 ? fwd_grid(p, false) : dq_grid(p, false);
    *count = n;
    for (int i = 0; i < n && i < capacity; ++i) {
      const Tile t = fwd_tile_fixed(i, p->batch, p->num_heads_q, nm, sec, kNxcd,
                                    p->opt.tile_order != 0);
      out[3 * i] = t.seq; out[3 * i + 1] = t.head; out[3 * i + 2] = t.block;
    }
  } else {
    const bool fz = which == 2;   // 1: dK/dV kernel; 2: fused deterministic (ticket order)
    const int nn = cdiv(p->seqlen_k, fz ? fused_block_n(d) : dkdv_block_n(d));
    const int grp = p->num_heads_q / p->num_heads_kv;
    const int split = head_split_of(p, false, fz ? ATTN_BWD_FUSED_DQ : ATTN_BWD_RECOMPUTE);
    const int sec = section_width(2ll * (grp / split) * p->seqlen_q * d * 2);
    const int n = bwd_grid(p, false, fz, split);
    *count = n;
    for (int i = 0; i < n && i < capacity; ++i) {
      // with a head split the head is KV head * split + part
      const Tile t = bwd_tile_fixed(i, p->batch, p->num_heads_kv * split, nn, sec, which == 2,
                                    kNxcd, p->opt.tile_order != 0);
      out[3 * i] = t.seq; out[3 * i + 1] = t.head; out[3 * i + 2] = t.block;
    }
  }
  return ATTN_OK;
}

attn_status attn_varlen_key_order(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k,
                                  int32_t* out, int64_t capacity, int64_t* count) {
  if (!count || !cu_q || !cu_k || capacity < 0 || (capacity > 0 && !out))
    return ATTN_ERR_INVALID_ARGUMENT;
  *count = 0;
  attn_status st = check_params(p, true);
  if (st != ATTN_OK) return st;
  const int cap = key_list_cap(p, kSetDkdv);
  const int d = p->head_dim, bn = dkdv_block_n(d);
  const int bm = d == 64 ? DkdvCfg<64>::BM : DkdvCfg<128>::BM;
  std::vector<int> lq(p->batch), lk(p->batch);
  int nkb = 0;
  for (int s = 0; s < p->batch; ++s) {
    lq[s] = cu_q[s + 1] - cu_q[s];
    lk[s] = cu_k[s + 1] - cu_k[s];
    nkb += imax(0, cdiv(lk[s], bn));
  }
  *count = nkb;
  if (cap == 0 || nkb > cap) return ATTN_ERR_UNSUPPORTED;
  for (int e = 0; e < nkb; ++e) {
    int s, b;
    key_block_at(lk.data(), p->batch, bn, e, &s, &b);
    const int r = key_block_rank(lq.data(), lk.data(), p->batch, bm, bn, p->causal != 0, s, b);
    if (r < 0 || r >= nkb) return ATTN_ERR_INVALID_ARGUMENT;
    if (r < capacity) { out[2 * r] = s; out[2 * r + 1] = b; }
  }
  return ATTN_OK;
}

int32_t attn_bwd_head_split(const attn_params* p, int32_t varlen) {
  if (check_params(p, varlen != 0) != ATTN_OK) return -1;
  const int design = bwd_design_of(p, varlen != 0);
  return design < 0 ? -1 : head_split_of(p, varlen != 0, design);
}

int64_t attn_bwd_ds_subtile(const attn_params* p, int32_t row32, int32_t col32,
                            int64_t* region_tiles) {
  if (check_params(p, false) != ATTN_OK) return -1;
  const DsGeom g = ds_geom(p->seqlen_q, p->seqlen_k, p->causal != 0);
  if (region_tiles) *region_tiles = ds_region_tiles(g);
  return ds_subtile(g, row32, col32);
}

int32_t attn_persistent_tile(int32_t g, int32_t r, int32_t grid, int32_t ntiles, int32_t nx) {
  if (g < 0 || g >= grid || r < 0 || ntiles < 0 || nx < 1 || grid < (ntiles < nx ? ntiles : nx))
    return -1;
  return persistent_index(g, r, grid, ntiles, nx);
}

}  // extern "C"
