// C ABI of the attention library: validation, workspace layout, dispatch.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing (and the argument checks run without a GPU).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

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
  // one (sequence, head) slab must stay within 32-bit byte offsets
  const int64_t d = p->head_dim;
  const int64_t ext_q = (int64_t)p->seqlen_q * p->num_heads_q * d * 4;  // fp32 dQ accumulator
  const int64_t ext_k = (int64_t)p->seqlen_k * p->num_heads_kv * d * 2;
  if (ext_q > kMaxExtent || ext_k > kMaxExtent) return ATTN_ERR_UNSUPPORTED;
  const int64_t rows_q = varlen ? p->total_q : (int64_t)p->batch * p->seqlen_q;
  const int64_t rows_k = varlen ? p->total_k : (int64_t)p->batch * p->seqlen_k;
  // grids stay below 2^31 workgroups and row indices in int32
  if (rows_q * p->num_heads_q > (1ll << 30) || rows_k > (1ll << 30)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

int64_t rows_q_of(const attn_params* p, bool varlen) {
  return varlen ? p->total_q : (int64_t)p->batch * p->seqlen_q;
}

// ------------------------------------------------------------ workspace maps
struct FwdWs {
  size_t order = 0, tile_prefix = 0, queue = 0, total = 0;
};
FwdWs fwd_ws(const attn_params* p, bool varlen) {
  FwdWs w;
  if (!varlen) return w;
  size_t off = 0;
  w.order = off; off = align_up(off + sizeof(int) * (size_t)p->batch);
  w.tile_prefix = off; off = align_up(off + sizeof(int) * ((size_t)p->batch + 1));
  w.queue = off; off = align_up(off + sizeof(unsigned));
  w.total = off;
  return w;
}

struct BwdWs {
  size_t dsum = 0, lse2 = 0, dq_acc = 0, sem = 0, misc = 0, order = 0, tile_prefix = 0, mb_prefix = 0;
  size_t order_dq = 0, tile_prefix_dq = 0, ds = 0, ds_prefix = 0;
  size_t total = 0;
  int64_t n_sem = 0;
  int design = ATTN_BWD_RECOMPUTE;
};
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
  const bool fits = ds_area_bytes(p, varlen) <= o.ds_budget;
  if (o.bwd_design == ATTN_BWD_STORED_DS) return fits ? ATTN_BWD_STORED_DS : -1;
  return (p->head_dim >= 128 && fits) ? ATTN_BWD_STORED_DS : ATTN_BWD_RECOMPUTE;
}
int64_t bwd_mblocks(const attn_params* p, bool varlen) {
  const int bm = bwd_block_m(p->head_dim);
  return varlen ? (int64_t)cdiv(p->total_q, bm) + p->batch
                : (int64_t)p->batch * cdiv(p->seqlen_q, bm);
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
  if (varlen) {
    w.order = off; off = align_up(off + sizeof(int) * (size_t)p->batch);
    w.tile_prefix = off; off = align_up(off + sizeof(int) * ((size_t)p->batch + 1));
    w.mb_prefix = off; off = align_up(off + sizeof(int) * ((size_t)p->batch + 1));
    w.order_dq = off; off = align_up(off + sizeof(int) * (size_t)p->batch);
    w.tile_prefix_dq = off; off = align_up(off + sizeof(int) * ((size_t)p->batch + 1));
  }
  if (w.design == ATTN_BWD_STORED_DS) {
    if (varlen) {
      w.ds_prefix = off;
      off = align_up(off + sizeof(int64_t) * ((size_t)p->batch + 1));
    }
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
int bwd_grid(const attn_params* p, bool varlen, bool fused) {
  const int bn = fused ? bwd_block_n(p->head_dim) : dkdv_block_n(p->head_dim);
  if (varlen) return (cdiv(p->total_k, bn) + p->batch) * p->num_heads_kv;
  return p->batch * p->num_heads_kv * cdiv(p->seqlen_k, bn);
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

attn_status fwd_impl(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k,
                     const void* q, const void* k, const void* v, void* o, float* lse,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  const bool varlen = cu_q != nullptr;
  attn_status st = check_params(p, varlen);
  if (st != ATTN_OK) return st;
  if (varlen && !cu_k) return ATTN_ERR_INVALID_ARGUMENT;
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_INVALID_ARGUMENT;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_INVALID_ARGUMENT;
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
  const int pcus = launch_cus(op.persistent);
  if (varlen) {
    char* base = static_cast<char*>(ws);
    int* order = reinterpret_cast<int*>(base + wl.order);
    int* tp = reinterpret_cast<int*>(base + wl.tile_prefix);
    unsigned* queue = pcus ? reinterpret_cast<unsigned*>(base + wl.queue) : nullptr;
    if (launch_varlen_schedule(cu_k, cu_q, cu_q, p->batch, p->num_heads_q, bm, order, tp, nullptr,
                               1, queue, nullptr, 0, 0, stream) != hipSuccess)
      return ATTN_ERR_HIP;
    fp.order = order;
    fp.tile_prefix = tp;
    fp.queue = queue;
  }
  // the FMA-path exp2 issues from the same VALU port as v_exp_f32 here, and
  // with the hand-scheduled forward step every share E > 0 measured slower at
  // head_dim 64, 128 and 256, so the default is none
  if (launch_fwd(fp, d, pcus, op.exp_emulation, stream) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status bwd_impl(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k, int phases,
                     const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  const bool varlen = cu_q != nullptr;
  attn_status st = check_params(p, varlen);
  if (st != ATTN_OK) return st;
  if (varlen && !cu_k) return ATTN_ERR_INVALID_ARGUMENT;
  if (phases <= 0 || phases > ATTN_BWD_ALL) return ATTN_ERR_INVALID_ARGUMENT;
  const BwdWs wl = bwd_ws(p, varlen);
  if (wl.design < 0) return ATTN_ERR_UNSUPPORTED;   // stored dS requested over the budget
  const bool fused_mode = wl.design == ATTN_BWD_FUSED_DQ;
  const bool pre = phases & ATTN_BWD_PREPROCESS, main = phases & ATTN_BWD_MAIN,
             post = (phases & ATTN_BWD_POSTPROCESS) && fused_mode,
             dqk = (phases & ATTN_BWD_DQ) && !fused_mode;
  if (pre && (!o || !dout || !aligned16(o) || !aligned16(dout))) return ATTN_ERR_INVALID_ARGUMENT;
  if ((main || dqk) && (!q || !k || !v || !dout || !lse)) return ATTN_ERR_INVALID_ARGUMENT;
  if ((main || dqk) && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) ||
                        (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (main && (!dk || !dv || !aligned16(dk) || !aligned16(dv))) return ATTN_ERR_INVALID_ARGUMENT;
  if ((post || dqk) && (!dq || !aligned16(dq))) return ATTN_ERR_INVALID_ARGUMENT;
  if (ws_bytes < wl.total) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (!ws) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->batch == 0) return ATTN_OK;
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
  const int bn = fused ? bwd_block_n(d) : dkdv_block_n(d), bm = bwd_block_m(d);
  bp.nn = cdiv(p->seqlen_k, bn);
  bp.nm = cdiv(p->seqlen_q, bm);
  bp.sec = section_width(2ll * bp.group * p->seqlen_q * d * 2);
  bp.nxcd = kNxcd;
  bp.natural = op.natural ? 1 : 0;
  bp.ntiles = bwd_grid(p, varlen, fused);
  bp.ntiles_dq = dq_grid(p, varlen);
  bp.causal = p->causal;
  bp.deterministic = p->deterministic;
  bp.alpha = p->softmax_scale;
  bp.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  bp.rows_q = rows_q_of(p, varlen);
  bp.n_sem = fused ? wl.n_sem : 0;
  bp.zero_acc = fused ? 1 : 0;
  bp.spin_limit = op.spin_limit;
  const int bmq = use_ds ? DqDsCfg<128>::BM : dq_block_m(d);
  bp.nm_dq = cdiv(p->seqlen_q, bmq);
  if (use_ds) {
    bp.ds = base + wl.ds;
    bp.ds_bytes = static_cast<int64_t>(wl.total - wl.ds);
    bp.ds_prefix = varlen ? reinterpret_cast<const int64_t*>(base + wl.ds_prefix) : nullptr;
    bp.ntiles_dq = varlen ? (cdiv(p->total_q, bmq) + p->batch) * p->num_heads_q
                          : p->batch * p->num_heads_q * bp.nm_dq;
  }
  bp.sec_dq = section_width(2ll * p->seqlen_k * d * 2);
  if (varlen) {
    bp.order = reinterpret_cast<int*>(base + wl.order);
    bp.tile_prefix = reinterpret_cast<int*>(base + wl.tile_prefix);
    bp.mb_prefix = reinterpret_cast<int*>(base + wl.mb_prefix);
    bp.order_dq = reinterpret_cast<int*>(base + wl.order_dq);
    bp.tile_prefix_dq = reinterpret_cast<int*>(base + wl.tile_prefix_dq);
  }
  // Packed sequences of very different lengths make tiles too unequal for a
  // static walk (measured 19 % slower dK/dV on 16 sequences of 512..8192):
  // there the persistent workgroups draw tiles from device counters, which
  // the varlen schedule pass clears.
  const int pcus = launch_cus(op.persistent);
  if (varlen && pcus) {
    bp.queue = reinterpret_cast<unsigned*>(base + wl.misc + 8);
    bp.queue_dq = reinterpret_cast<unsigned*>(base + wl.misc + 12);
  }
  if (pre) {
    if (varlen && launch_varlen_schedule(cu_q, cu_k, cu_q, p->batch, p->num_heads_kv, bn,
                                         const_cast<int*>(bp.order),
                                         const_cast<int*>(bp.tile_prefix),
                                         const_cast<int*>(bp.mb_prefix), bm, bp.queue,
                                         const_cast<int64_t*>(bp.ds_prefix), p->num_heads_q,
                                         p->causal, stream) != hipSuccess)
      return ATTN_ERR_HIP;
    if (varlen && !fused &&
        launch_varlen_schedule(cu_k, cu_q, cu_q, p->batch, p->num_heads_q, bmq,
                               const_cast<int*>(bp.order_dq), const_cast<int*>(bp.tile_prefix_dq),
                               nullptr, 1, bp.queue_dq, nullptr, 0, 0, stream) != hipSuccess)
      return ATTN_ERR_HIP;
    if (launch_bwd_pre(bp, d, stream) != hipSuccess) return ATTN_ERR_HIP;
  }
  if (main) {
    const hipError_t e = fused ? launch_bwd_main(bp, d, bp.ntiles, true, stream)
                               : launch_bwd_dkdv(bp, d, pcus, stream);
    if (e != hipSuccess) return ATTN_ERR_HIP;
  }
  if (dqk) {
    const hipError_t e = use_ds ? launch_bwd_dq_ds(bp, d, pcus, stream)
                                   : launch_bwd_dq(bp, d, pcus, stream);
    if (e != hipSuccess) return ATTN_ERR_HIP;
  }
  if (post && launch_bwd_post(bp, d, stream) != hipSuccess) return ATTN_ERR_HIP;
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
    const int nn = cdiv(p->seqlen_k, fz ? bwd_block_n(d) : dkdv_block_n(d));
    const int grp = p->num_heads_q / p->num_heads_kv;
    const int sec = section_width(2ll * grp * p->seqlen_q * d * 2);
    const int n = bwd_grid(p, false, fz);
    *count = n;
    for (int i = 0; i < n && i < capacity; ++i) {
      const Tile t = bwd_tile_fixed(i, p->batch, p->num_heads_kv, nn, sec, which == 2, kNxcd,
                                    p->opt.tile_order != 0);
      out[3 * i] = t.seq; out[3 * i + 1] = t.head; out[3 * i + 2] = t.block;
    }
  }
  return ATTN_OK;
}

int32_t attn_persistent_tile(int32_t g, int32_t r, int32_t grid, int32_t ntiles, int32_t nx) {
  if (g < 0 || g >= grid || r < 0 || ntiles < 0 || nx < 1 || grid < (ntiles < nx ? ntiles : nx))
    return -1;
  return persistent_index(g, r, grid, ntiles, nx);
}

}  // extern "C"
