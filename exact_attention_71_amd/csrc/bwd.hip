// Backward attention kernels for gfx950.
//
// Method (FlashAttention-4 blog page, backward section; digest page,
// roofline paragraph): recompute S = Q K^T and P from the stored LSE, then
// five GEMMs: S, dP = dO V^T, dV += P^T dO, dK += dS^T Q, dQ += dS K, with the
// elementwise dS = P o (dP - D), D = rowsum(dO o O). One workgroup owns a key
// block and walks the query blocks; dQ is reduced across key blocks through
// global fp32 atomics (blog page, 2-CTA backward section, "dQ atomic
// accumulation"), or, in deterministic mode, through a semaphore that hands
// each query block's dQ to the key blocks in a fixed order (blog page,
// deterministic-mode section). Causal inputs take the shortest key blocks
// first in that mode, so the chain rarely waits.
//
// Kernels:
//   bwd_pre   D = rowsum(dO o O) and LSE * log2(e) (fp32), zero the dQ
//             accumulator and the semaphores / ticket / status words;
//   bwd_main  the fused design at head_dim 256, per (sequence, KV head,
//             128-key block): dK, dV in registers, dQ atomics; all query
//             heads of the KV group are walked here so dK, dV need no
//             cross-workgroup reduction (at head_dim 64 and 128 the 256-key
//             dK/dV kernel of bwd_dkdv.hip forms and adds dQ itself, one
//             reduction per 256 keys; at 256 its Q / dO ring leaves no LDS
//             for the K tile that needs);
//   bwd_post  dQ = bf16(alpha * dQ_acc).
//
// gfx950 layout of bwd_main: 4 wavefronts, wave w owns keys 32w..32w+31 of
// the block. K and V of those keys stay in registers as MFMA B operands for
// S and dP. S and dP come out with the key on the lane (lane % 32) and the
// query on the register, which is exactly the B operand layout of
// dV^T = dO^T P and dK^T = Q^T dS. Q and dO are staged in LDS twice (row-major
// for S and dP, transposed for dV and dK); dS goes through LDS once for the
// dQ product, which reads K^T from LDS.
#include "common.hpp"
#include "kernels.hpp"
#include "schedule.hpp"

namespace attn71 {

namespace {

__device__ __forceinline__ void seq_bounds_b(const SeqView& sv, int seq, int64_t* q0, int* lq,
                                             int64_t* k0, int* lk) {
  if (sv.cu_q) {
    const int a = sv.cu_q[seq], b = sv.cu_q[seq + 1];
    const int c = sv.cu_k[seq], d = sv.cu_k[seq + 1];
    *q0 = a; *lq = b - a; *k0 = c; *lk = d - c;
  } else {
    *q0 = (int64_t)seq * sv.seqlen_q; *lq = sv.seqlen_q;
    *k0 = (int64_t)seq * sv.seqlen_k; *lk = sv.seqlen_k;
  }
}

// offset of (sequence seq starting at packed row q0, head h, row r) in the
// [B, Hq, Sq] (fixed) or [Hq, total] (varlen) LSE / D layout
__device__ __forceinline__ int64_t stat_off(const SeqView& sv, int hq, int seq, int64_t q0, int h,
                                            int r) {
  return sv.cu_q ? (int64_t)h * sv.total_q + q0 + r
                 : ((int64_t)seq * hq + h) * sv.seqlen_q + r;
}

// ---------------------------------------------------------------------------
// bwd_pre: one 16-lane group per (row, query head).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int64_t n_pairs, int n_sem) {
  constexpr int L = 16;                 // lanes per (row, head)
  constexpr int E = D / L;              // elements per lane (4, 8 or 16)
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t pair = gid / L;
  const int sub = (int)(gid % L);
  if (gid < n_sem) p.sem[gid] = 0;
  if (gid == 0) { *p.ticket = 0; *p.status = 0; }
  if (pair >= n_pairs) return;
  const int64_t row = pair / p.hq;      // packed row (fixed: b * Sq + s)
  const int h = (int)(pair % p.hq);
  const int64_t base = (row * p.hq + h) * D + sub * E;
  const bf16* o = static_cast<const bf16*>(p.o) + base;
  const bf16* g = static_cast<const bf16*>(p.dout) + base;
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(o + e);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(g + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc += (float)a[j] * (float)b[j];
  }
  if (p.zero_acc) {
    float* z = p.dq_acc + base;
#pragma unroll
    for (int e = 0; e < E; e += 4) *reinterpret_cast<f32x4*>(z + e) = f32x4{};
  }
#pragma unroll
  for (int s = L / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, kWave);
  if (sub == 0) {
    int64_t off;
    if (p.sv.cu_q) {
      off = (int64_t)h * p.sv.total_q + row;
    } else {
      const int64_t b = row / p.sv.seqlen_q, s = row % p.sv.seqlen_q;
      off = (b * p.hq + h) * p.sv.seqlen_q + s;
    }
    p.dsum[off] = -acc;
    p.lse2[off] = lse_log2(p.lse[off]);
  }
}

// ---------------------------------------------------------------------------
// bwd_post: dQ = bf16(alpha * dQ_acc), 8 elements per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_post_kernel(const float* __restrict__ acc,
                                                       bf16* __restrict__ dq, int64_t n8,
                                                       float alpha) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(acc + 8 * i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(acc + 8 * i + 4);
  *reinterpret_cast<bf16x8*>(dq + 8 * i) = pack8(a[0] * alpha, a[1] * alpha, a[2] * alpha,
                                                 a[3] * alpha, b[0] * alpha, b[1] * alpha,
                                                 b[2] * alpha, b[3] * alpha);
}

// ---------------------------------------------------------------------------
// bwd_dkdv_reduce: with a head split, dK = bf16(alpha sum of the parts' dK
// partials), dV = bf16(sum of the dV partials), parts added in order (the
// same bits for every run), 8 elements per thread. Packed rows past the last
// sequence (total_k above cu_seqlens_k[batch]) have no partials: untouched.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(const float* __restrict__ dkp,
                                                              const float* __restrict__ dvp,
                                                              bf16* __restrict__ dk,
                                                              bf16* __restrict__ dv, int64_t n8,
                                                              int64_t part_stride, int parts,
                                                              float alpha, const int* cu_k,
                                                              int nseq, int64_t row8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  if (cu_k && i / row8 >= cu_k[nseq]) return;
  f32x4 k0 = {}, k1 = {}, v0 = {}, v1 = {};
  for (int s = 0; s < parts; ++s) {
    const int64_t o = s * part_stride + 8 * i;
    k0 += *reinterpret_cast<const f32x4*>(dkp + o);
    k1 += *reinterpret_cast<const f32x4*>(dkp + o + 4);
    v0 += *reinterpret_cast<const f32x4*>(dvp + o);
    v1 += *reinterpret_cast<const f32x4*>(dvp + o + 4);
  }
  *reinterpret_cast<bf16x8*>(dk + 8 * i) = pack8(k0[0] * alpha, k0[1] * alpha, k0[2] * alpha,
                                                 k0[3] * alpha, k1[0] * alpha, k1[1] * alpha,
                                                 k1[2] * alpha, k1[3] * alpha);
  *reinterpret_cast<bf16x8*>(dv + 8 * i) = pack8(v0[0], v0[1], v0[2], v0[3], v1[0], v1[1],
                                                 v1[2], v1[3]);
}

// ---------------------------------------------------------------------------
// bwd_main
// ---------------------------------------------------------------------------
template <int D, int BM, int BN>
struct alignas(16) BwdSmem {
  static constexpr int QR = D + 8;    // row-major Q / dO (rows = queries)
  static constexpr int TR = BM + 8;   // transposed Q^T / dO^T (rows = dims)
  static constexpr int SR = BN + 8;   // dS (rows = queries)
  static constexpr int KR = BN + 8;   // K^T (rows = dims)
  alignas(16) bf16 q[BM * QR];
  alignas(16) bf16 dout[BM * QR];
  alignas(16) bf16 qt[D * TR];
  alignas(16) bf16 dot[D * TR];
  alignas(16) bf16 ds[BM * SR];
  alignas(16) bf16 kt[D * KR];
  alignas(16) float lse2[BM];
  alignas(16) float dsum[BM];
  int ticket;
};

template <int D, bool MASK>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(BwdParams p) {
  constexpr int BN = BwdCfg<D>::BN;     // 128 keys, 32 per wave
  constexpr int BM = BwdCfg<D>::BM;     // queries per step
  constexpr int KS = D / 16;            // k-steps over dims
  constexpr int NDB = D / 32;           // 32-row dim blocks of dK^T / dV^T
  constexpr int NQB = BM / 32;          // 32-query blocks per step
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int QU = (BM / 4) * CPR;    // 4-row x 8-dim staging units per tile
  constexpr int QUT = (QU + 255) / 256; // units per thread
  constexpr int NUNIT = NQB * NDB;      // dQ output units (32 x 32)
  static_assert(NUNIT % 4 == 0, "dQ units must split over 4 waves");
  using SM = BwdSmem<D, BM, BN>;
  __shared__ SM sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63, g = lane >> 5, c = lane & 31;
  const bool det = p.deterministic != 0;
  const bool causal = p.causal != 0;

  // ---- which key block (deterministic: ticket order = shortest first)
  int v = blockIdx.x;
  if (det) {
    // Every workgroup of a launch takes one ticket, so a launch consumes
    // exactly gridDim.x tickets; the modulo keeps v inside this launch's grid
    // even if the counter was not cleared since the previous launch.
    if (tid == 0) sm.ticket = (int)((unsigned)atomicAdd(p.ticket, 1) % gridDim.x);
    __syncthreads();
    v = sm.ticket;
  }
  Tile t;
  if (p.sv.cu_q) {
    t = varlen_tile(v, p.order, p.tile_prefix, p.sv.batch, p.hkv, /*reverse=*/det);
    if (t.seq < 0) return;
  } else {
    if (v >= p.sv.batch * p.hkv * p.nn) return;
    t = bwd_tile_fixed(v, p.sv.batch, p.hkv, p.nn, p.sec, det, p.nxcd, p.natural != 0);
  }
  int64_t qs, ks0;
  int lq, lk;
  seq_bounds_b(p.sv, t.seq, &qs, &lq, &ks0, &lk);
  const int n0 = t.block * BN;
  if (n0 >= lk) return;
  const int kvh = t.head;
  const int64_t qstride = (int64_t)p.hq * D, kstride = (int64_t)p.hkv * D;
  const float sl2 = p.scale_log2;
  const int nm = cdiv(lq, BM);
  const int shift = lk - lq;            // causal: row i sees keys j <= i + shift
  const int m_first = causal ? causal_row_begin(n0, shift) / BM : 0;
  const int nlast_all = cdiv(lk, BN) - 1;   // last key block of this sequence
  // block mask (MASK): the block's 128 keys form one mask column, each step's
  // rows lie in one 128-row block
  const rsrc_t mrs = raw_rsrc(p.mask.mask, MASK ? p.mask.range : 0);
  uint32_t mcol = 0;
  if constexpr (MASK) {
    static_assert(BN == kMaskBlock, "one mask column per key block");
    mcol = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        (int64_t)t.seq * p.mask.sb + n0 / kMaskBlock));
  }

  // ---- K, V of this wave's keys as B operands; K^T of the block in LDS
  const int64_t kv_bytes = ((int64_t)(lk - 1) * kstride + D) * 2;
  const bf16* kbase = static_cast<const bf16*>(p.k) + ks0 * kstride + (int64_t)kvh * D;
  const bf16* vbase = static_cast<const bf16*>(p.v) + ks0 * kstride + (int64_t)kvh * D;
  const rsrc_t kr = make_rsrc(kbase, kv_bytes);
  const rsrc_t vr = make_rsrc(vbase, kv_bytes);
  const int mykey = n0 + 32 * w + c;
  bf16x8 kf[KS], vf[KS];
  {
    const int off = (mykey * (int)kstride + 8 * g) * 2;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      kf[kk] = buf_load16(kr, off + 32 * kk, 0);
      vf[kk] = buf_load16(vr, off + 32 * kk, 0);
    }
  }
  {
    constexpr int KU = (BN / 4) * CPR;
    for (int u = tid; u < KU; u += 256) {
      const int kg = u / CPR, dc = u % CPR;
      bf16x8 x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[r] = buf_load16(kr, ((n0 + 4 * kg + r) * (int)kstride + dc * 8) * 2, 0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 y;
        y[0] = x[0][e]; y[1] = x[1][e]; y[2] = x[2][e]; y[3] = x[3][e];
        *reinterpret_cast<bf16x4*>(&sm.kt[(dc * 8 + e) * SM::KR + 4 * kg]) = y;
      }
    }
  }

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkacc[db] = f32x16{}; dvacc[db] = f32x16{}; }

  // ---- staging of one (query head, query block) step
  bf16x8 qreg[QUT][4], oreg[QUT][4];
  float lreg = 0.0f, dreg = 0.0f;
  auto load_step = [&](int hq, int m) {
    const int64_t qb0 = (qs + (int64_t)m * BM) * qstride + (int64_t)hq * D;
    const int rows = imin(BM, lq - m * BM);
    const int64_t bytes = ((int64_t)(rows - 1) * qstride + D) * 2;
    const rsrc_t qrs = make_rsrc(static_cast<const bf16*>(p.q) + qb0, bytes);
    const rsrc_t ors = make_rsrc(static_cast<const bf16*>(p.dout) + qb0, bytes);
#pragma unroll
    for (int j = 0; j < QUT; ++j) {
      const int u = imin(tid + 256 * j, QU - 1);
      int qg, dc;
      unit_coords<CPR, BM / 4>(u, &qg, &dc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int off = ((4 * qg + r) * (int)qstride + dc * 8) * 2;
        qreg[j][r] = buf_load16(qrs, off, 0);
        oreg[j][r] = buf_load16(ors, off, 0);
      }
    }
    if (tid < BM) {
      const int r = m * BM + tid;
      if (r < lq) {
        const int64_t so = stat_off(p.sv, p.hq, t.seq, qs, hq, r);
        lreg = lse_log2(p.lse[so]);
        dreg = p.dsum[so];
      } else {
        lreg = __builtin_inff();   // padding rows: P = 0
        dreg = 0.0f;
      }
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int j = 0; j < QUT; ++j) {
      const int u = tid + 256 * j;
      if (QU % 256 == 0 || u < QU) {
        int qg, dc;
        unit_coords<CPR, BM / 4>(u, &qg, &dc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          *reinterpret_cast<bf16x8*>(&sm.q[(4 * qg + r) * SM::QR + dc * 8]) = qreg[j][r];
          *reinterpret_cast<bf16x8*>(&sm.dout[(4 * qg + r) * SM::QR + dc * 8]) = oreg[j][r];
        }
        const int pos = perm16(4 * qg);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16x4 a, b;
          a[0] = qreg[j][0][e]; a[1] = qreg[j][1][e]; a[2] = qreg[j][2][e]; a[3] = qreg[j][3][e];
          b[0] = oreg[j][0][e]; b[1] = oreg[j][1][e]; b[2] = oreg[j][2][e]; b[3] = oreg[j][3][e];
          *reinterpret_cast<bf16x4*>(&sm.qt[(dc * 8 + e) * SM::TR + pos]) = a;
          *reinterpret_cast<bf16x4*>(&sm.dot[(dc * 8 + e) * SM::TR + pos]) = b;
        }
      }
    }
    if (tid < BM) { sm.lse2[tid] = lreg; sm.dsum[tid] = dreg; }
  };

  const int n_steps = p.group * (nm - m_first);
  if (n_steps > 0) {
    load_step(kvh * p.group, m_first);
    store_step();
  }
  __syncthreads();

  float* __restrict__ dq_acc = p.dq_acc;
  for (int step = 0; step < n_steps; ++step) {
    const int hq = kvh * p.group + step / (nm - m_first);
    const int m = m_first + step % (nm - m_first);
    if (step + 1 < n_steps) {
      const int s1 = step + 1;
      load_step(kvh * p.group + s1 / (nm - m_first), m_first + s1 % (nm - m_first));
    }
    const int mq0 = m * BM;              // first query row of this step

    // S = Q K^T and dP - D = dO V^T - D: key on the lane, query on the
    // register; the dP accumulators start from the rows' -D (as in the dK/dV
    // kernel, so both designs compute dS in the same order)
    f32x16 s[NQB], dp[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      s[qb] = f32x16{};
#pragma unroll
      for (int i = 0; i < 16; ++i) dp[qb][i] = sm.dsum[qb * 32 + c_row(i, g)];
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int o = (qb * 32 + c) * SM::QR + 16 * kk + 8 * g;
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sm.q[o]);
        const bf16x8 ao = *reinterpret_cast<const bf16x8*>(&sm.dout[o]);
        s[qb] = mfma32(aq, kf[kk], s[qb]);
        dp[qb] = mfma32(ao, vf[kk], dp[qb]);
      }

    // P = 2^(S alpha log2e - LSE log2e), dS = P (dP - D) (the stored rows hold -D);
    // a cleared mask block hides the whole step
    bool hid = false;
    if constexpr (MASK)
      hid = !mask_set(mrs, mcol + static_cast<uint32_t>((int64_t)hq * p.mask.sh +
                                                         (int64_t)(mq0 / kMaskBlock) * p.mask.nkb));
    const bool need_mask = hid || (n0 + BN > lk) || (causal && n0 + BN - 1 > mq0 + shift);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q4 = qb * 32 + 8 * j + 4 * g;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[q4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * j + r;
          float pv = fast_exp2(__builtin_fmaf(s[qb][i], sl2, -l4[r]));
          if (need_mask) {
            const int qrow = mq0 + q4 + r;
            if (hid || mykey >= lk || (causal && mykey > qrow + shift)) pv = 0.0f;
          }
          s[qb][i] = pv;
          dp[qb][i] = pv * dp[qb][i];
        }
      }

    // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 pb = pack_half(s[qb], tt);
        const bf16x8 sb = pack_half(dp[qb], tt);
        const int col = qb * 32 + 16 * tt + 8 * g;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int o = (db * 32 + c) * SM::TR + col;
          const bf16x8 ao = *reinterpret_cast<const bf16x8*>(&sm.dot[o]);
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sm.qt[o]);
          dvacc[db] = mfma32(ao, pb, dvacc[db]);
          dkacc[db] = mfma32(aq, sb, dkacc[db]);
        }
      }

    // dS -> LDS as [query][key]
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        sm.ds[(qb * 32 + c_row(i, g)) * SM::SR + 32 * w + c] = (bf16)dp[qb][i];
    __syncthreads();

    // dQ_part = dS K over this block's 128 keys; units of 32 queries x 32 dims
    f32x16 dqp[NUNIT / 4];
#pragma unroll
    for (int uu = 0; uu < NUNIT / 4; ++uu) {
      const int unit = w * (NUNIT / 4) + uu;
      const int qb = unit / NDB, db = unit % NDB;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < BN / 16; ++kk) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&sm.ds[(qb * 32 + c) * SM::SR + 16 * kk + 8 * g]);
        const bf16x8 b =
            *reinterpret_cast<const bf16x8*>(&sm.kt[(db * 32 + c) * SM::KR + 16 * kk + 8 * g]);
        acc = mfma32(a, b, acc);
      }
      dqp[uu] = acc;
    }
    // deterministic: wait until the key blocks after this one have added
    int* semp = nullptr;
    if (det) {
      const int64_t mb = p.sv.cu_q ? (int64_t)p.mb_prefix[t.seq] + m : (int64_t)t.seq * p.nm + m;
      semp = p.sem + mb * p.hq + hq;
      const int nlast = causal ? imin(nlast_all, (mq0 + BM - 1 + shift) / BN) : nlast_all;
      const int turn = nlast - t.block;
      if (tid == 0) {
        // bounded wait: once any wait has expired (status set) nobody waits again
        int it = 0;
        while (__hip_atomic_load(semp, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < turn) {
          if (++it > p.spin_limit) { atomicOr(p.status, 1); break; }
          if ((it & 255) == 0 &&
              __hip_atomic_load(p.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
            break;
          __builtin_amdgcn_s_sleep(2);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int uu = 0; uu < NUNIT / 4; ++uu) {
      const int unit = w * (NUNIT / 4) + uu;
      const int qb = unit / NDB, db = unit % NDB;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qrow = mq0 + qb * 32 + c_row(i, g);
        if (qrow < lq) {
          float* dst = dq_acc + (qs + qrow) * qstride + (int64_t)hq * D + db * 32 + c;
          unsafeAtomicAdd(dst, dqp[uu][i]);
        }
      }
    }
    if (det) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(semp, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      __syncthreads();
    }
    if (step + 1 < n_steps) {
      store_step();
      __syncthreads();
    }
  }

  // ---- epilogue: dK = alpha dK^T, dV = dV^T, rows of this wave's keys
  if (mykey < lk) {
    const int64_t ro = (ks0 + mykey) * kstride + (int64_t)kvh * D + 4 * g;
    bf16* dk = static_cast<bf16*>(p.dk) + ro;
    bf16* dv = static_cast<bf16*>(p.dv) + ro;
    const float a = p.alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& x = dkacc[db];
        const f32x16& y = dvacc[db];
        *reinterpret_cast<bf16x4*>(dk + db * 32 + 8 * j) =
            pack4(x[4 * j] * a, x[4 * j + 1] * a, x[4 * j + 2] * a, x[4 * j + 3] * a);
        *reinterpret_cast<bf16x4*>(dv + db * 32 + 8 * j) =
            pack4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
      }
  }
}

}  // namespace

hipError_t launch_bwd_pre(const BwdParams& p, int d, hipStream_t stream) {
  const int64_t pairs = p.rows_q * p.hq;
  int64_t threads = pairs * 16;
  if (threads < p.n_sem) threads = p.n_sem;
  int64_t blocks = (threads + 255) / 256;
  if (blocks < 1) blocks = 1;
  const int ns = (int)p.n_sem;
  switch (d) {
    case 64: hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, p, pairs, ns); break;
    case 128: hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, p, pairs, ns); break;
    case 256: hipLaunchKernelGGL(bwd_pre_kernel<256>, dim3((unsigned)blocks), dim3(256), 0, stream, p, pairs, ns); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_main(const BwdParams& p, int d, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (d != 256) return hipErrorInvalidValue;   // 64, 128: the 256-key dK/dV kernel
  if (p.mask.mask)
    hipLaunchKernelGGL((bwd_main_kernel<256, true>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((bwd_main_kernel<256, false>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_reduce(const BwdParams& p, int d, hipStream_t stream) {
  if (p.hsplit <= 1) return hipSuccess;
  const int64_t per_part = p.rows_k * p.hkv * d;
  const int64_t n8 = per_part / 8;
  if (n8 <= 0) return hipSuccess;
  const int64_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(bwd_dkdv_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     p.dk_part, p.dv_part, static_cast<bf16*>(p.dk), static_cast<bf16*>(p.dv), n8,
                     per_part, p.hsplit, p.alpha, p.sv.cu_k, p.sv.batch, (int64_t)p.hkv * d / 8);
  return hipGetLastError();
}

hipError_t launch_bwd_post(const BwdParams& p, int d, hipStream_t stream) {
  const int64_t n8 = p.rows_q * p.hq * d / 8;
  if (n8 <= 0) return hipSuccess;
  const int64_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(bwd_post_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p.dq_acc,
                     static_cast<bf16*>(p.dq), n8, p.alpha);
  return hipGetLastError();
}

}  // namespace attn71
