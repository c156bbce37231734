// dK and dV of the attention backward (the four GEMMs that need no
// cross-workgroup reduction): S = Q K^T, dP = dO V^T, dV += P^T dO,
// dK += dS^T Q with P = exp(S - LSE) and dS = P o (dP - D)
// (FlashAttention-4 blog page, backward section). dQ comes from the
// query-block kernel in bwd_dq.hip.
//
// One workgroup owns NW * 32 keys of one (sequence, KV head); wave w owns 32
// of them, keeping their K and V as MFMA B operands and their dK^T, dV^T
// accumulators in registers, and walks every query head of the KV group and
// every query block (from the causal diagonal) in steps of BM queries.
// S and dP come out with the key on the lane and the query on the register,
// which is the B-operand layout of dV^T = dO^T P and dK^T = Q^T dS, so P and
// dS never leave the registers. Q and dO of the next step are fetched into
// registers during the current step and written, row-major (A of S, dP) and
// transposed (A of dV^T, dK^T), into the other half of a double buffer:
// one barrier per step. With 8 wavefronts two waves share each SIMD, so one
// wave's MFMAs overlap the other's elementwise work.
#include "common.hpp"
#include "kernels.hpp"
#include "schedule.hpp"

namespace attn71 {

namespace {

template <int D, int BM>
struct alignas(16) DkdvSmem {
  static constexpr int QR = D + 8;    // row-major Q / dO (rows = queries)
  static constexpr int TR = BM + 8;   // transposed Q^T / dO^T (rows = dims)
  alignas(16) bf16 q[2][BM * QR];
  alignas(16) bf16 dout[2][BM * QR];
  alignas(16) bf16 qt[2][D * TR];
  alignas(16) bf16 dot[2][D * TR];
  alignas(16) float lse2[2][BM];
  alignas(16) float dsum[2][BM];
};

template <int D, int NW, int BM>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BN = NW * 32;           // keys per workgroup
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NQB = BM / 32;
  constexpr int CPR = D / 8;
  using SM = DkdvSmem<D, BM>;
  __shared__ SM sm;

  Tile t;
  if (p.sv.cu_q) {
    t = varlen_tile(blockIdx.x, p.order, p.tile_prefix, p.sv.batch, p.hkv, /*reverse=*/false);
    if (t.seq < 0) return;
  } else {
    if ((int)blockIdx.x >= p.sv.batch * p.hkv * p.nn) return;
    t = bwd_tile_fixed(blockIdx.x, p.sv.batch, p.hkv, p.nn, p.sec, false, p.nxcd, p.natural != 0);
  }
  int64_t qs, ks0;
  int lq, lk;
  if (p.sv.cu_q) {
    const int a = p.sv.cu_q[t.seq], b = p.sv.cu_q[t.seq + 1];
    const int c0 = p.sv.cu_k[t.seq], d0 = p.sv.cu_k[t.seq + 1];
    qs = a; lq = b - a; ks0 = c0; lk = d0 - c0;
  } else {
    qs = (int64_t)t.seq * p.sv.seqlen_q; lq = p.sv.seqlen_q;
    ks0 = (int64_t)t.seq * p.sv.seqlen_k; lk = p.sv.seqlen_k;
  }
  const int n0 = t.block * BN;
  if (n0 >= lk) return;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const bool causal = p.causal != 0;
  const int kvh = t.head;
  const int64_t qstride = (int64_t)p.hq * D, kstride = (int64_t)p.hkv * D;
  const float sl2 = p.scale_log2;
  const int nm = cdiv(lq, BM);
  const int m_first = causal ? imin(n0 / BM, nm) : 0;
  const int per_head = nm - m_first;
  const int n_steps = p.group * per_head;

  // ---- this wave's 32 keys: K and V as B operands
  const int mykey = n0 + 32 * w + c;
  bf16x8 kf[KS], vf[KS];
  {
    const int64_t kv_bytes = ((int64_t)(lk - 1) * kstride + D) * 2;
    const rsrc_t kr = make_rsrc(static_cast<const bf16*>(p.k) + ks0 * kstride + (int64_t)kvh * D, kv_bytes);
    const rsrc_t vr = make_rsrc(static_cast<const bf16*>(p.v) + ks0 * kstride + (int64_t)kvh * D, kv_bytes);
    const int off = (mykey * (int)kstride + 8 * g) * 2;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      kf[kk] = buf_load16(kr, off + 32 * kk, 0);
      vf[kk] = buf_load16(vr, off + 32 * kk, 0);
    }
  }
  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkacc[db] = f32x16{}; dvacc[db] = f32x16{}; }

  // ---- staging of one (query head, query block) step. A unit is RU rows x 8
  // dims of Q (units [0, QU)) or dO (units [QU, 2QU)); RU = 2 when that lets
  // every thread hold one unit (fewer live registers), else 4.
  constexpr int RU = (2 * (BM / 2) * CPR <= NT) ? 2 : 4;
  constexpr int QU2 = (BM / RU) * CPR;
  constexpr int UPT2 = (2 * QU2 + NT - 1) / NT;
  static_assert((2 * QU2) % 64 == 0, "staging covers whole wavefronts");
  bf16x8 sreg[UPT2][RU];
  float lreg = 0.0f, dreg = 0.0f;
  auto step_hm = [&](int s, int* hq, int* m) {
    *hq = kvh * p.group + s / per_head;
    *m = m_first + s % per_head;
  };
  auto coords = [&](int u, int* rg, int* dc) {
    if constexpr (RU == 4) unit_coords<CPR, BM / 4>(u, rg, dc);
    else unit_coords<CPR, BM / 2>(u, rg, dc);
  };
  auto load_step = [&](int s) {
    int hq, m;
    step_hm(s, &hq, &m);
    const int64_t qb0 = (qs + (int64_t)m * BM) * qstride + (int64_t)hq * D;
    const int rows = imin(BM, lq - m * BM);
    const int64_t bytes = ((int64_t)(rows - 1) * qstride + D) * 2;
    const rsrc_t qrs = make_rsrc(static_cast<const bf16*>(p.q) + qb0, bytes);
    const rsrc_t ors = make_rsrc(static_cast<const bf16*>(p.dout) + qb0, bytes);
#pragma unroll
    for (int j = 0; j < UPT2; ++j) {
      const int u = tid + NT * j;
      if (u < 2 * QU2) {
        const bool isq = u < QU2;
        int rg, dc;
        coords(isq ? u : u - QU2, &rg, &dc);
#pragma unroll
        for (int r = 0; r < RU; ++r)
          sreg[j][r] = buf_load16(isq ? qrs : ors, ((RU * rg + r) * (int)qstride + dc * 8) * 2, 0);
      }
    }
    if (tid < BM) {
      const int r = m * BM + tid;
      if (r < lq) {
        const int64_t so = p.sv.cu_q ? (int64_t)hq * p.sv.total_q + qs + r
                                     : ((int64_t)t.seq * p.hq + hq) * p.sv.seqlen_q + r;
        lreg = p.lse[so] * 1.4426950408889634f;
        dreg = p.dsum[so];
      } else {
        lreg = __builtin_inff();   // padding rows: P = 0
        dreg = 0.0f;
      }
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int j = 0; j < UPT2; ++j) {
      const int u = tid + NT * j;
      if (u < 2 * QU2) {
        const bool isq = u < QU2;
        int rg, dc;
        coords(isq ? u : u - QU2, &rg, &dc);
        bf16* rm = isq ? sm.q[buf] : sm.dout[buf];
        bf16* tr = isq ? sm.qt[buf] : sm.dot[buf];
#pragma unroll
        for (int r = 0; r < RU; ++r)
          *reinterpret_cast<bf16x8*>(&rm[(RU * rg + r) * SM::QR + dc * 8]) = sreg[j][r];
        const int pos = perm16(RU * rg);   // RU consecutive rows stay contiguous
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (RU == 4) {
            bf16x4 x;
            x[0] = sreg[j][0][e]; x[1] = sreg[j][1][e]; x[2] = sreg[j][2][e]; x[3] = sreg[j][3][e];
            *reinterpret_cast<bf16x4*>(&tr[(dc * 8 + e) * SM::TR + pos]) = x;
          } else {
            bf16x2 x;
            x[0] = sreg[j][0][e]; x[1] = sreg[j][1][e];
            *reinterpret_cast<bf16x2*>(&tr[(dc * 8 + e) * SM::TR + pos]) = x;
          }
        }
      }
    }
    if (tid < BM) { sm.lse2[buf][tid] = lreg; sm.dsum[buf][tid] = dreg; }
  };

  if (n_steps > 0) {
    load_step(0);
    store_step(0);
  }
  __syncthreads();

  for (int step = 0; step < n_steps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < n_steps;
    if (more) load_step(step + 1);
    int hq, m;
    step_hm(step, &hq, &m);
    const int mq0 = m * BM;
    // whole wave above the diagonal: no visible pair in this step
    const bool active = !(causal && n0 + 32 * w > mq0 + BM - 1);
    if (active) {
      f32x16 s[NQB], dp[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) { s[qb] = f32x16{}; dp[qb] = f32x16{}; }
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const int o = (qb * 32 + c) * SM::QR + 16 * kk + 8 * g;
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sm.q[buf][o]);
          const bf16x8 ao = *reinterpret_cast<const bf16x8*>(&sm.dout[buf][o]);
          s[qb] = mfma32(aq, kf[kk], s[qb]);
          dp[qb] = mfma32(ao, vf[kk], dp[qb]);
        }
      const bool need_mask = (n0 + 32 * w + 31 >= lk) || (causal && n0 + 32 * w + 31 > mq0);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q4 = qb * 32 + 8 * j + 4 * g;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][q4]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dsum[buf][q4]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * j + r;
            float pv = fast_exp2(__builtin_fmaf(s[qb][i], sl2, -l4[r]));
            if (need_mask) {
              const int qrow = mq0 + q4 + r;
              if (mykey >= lk || (causal && mykey > qrow)) pv = 0.0f;
            }
            s[qb][i] = pv;
            dp[qb][i] = pv * (dp[qb][i] - d4[r]);
          }
        }
      // pack P and dS to bf16 first so the fp32 tiles die before the next GEMMs
      bf16x8 pbs[NQB][2], sbs[NQB][2];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          pbs[qb][tt] = pack_half(s[qb], tt);
          sbs[qb][tt] = pack_half(dp[qb], tt);
        }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bf16x8 pb = pbs[qb][tt];
          const bf16x8 sb = sbs[qb][tt];
          const int col = qb * 32 + 16 * tt + 8 * g;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int o = (db * 32 + c) * SM::TR + col;
            const bf16x8 ao = *reinterpret_cast<const bf16x8*>(&sm.dot[buf][o]);
            const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sm.qt[buf][o]);
            dvacc[db] = mfma32(ao, pb, dvacc[db]);
            dkacc[db] = mfma32(aq, sb, dkacc[db]);
          }
        }
    }
    if (more) store_step(buf ^ 1);
    __syncthreads();
  }

  // ---- dK = alpha dK^T, dV = dV^T for this wave's keys
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

template <int D>
hipError_t launch_dkdv_d(const BwdParams& p, int grid, hipStream_t stream) {
  using C = DkdvCfg<D>;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, C::NW, C::BM>), dim3(grid), dim3(C::NW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdParams& p, int d, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (d) {
    case 64: return launch_dkdv_d<64>(p, grid, stream);
    case 128: return launch_dkdv_d<128>(p, grid, stream);
    case 256: return launch_dkdv_d<256>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn71
