// dQ of the attention backward without atomics.
//
// dQ_i = alpha * sum_j dS_ij k_j with dS = P o (dP - D), P = exp(S - LSE),
// dP = dO V^T (FlashAttention-4 blog page, backward section: the backward
// recomputes S and P and runs the dQ, dK, dP, dV GEMMs). The pages reduce dQ
// across key blocks with global atomics (2-CTA backward section); on MI355X
// those fp32 partials reach HBM (32 KiB per 64x128 tile pair), so here one
// workgroup owns a query block and walks the key blocks instead, recomputing
// S^T and dP^T. Shaped like the forward kernel: S^T = K Q^T and
// dP^T = V dO^T put the query on the lane, so dS^T leaves the MFMA
// accumulator already in the B-operand layout of dQ^T += K^T dS^T, LSE and D
// are per-lane scalars, and dQ is written once, in bf16. No cross-workgroup
// reduction: the result is bit-reproducible by construction.
//
// Per workgroup: NW wavefronts x 32 query rows. LDS per key tile (double
// buffered): K row-major (A of S^T), V row-major (A of dP^T), K^T with the
// key order permuted inside each 16 keys (A of dQ^T).
#include "common.hpp"
#include "kernels.hpp"
#include "schedule.hpp"

namespace attn71 {

namespace {

template <int D, int BN>
struct alignas(16) DqSmem {
  static constexpr int KR = D + 8;    // K, V row stride (elements)
  static constexpr int TR = BN + 8;   // K^T row stride
  alignas(16) bf16 k[2][BN * KR];
  alignas(16) bf16 v[2][BN * KR];
  alignas(16) bf16 kt[2][D * TR];
};

template <int D, int NW, int BN>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_kernel(BwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int KS = D / 16;
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int KUN = (BN / 4) * CPR;        // 4-key x 8-dim units of K
  constexpr int KU = (KUN + NT - 1) / NT;
  constexpr int VCH = BN * CPR / NT;         // 16-byte chunks of V per thread
  static_assert(VCH * NT == BN * CPR, "V staging must divide evenly");
  static_assert(KUN % 64 == 0, "K staging covers whole wavefronts");
  using SM = DqSmem<D, BN>;
  __shared__ SM sm;

  Tile t;
  if (p.sv.cu_q) {
    t = varlen_tile(blockIdx.x, p.order_dq, p.tile_prefix_dq, p.sv.batch, p.hq, true);
    if (t.seq < 0) return;
  } else {
    if ((int)blockIdx.x >= p.sv.batch * p.hq * p.nm_dq) return;
    t = fwd_tile_fixed(blockIdx.x, p.sv.batch, p.hq, p.nm_dq, p.sec_dq, p.nxcd, p.natural != 0);
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
  const int m0 = t.block * BM;
  if (m0 >= lq) return;
  const int h = t.head;
  const int kvh = h / p.group;
  const bool causal = p.causal != 0;
  const int n_tiles = causal ? cdiv(imin(m0 + BM, lq), BN) : cdiv(lk, BN);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int qw0 = m0 + w * 32;
  const int myq = qw0 + c;
  const int64_t qstride = (int64_t)p.hq * D, kstride = (int64_t)p.hkv * D;
  const float sl2 = p.scale_log2;

  // ---- this lane's query row: Q and dO as B operands, LSE and D as scalars
  const int64_t qbytes = ((int64_t)(lq - 1) * qstride + D) * 2;
  const rsrc_t qr = make_rsrc(static_cast<const bf16*>(p.q) + qs * qstride + (int64_t)h * D, qbytes);
  const rsrc_t dr = make_rsrc(static_cast<const bf16*>(p.dout) + qs * qstride + (int64_t)h * D, qbytes);
  bf16x8 qf[KS], df[KS];
  {
    const int voff = (myq * (int)qstride + 8 * g) * 2;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      qf[kk] = buf_load16(qr, voff + 32 * kk, 0);
      df[kk] = buf_load16(dr, voff + 32 * kk, 0);
    }
  }
  float lse2 = __builtin_inff(), dsum = 0.0f;   // padding rows: P = 0
  if (myq < lq) {
    const int64_t so = p.sv.cu_q ? (int64_t)h * p.sv.total_q + qs + myq
                                 : ((int64_t)t.seq * p.hq + h) * p.sv.seqlen_q + myq;
    lse2 = p.lse[so] * 1.4426950408889634f;
    dsum = p.dsum[so];
  }

  // ---- K / V staging
  const int64_t kv_bytes = ((int64_t)(lk - 1) * kstride + D) * 2;
  const bf16* kbase = static_cast<const bf16*>(p.k) + ks0 * kstride + (int64_t)kvh * D;
  const bf16* vbase = static_cast<const bf16*>(p.v) + ks0 * kstride + (int64_t)kvh * D;
  int koffs[KU], voffs[VCH];
#pragma unroll
  for (int j = 0; j < KU; ++j) {
    const int u = imin(tid + NT * j, KUN - 1);
    int kg, dc;
    unit_coords<CPR, BN / 4>(u, &kg, &dc);
    koffs[j] = ((4 * kg) * (int)kstride + dc * 8) * 2;
  }
#pragma unroll
  for (int j = 0; j < VCH; ++j) {
    const int u = tid + NT * j;
    voffs[j] = ((u / CPR) * (int)kstride + (u % CPR) * 8) * 2;
  }
  bf16x8 kreg[KU][4], vreg[VCH];
  auto load_tile = [&](int n) {
    const int64_t t0 = (int64_t)n * BN * kstride;
    const rsrc_t kr = make_rsrc(kbase + t0, kv_bytes - 2 * t0);
    const rsrc_t vr = make_rsrc(vbase + t0, kv_bytes - 2 * t0);
#pragma unroll
    for (int j = 0; j < KU; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) kreg[j][r] = buf_load16(kr, koffs[j] + r * (int)kstride * 2, 0);
#pragma unroll
    for (int j = 0; j < VCH; ++j) vreg[j] = buf_load16(vr, voffs[j], 0);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int u = tid + NT * j;
      if (KUN % NT != 0 && u >= KUN) continue;
      int kg, dc;
      unit_coords<CPR, BN / 4>(u, &kg, &dc);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<bf16x8*>(&sm.k[buf][(4 * kg + r) * SM::KR + dc * 8]) = kreg[j][r];
      const int pos = perm16(4 * kg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 x;
        x[0] = kreg[j][0][e]; x[1] = kreg[j][1][e]; x[2] = kreg[j][2][e]; x[3] = kreg[j][3][e];
        *reinterpret_cast<bf16x4*>(&sm.kt[buf][(dc * 8 + e) * SM::TR + pos]) = x;
      }
    }
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
      const int u = tid + NT * j;
      *reinterpret_cast<bf16x8*>(&sm.v[buf][(u / CPR) * SM::KR + (u % CPR) * 8]) = vreg[j];
    }
  };

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int n = 0; n < n_tiles; ++n) {
    const int buf = n & 1;
    if (n + 1 < n_tiles) load_tile(n + 1);
    const int k0 = n * BN;
    const bool active = !(causal && k0 > qw0 + 31);
    if (active) {
      f32x16 s[NKB], dp[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) { s[kb] = f32x16{}; dp[kb] = f32x16{}; }
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int o = (kb * 32 + c) * SM::KR + (2 * kk + g) * 8;
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&sm.k[buf][o]);
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sm.v[buf][o]);
          s[kb] = mfma32(ak, qf[kk], s[kb]);
          dp[kb] = mfma32(av, df[kk], dp[kb]);
        }
      const bool need_mask = (k0 + BN > lk) || (causal && k0 + BN - 1 > qw0);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = __builtin_fmaf(s[kb][i], sl2, -lse2);
          if (need_mask) {   // select on the exponent: 2^-inf = 0, no per-lane branch
            const int key = k0 + kb * 32 + c_row(i, g);
            const bool hide = (key >= lk) | (causal & (key > myq));
            x = hide ? neg_inf() : x;
          }
          const float pv = fast_exp2(x);
          dp[kb][i] = pv * (dp[kb][i] - dsum);
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bf16x8 sb = pack_half(dp[kb], tt);
          const int col = kb * 32 + 16 * tt + 8 * g;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                &sm.kt[buf][(db * 32 + c) * SM::TR + col]);
            dqacc[db] = mfma32(a, sb, dqacc[db]);
          }
        }
    }
    if (n + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- dQ = alpha * dQ^T, bf16, this lane's query row
  if (myq < lq) {
    bf16* dst = static_cast<bf16*>(p.dq) + (qs + myq) * qstride + (int64_t)h * D + 4 * g;
    const float a = p.alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& x = dqacc[db];
        *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * j) =
            pack4(x[4 * j] * a, x[4 * j + 1] * a, x[4 * j + 2] * a, x[4 * j + 3] * a);
      }
  }
}

template <int D>
hipError_t launch_dq_d(const BwdParams& p, int grid, hipStream_t stream) {
  using C = DqCfg<D>;
  hipLaunchKernelGGL((bwd_dq_kernel<D, C::NW, C::BN>), dim3(grid), dim3(C::NW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq(const BwdParams& p, int d, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (d) {
    case 64: return launch_dq_d<64>(p, grid, stream);
    case 128: return launch_dq_d<128>(p, grid, stream);
    case 256: return launch_dq_d<256>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn71
