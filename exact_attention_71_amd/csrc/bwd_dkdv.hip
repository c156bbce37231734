// dK and dV of the attention backward (the four GEMMs that need no
// cross-workgroup reduction): S = Q K^T, dP = dO V^T, dV += P^T dO,
// dK += dS^T Q with P = exp(S - LSE) and dS = P o (dP - D)
// (FlashAttention-4 blog page, backward section). dQ comes from the
// query-block kernel in bwd_dq.hip.
//
// One workgroup of four wavefronts (one per SIMD, so each may hold 512
// registers) owns 4 * 32 * KB keys of one (sequence, KV head). Wave w owns
// 32 * KB of them: their K and V stay in VGPRs as MFMA B operands for the
// whole kernel and their dK^T, dV^T accumulators in AGPRs (pinned there by
// mfma32_agpr; S and dP use the VGPR form). The workgroup walks
// every query head of the KV group and every query block from the causal
// diagonal on, BM queries per step.
//
// Per step, Q and dO (BM x D each) and the rows' LSE and D arrive in LDS by
// direct global->LDS loads, issued NS - 1 steps ahead into an NS-deep ring,
// so no registers or VALU work go into staging. The same row-major tiles
// serve both products: ds_read_b128 gives the A operand of S and dP, and the
// transposing LDS read gives the A operand (Q^T, dO^T) of dK^T and dV^T. S
// and dP come out with the key on the lane and the query on the register,
// which is the B-operand layout of dV^T = dO^T P and dK^T = Q^T dS, so P and
// dS never leave the registers. Each LDS operand fragment feeds KB MFMAs.
#include "common.hpp"
#include "kernels.hpp"
#include "schedule.hpp"

namespace attn71 {

namespace {

template <int D, int KB, int BM>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int NW = 4, NT = NW * 64;
  constexpr int KPW = 32 * KB;          // keys per wave
  constexpr int BN = NW * KPW;          // keys per workgroup
  constexpr int KS = D / 16;            // k-steps of S and dP
  constexpr int NDB = D / 32;           // 32-dim blocks of dK^T, dV^T
  constexpr int NQB = BM / 32;          // 32-query blocks per step
  constexpr int RB = 2 * D;             // bytes per tile row
  constexpr int SPR = D / 8;            // 16-byte slots per row
  constexpr int TILE = BM * RB;         // bytes of one Q (or dO) tile
  constexpr int NS = 3;                 // ring depth
  static_assert(NS == 3, "wait_next() counts at most one later step in flight");
  constexpr int CH = TILE / (16 * NT);  // dma16 per thread per tile
  constexpr int NLD = 2 * BM / 64;      // dma4 (LSE and D) per step, waves 0 .. NLD-1
  static_assert(TILE % (16 * NT) == 0 && NLD <= NW, "tile split over the workgroup");
  constexpr int OPS = 2 * CH;           // dma per step by waves >= NLD (one more below)
  static_assert(OPS + 1 < 64, "vmcnt range");
  // [NS] Q tiles | [NS] dO tiles | [NS][LSE BM | D BM] fp32
  __shared__ __attribute__((aligned(1024))) char smem[2 * NS * TILE + NS * 2 * BM * 4];
  char* const qtile = smem;
  char* const otile = smem + NS * TILE;
  float* const lsed = reinterpret_cast<float*>(smem + 2 * NS * TILE);
  static_assert(BN == DkdvCfg<D>::BN && BM == DkdvCfg<D>::BM, "host and kernel tiling agree");

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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63, g = lane >> 5, c = lane & 31;
  const bool causal = p.causal != 0;
  const int kvh = t.head;
  const int64_t qstride = (int64_t)p.hq * D, kstride = (int64_t)p.hkv * D;
  const float sl2 = p.scale_log2;
  const int nm = cdiv(lq, BM);
  const int m_first = causal ? imin(n0 / BM, nm) : 0;
  const int per_head = nm - m_first;
  const int n_steps = p.group * per_head;
  const int wk0 = n0 + KPW * w;         // first key of this wave

  // ---- this wave's keys: K and V as B operands (key on the lane)
  bf16x8 kf[KB][KS], vf[KB][KS];
  {
    const int64_t kv_bytes = ((int64_t)(lk - 1) * kstride + D) * 2;
    const rsrc_t kr = make_rsrc(static_cast<const bf16*>(p.k) + ks0 * kstride + (int64_t)kvh * D, kv_bytes);
    const rsrc_t vr = make_rsrc(static_cast<const bf16*>(p.v) + ks0 * kstride + (int64_t)kvh * D, kv_bytes);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int off = ((wk0 + 32 * kb + c) * (int)kstride + 8 * g) * 2;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        kf[kb][kk] = buf_load16(kr, off + 32 * kk, 0);
        vf[kb][kk] = buf_load16(vr, off + 32 * kk, 0);
      }
    }
  }
  f32x16 dk[KB][NDB], dv[KB][NDB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) { dk[kb][db] = agpr_zero(); dv[kb][db] = agpr_zero(); }

  // Steps walk (query head of the group, query block) with the block fastest.
  // Cursors replace a division per step: the issue cursor runs NS - 1 steps
  // ahead of the compute cursor (which only needs the block).
  int i_hq = kvh * p.group, i_m = m_first;   // next step to load
  int c_m = m_first;                          // step being computed
  const int64_t full_bytes = ((int64_t)(BM - 1) * qstride + D) * 2;
  const int64_t last_bytes = ((int64_t)(lq - (nm - 1) * BM - 1) * qstride + D) * 2;
  const int64_t lse_seq = p.sv.cu_q ? qs : (int64_t)t.seq * p.hq * p.sv.seqlen_q;
  const int64_t lse_head = p.sv.cu_q ? p.sv.total_q : p.sv.seqlen_q;
  // Load the step at the issue cursor into ring slot st and advance the
  // cursor. Rows past the sequence read as zero (buffer range), so their P
  // never reaches dK or dV: both products multiply it by a zero row of Q or
  // dO. Their LSE and D are clamped to the last row to stay finite.
  auto issue = [&](int st) {
    const int64_t row0 = (qs + (int64_t)i_m * BM) * qstride + (int64_t)i_hq * D;
    const int64_t bytes = i_m == nm - 1 ? last_bytes : full_bytes;
    const rsrc_t qr = make_rsrc(static_cast<const bf16*>(p.q) + row0, bytes);
    const rsrc_t orr = make_rsrc(static_cast<const bf16*>(p.dout) + row0, bytes);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int base = (i * NW + w) * 64;          // first slot of this wave's 1 KB
      const int slot = base + lane;
      const int r = slot / SPR, pos = slot % SPR;
      const int voff = (r * (int)qstride + (pos ^ dma_swz<D>(r)) * 8) * 2;
      dma16(qr, qtile + st * TILE + base * 16, voff);
      dma16(orr, otile + st * TILE + base * 16, voff);
    }
    if (w < NLD) {
      const int idx = 64 * w + lane;                // [LSE * log2 e rows | D rows]
      const bool is_l = idx < BM;
      const int r = imin(i_m * BM + (idx & (BM - 1)), lq - 1);
      const int64_t so = lse_seq + (int64_t)i_hq * lse_head + r;
      dma4(is_l ? p.lse2 + so : p.dsum + so, lsed + st * 2 * BM + 64 * w);
    }
    if (++i_m == nm) { i_m = m_first; ++i_hq; }
  };
  // wait until the loads of the next step are in LDS (those of later steps may
  // still be in flight), then make them visible to the workgroup
  auto wait_next = [&](bool later_issued) {
    if (later_issued) {
      if (w < NLD) wait_vm<OPS + 1>(); else wait_vm<OPS>();
    } else {
      wait_vm<0>();
    }
    __builtin_amdgcn_s_barrier();
  };

  // per-lane LDS addresses (byte offsets; see dma_swz)
  // A of S and dP: row c, logical chunk 2kk + g  ->  (a_rm ^ 32 kk)
  const int a_rm = c * RB + 16 * (g ^ dma_swz<D>(c));
  // A of dV^T and dK^T by transposing reads: 16-lane group (g, dh), lane s16
  // reads row 4g + s16/4 (+8 for k slots 4..7), columns 32db + 16dh + 4(s16%4)
  const int s16 = lane & 15, dh = (lane >> 4) & 1;
  const int rq = 4 * g + (s16 >> 2);
  const int cl = 2 * dh + ((s16 & 3) >> 1);
  // Row rq + 8 has dma_swz(rq) ^ 2 (rq < 8), so the k slots 4..7 read at
  // (a_t ^ 32) + 8 RB.
  const int a_t = rq * RB + 16 * (cl ^ dma_swz<D>(rq)) + 8 * (s16 & 1);
  // Absolute LDS addresses of the Q tile of the current ring slot (dO at
  // + NS * TILE): ar[kk] for the S / dP operands, at[db][h] for the two
  // transposing reads. They move by one slot per step; slot offsets are
  // multiples of TILE, above every bit the XORs touch.
  const uint32_t lds_q = lds_addr(qtile), lds_l = lds_addr(lsed);
  uint32_t ar[KS], at[NDB][2];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) ar[kk] = lds_q + (a_rm ^ (32 * kk));
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    at[db][0] = lds_q + (a_t ^ (64 * db));
    at[db][1] = lds_q + (a_t ^ (64 * db + 32)) + 8 * RB;
  }
  uint32_t al = lds_l + 16 * g;   // LSE / D of rows 4g .. 4g+3 of the slot
  auto advance_slot = [&](int st) {
    const int dq = st == NS - 1 ? -(NS - 1) * TILE : TILE;
    const int dl = st == NS - 1 ? -(NS - 1) * 2 * BM * 4 : 2 * BM * 4;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) ar[kk] += dq;
#pragma unroll
    for (int db = 0; db < NDB; ++db) { at[db][0] += dq; at[db][1] += dq; }
    al += dl;
  };
  static_assert(TILE % 8192 == 0 || TILE >= 2 * RB * 32, "slot offsets clear the XOR bits");

  // One step on ring slot st for query block mq0. Masking (causal diagonal,
  // key tail) is one compare and one select per element: register i of a
  // tile is query row mq0 + 32 qb + 8 (i / 4) + 4 g + i % 4, so with
  // rel = key - mq0 - 4g the pair is hidden iff rel > 32 qb + 8 (i / 4) + i % 4
  // (rel = INT_MAX for keys past the sequence, -1 where nothing is hidden).
  // A second, unmasked copy of the body would split the AGPR accumulators
  // over two paths, which the register allocator answers with spills.
  auto step_body = [&](int mq0, bool need_mask) {
    constexpr int OT = NS * TILE;   // dO tile offset from the Q tile
    int rel[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = wk0 + 32 * kb + c;
      rel[kb] = !need_mask ? -1 : key >= lk ? 0x7fffffff : (causal ? key - mq0 - 4 * g : -1);
    }
    // The step runs in phases (S, P, dV, dP, dS, dK) fenced against the
    // scheduler so that at most two 32 x 32 fp32 tiles per key block are
    // live next to the resident K and V fragments.
    // ---- S = Q K^T (query on the register, key on the lane)
    f32x16 s[NQB][KB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const bf16x8 aq = lds_ld16(ar[kk] + qb * 32 * RB);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[qb][kb] = mfma32(aq, kf[kb][kk], s[qb][kb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- P = 2^(S scale log2 e - LSE log2 e), masked on the exponent
    bf16x8 pb[NQB][KB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 l4 = lds_ldf4(al + 4 * (qb * 32 + 8 * j));
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = __builtin_fmaf(s[qb][kb][4 * j + r], sl2, -l4[r]);
            s[qb][kb][4 * j + r] = fast_exp2(rel[kb] > qb * 32 + 8 * j + r ? neg_inf() : x);
          }
      }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) pb[qb][kb][tt] = pack_half(s[qb][kb], tt);
    __builtin_amdgcn_sched_barrier(0);
    // ---- dV^T += dO^T P over every 32-dim block (A by transposing reads)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int toff = (qb * 32 + 16 * tt) * RB;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 ao = cat8(ds_read_tr(at[db][0] + OT + toff), ds_read_tr(at[db][1] + OT + toff));
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) mfma32_agpr(dv[kb][db], ao, pb[qb][kb][tt]);
        }
      }
    __builtin_amdgcn_sched_barrier(0);
    // ---- dP = dO V^T
    f32x16 dp[NQB][KB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) dp[qb][kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const bf16x8 ao = lds_ld16(ar[kk] + OT + qb * 32 * RB);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) dp[qb][kb] = mfma32(ao, vf[kb][kk], dp[qb][kb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- dS = P o (dP - D)
    bf16x8 sb[NQB][KB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 d4 = lds_ldf4(al + 4 * (BM + qb * 32 + 8 * j));
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            dp[qb][kb][4 * j + r] = s[qb][kb][4 * j + r] * (dp[qb][kb][4 * j + r] - d4[r]);
      }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) sb[qb][kb][tt] = pack_half(dp[qb][kb], tt);
    __builtin_amdgcn_sched_barrier(0);
    // ---- dK^T += Q^T dS
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int toff = (qb * 32 + 16 * tt) * RB;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 aq = cat8(ds_read_tr(at[db][0] + toff), ds_read_tr(at[db][1] + toff));
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) mfma32_agpr(dk[kb][db], aq, sb[qb][kb][tt]);
        }
      }
  };

  // ---- prologue: fill NS - 1 ring slots
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < n_steps) issue(s);
  if (n_steps > 0) wait_next(n_steps > 1);

  for (int step = 0; step < n_steps; ++step) {
    const int st = step % NS;
    if (step + NS - 1 < n_steps) issue((step + NS - 1) % NS);
    const int mq0 = c_m * BM;
    if (++c_m == nm) c_m = m_first;
    // whole wave above the diagonal: no visible pair in this step
    const bool active = !(causal && wk0 > mq0 + BM - 1);
    const bool need_mask = (wk0 + KPW > lk) || (causal && wk0 + KPW - 1 > mq0);
    if (active) step_body(mq0, need_mask);
    advance_slot(st);
    if (step + 1 < n_steps) wait_next(step + NS - 1 < n_steps);
  }

  // ---- dK = alpha dK^T, dV = dV^T for this wave's keys
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) { agpr_fence(dk[kb][db]); agpr_fence(dv[kb][db]); }
  const float a = p.alpha;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = wk0 + 32 * kb + c;
    if (key < lk) {
      const int64_t ro = (ks0 + key) * kstride + (int64_t)kvh * D + 4 * g;
      bf16* dkp = static_cast<bf16*>(p.dk) + ro;
      bf16* dvp = static_cast<bf16*>(p.dv) + ro;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16& x = dk[kb][db];
          const f32x16& y = dv[kb][db];
          *reinterpret_cast<bf16x4*>(dkp + db * 32 + 8 * j) =
              pack4(x[4 * j] * a, x[4 * j + 1] * a, x[4 * j + 2] * a, x[4 * j + 3] * a);
          *reinterpret_cast<bf16x4*>(dvp + db * 32 + 8 * j) =
              pack4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
        }
    }
  }
}

template <int D>
hipError_t launch_dkdv_d(const BwdParams& p, int grid, hipStream_t stream) {
  using C = DkdvCfg<D>;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, C::KB, C::BM>), dim3(grid), dim3(256), 0, stream, p);
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
