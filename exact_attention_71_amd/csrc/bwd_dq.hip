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
// Per workgroup: NW wavefronts x 32 query rows (two per SIMD: one wave's
// MFMAs overlap the other's elementwise work). K and V tiles of BN keys stream
// into a three-deep LDS ring by direct global->LDS loads issued two tiles
// ahead (row-major, XOR row swizzle dma_swz). ds_read_b128 gives the A
// operands of S^T and dP^T; the transposing read ds_read_b64_tr_b16 gives K^T,
// the A operand of dQ^T, from the same K tile.
#include "common.hpp"
#include "kernels.hpp"
#include "schedule.hpp"

namespace attn71 {

namespace {

// LDS of one workgroup: [NS] K tiles | [NS] V tiles
template <int D, int BN>
constexpr int dq_smem_bytes() { return 2 * 3 * BN * 2 * D; }

// One tile: query block t.block of (sequence t.seq, query head t.head).
template <int D, int NW, int BN, bool MASK>
__device__ __forceinline__ void dq_tile(const BwdParams& p, const Tile& t, char* smem,
                                        uint16_t* vis, int* vis_n) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int KS = D / 16;            // k-steps of S^T and dP^T
  constexpr int NKB = BN / 32;          // 32-key blocks per tile
  constexpr int NDB = D / 32;           // 32-dim blocks of dQ^T
  constexpr int RB = 2 * D;             // bytes per tile row
  constexpr int SPR = D / 8;            // 16-byte slots per row
  constexpr int TILE = BN * RB;         // bytes of one K (or V) tile
  constexpr int NS = 3;                 // ring depth
  static_assert(NS == 3, "wait_next() counts at most one later tile in flight");
  constexpr int CH = TILE / (16 * NT);  // dma16 per thread per tile
  static_assert(CH * 16 * NT == TILE, "tile split over the workgroup");
  constexpr int OPS = 2 * CH;           // ring loads per thread per tile (K and V)
  static_assert(OPS < 64, "vmcnt range");
  static_assert(BM == DqCfg<D>::BM && BN == DqCfg<D>::BN, "host and kernel tiling agree");
  static_assert(dq_smem_bytes<D, BN>() == 2 * NS * TILE, "LDS layout");
  const uint32_t lds_k = lds_addr(smem);
  constexpr int VT = NS * TILE;         // V tile offset from the K tile

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
  const int shift = lk - lq;            // causal: row i sees keys j <= i + shift
  const int n_tiles = cdiv(causal ? causal_key_end(m0 + BM, shift, lk) : lk, BN);

  const int tid = tile_tid();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int qw0 = m0 + w * 32;
  const int myq = qw0 + c;
  const int64_t qstride = (int64_t)p.hq * D, kstride = (int64_t)p.hkv * D;
  const float sl2 = p.scale_log2;
  // block mask (MASK): this wave's rows lie in one 128-row block, whose mask
  // row starts at byte mrow of the mask buffer
  const rsrc_t mrs = raw_rsrc(p.mask.mask, MASK ? p.mask.range : 0);
  uint32_t mrow = 0;
  if constexpr (MASK) {
    mrow = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        (int64_t)t.seq * p.mask.sb + (int64_t)h * p.mask.sh + (int64_t)(qw0 / kMaskBlock) * p.mask.nkb));
  }
  // block mask: the key tiles with a set block in some mask row of this
  // workgroup's rows, listed by wave 0 (mask_list_tiles); the loop walks only
  // those, and a wave still skips a listed tile its own rows do not see
  int nv = n_tiles;
  if constexpr (MASK) {
    if (w == 0) {
      const int r0 = m0 / kMaskBlock, r1 = (imin(m0 + BM, lq) - 1) / kMaskBlock;
      const uint32_t mb0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
          (int64_t)t.seq * p.mask.sb + (int64_t)h * p.mask.sh + (int64_t)r0 * p.mask.nkb));
      const int cnt = mask_list_tiles(mrs, mb0, p.mask.nkb, r0, r1, n_tiles, BN, kMaskBlock, vis);
      if (lane == 0) *vis_n = cnt;
    }
    __syncthreads();
    nv = __builtin_amdgcn_readfirstlane(*vis_n);
  }
  auto tile_of = [&](int j) -> int {   // key tile of loop position j
    if constexpr (MASK) return __builtin_amdgcn_readfirstlane(static_cast<int>(vis[j]));
    return j;
  };

  // ---- this lane's query row: Q and dO as B operands, LSE log2 e and D as scalars
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
  float lse2 = __builtin_inff(), ndsum = 0.0f;   // -D; padding rows: P = 0
  if (myq < lq) {
    const int64_t so = p.sv.cu_q ? (int64_t)h * p.sv.total_q + qs + myq
                                 : ((int64_t)t.seq * p.hq + h) * p.sv.seqlen_q + myq;
    lse2 = p.lse2[so];
    ndsum = p.dsum[so];
  }
  // -D of this lane's row in every register of nd16, the dP^T accumulators'
  // starting value, so they end at dP - D and dS = P o (dP - D) is one
  // multiply (32 VALU adds fewer per key tile; at head_dim 64 the 16 registers
  // cost a wave per SIMD of occupancy, three to two, and the kernel still
  // runs 5 % faster)
  f32x16 nd16;
#pragma unroll
  for (int i = 0; i < 16; ++i) nd16[i] = ndsum;

  // ---- K / V ring: tile n into slot n % NS. Keys past the sequence read as
  // zero (buffer range) and are masked below.
  const int64_t kv_bytes = ((int64_t)(lk - 1) * kstride + D) * 2;
  const bf16* kbase = static_cast<const bf16*>(p.k) + ks0 * kstride + (int64_t)kvh * D;
  const bf16* vbase = static_cast<const bf16*>(p.v) + ks0 * kstride + (int64_t)kvh * D;
  int voffs[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int slot = (i * NW + w) * 64 + lane;
    const int r = slot / SPR, pos = slot % SPR;
    voffs[i] = (r * (int)kstride + (pos ^ dma_swz<D>(r)) * 8) * 2;
  }
  auto issue = [&](int j) {   // loop position j into ring slot j % NS
    const int64_t t0 = (int64_t)tile_of(j) * BN * kstride;
    const rsrc_t kr = make_rsrc(kbase + t0, kv_bytes - 2 * t0);
    const rsrc_t vr = make_rsrc(vbase + t0, kv_bytes - 2 * t0);
    const int st = j % NS;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t dst = lds_k + st * TILE + (i * NW + w) * 1024;
      dma16(kr, dst, voffs[i]);
      dma16(vr, dst + VT, voffs[i]);
    }
  };
  auto wait_next = [&](bool later_issued) {
    if (later_issued) wait_vm<OPS>(); else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
  };

  // per-lane LDS addresses of slot 0 (see dma_swz): ar[kk] for the A operands of
  // S^T / dP^T (key row c of each 32-key block, logical chunk 2kk + g), at[db][h]
  // for the transposing reads of K^T (16-lane group (g, dh), lane s16 reads key
  // row 4g + s16/4 (+8 for k slots 4..7), dims 32db + 16dh + 4(s16%4)). Row
  // rq + 8 has dma_swz(rq) ^ 2, so the second read is at (a_t ^ 32) + 8 RB.
  const int a_rm = c * RB + 16 * (g ^ dma_swz<D>(c));
  const int s16 = lane & 15, dh = (lane >> 4) & 1;
  const int rq = 4 * g + (s16 >> 2);
  const int cl = 2 * dh + ((s16 & 3) >> 1);
  const int a_t = rq * RB + 16 * (cl ^ dma_swz<D>(rq)) + 8 * (s16 & 1);
  uint32_t ar[KS], at[NDB][2];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) ar[kk] = lds_k + (a_rm ^ (32 * kk));
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    at[db][0] = lds_k + (a_t ^ (64 * db));
    at[db][1] = lds_k + (a_t ^ (64 * db + 32)) + 8 * RB;
  }
  // UNR: the loop holds one copy of the tile per ring slot, whose reads add
  // the slot's offset from slot 0 as an immediate instead of 16 VALU adds
  // per tile moving the addresses (dQ 0.5-2 % faster); the other form is
  // kept for comparison.
  constexpr bool UNR = true;
  auto advance_slot = [&](int st) {
    const int dq = st == NS - 1 ? -(NS - 1) * TILE : TILE;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) ar[kk] += dq;
#pragma unroll
    for (int db = 0; db < NDB; ++db) { at[db][0] += dq; at[db][1] += dq; }
  };

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};

  // One key tile. Register i of an S^T tile is key k0 + 32 kb + 8 (i / 4) +
  // 4 g + i % 4, so with lim = min(q + shift, lk - 1) - k0 - 4g (q + shift only
  // when causal)
  // the pair is hidden iff 32 kb + 8 (i / 4) + i % 4 > lim. The operands come
  // as one stream of fragments PF ahead of use: NG1 of K (S^T), NG1 of V
  // (dP^T), NG2 of K^T (dQ^T).
  constexpr int NG1 = KS * NKB, NG2 = NKB * 2 * NDB, NF = 2 * NG1 + NG2;
  constexpr int PF = 2;                 // fragments in flight ahead of use
  // slot: Slot<s>, the tile's offset from the addresses' ring slot in slots.
  auto tile_body = [&](auto slot, int k0, bool need_mask) {
    constexpr int SO = decltype(slot)::value * TILE;
    auto fetch = [&](int f) -> bf16x8 {
      if (f < 2 * NG1) {
        const int x = f % NG1, kk = x / NKB, kb = x % NKB;
        return lds_ld16(ar[kk] + SO + (f < NG1 ? 0 : VT) + kb * 32 * RB);
      }
      const int x = f - 2 * NG1;
      const int kb = x / (2 * NDB), tt = (x / NDB) % 2, db = x % NDB;
      const int off = SO + (kb * 32 + 16 * tt) * RB;
      return cat8(ds_read_tr(at[db][0] + off), ds_read_tr(at[db][1] + off));
    };
    f32x16 s[NKB], dp[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) { s[kb] = f32x16{}; dp[kb] = nd16; }
    // Hand schedule (as in the dK/dV kernel): after each dP^T MFMA its slice
    // of P = 2^(S scale log2 e - LSE log2 e); the dS^T = P o (dP^T - D) work in
    // groups of 8 elements (one 16-key half of a 32-key block: the B operand of
    // NDB dQ^T MFMAs), group q + 1 computed between the MFMAs of group q.
    constexpr int PPM = NKB * 16 / NG1;       // P elements per dP^T MFMA
    constexpr int NQG = 2 * NKB;              // dS groups
    constexpr int SPM = 8 / NDB;              // dS elements per dQ^T MFMA
    static_assert(PPM * NG1 == NKB * 16 && SPM * NDB == 8, "even slices");
    auto p_elem = [&](int e) {
      const int kb = e / 16, i = e % 16;
      float pv = fast_exp2(__builtin_fmaf(s[kb][i], sl2, -lse2));
      pin(pv);
      s[kb][i] = pv;
    };
    auto ds_elem = [&](int q, int j) {
      const int kb = q / 2, i = 8 * (q % 2) + j;
      float d = s[kb][i] * dp[kb][i];
      pin(d);
      dp[kb][i] = d;
    };
    bf16x8 dsb = {};
    bf16x8 fq[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) fq[i] = fetch(i);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const bf16x8 cur = fq[0];
#pragma unroll
      for (int i = 0; i + 1 < PF; ++i) fq[i] = fq[i + 1];
      if (f + PF < NF) fq[PF - 1] = fetch(f + PF);
      if (f < NG1) {                                  // S^T = K Q^T
        const int kk = f / NKB, kb = f % NKB;
        s[kb] = mfma32(cur, qf[kk], s[kb]);
        __builtin_amdgcn_sched_barrier(0);
        if (f == NG1 - 1 && need_mask) {
          const int lim = imin(causal ? myq + shift : 0x7fffffff, lk - 1) - k0 - 4 * g;
#pragma unroll
          for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              s[kb2][i] = 32 * kb2 + 8 * (i >> 2) + (i & 3) > lim ? neg_inf() : s[kb2][i];
        }
      } else if (f < 2 * NG1) {                       // dP^T = V dO^T, with P
        const int x = f - NG1, kk = x / NKB, kb = x % NKB;
        dp[kb] = mfma32(cur, df[kk], dp[kb]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < PPM; ++e) p_elem(x * PPM + e);
        __builtin_amdgcn_sched_barrier(0);
        if (x == NG1 - 1) {                           // dS group 0 before its MFMAs
#pragma unroll
          for (int j = 0; j < 8; ++j) ds_elem(0, j);
          dsb = pack_half(dp[0], 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {                                        // dQ^T += K^T dS^T, with dS
        const int x = f - 2 * NG1;
        const int q = x / NDB, db = x % NDB;
        dqacc[db] = mfma32(cur, dsb, dqacc[db]);
        __builtin_amdgcn_sched_barrier(0);
        if (q + 1 < NQG) {
#pragma unroll
          for (int j = 0; j < SPM; ++j) ds_elem(q + 1, db * SPM + j);
          if (db == NDB - 1) dsb = pack_half(dp[(q + 1) / 2], (q + 1) % 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // ---- prologue: fill NS - 1 ring slots. The full wait also retires the Q / dO
  // fragment loads, so the compiler places no wait of its own in the loop
  // (where the ring loads, which it cannot see, would make it stall).
#pragma unroll
  for (int n = 0; n < NS - 1; ++n)
    if (n < nv) issue(n);
  wait_vm<0>();
  __builtin_amdgcn_s_barrier();

  // loop position j; UNR: in ring slot `slot` (= j % NS)
  auto one_tile = [&](auto slot, int j) {
    if (j + NS - 1 < nv) issue(j + NS - 1);
    const int k0 = tile_of(j) * BN;
    // whole wave below the diagonal's start, or a cleared mask block: no
    // visible pair in this tile
    bool active = !(causal && k0 > qw0 + 31 + shift);
    if constexpr (MASK) active = active && mask_set(mrs, mrow + static_cast<uint32_t>(k0 / kMaskBlock));
    const bool need_mask = (k0 + BN > lk) || (causal && k0 + BN - 1 > qw0 + shift);
    if (active) tile_body(slot, k0, need_mask);
    if constexpr (!UNR) advance_slot(j % NS);
    if (j + 1 < nv) wait_next(j + NS - 1 < nv);
  };
  if constexpr (UNR) {
    for (int j = 0; j < nv; j += NS) {
      one_tile(Slot<0>{}, j);
      if (j + 1 < nv) one_tile(Slot<1>{}, j + 1);
      if (j + 2 < nv) one_tile(Slot<2>{}, j + 2);
    }
  } else {
    for (int j = 0; j < nv; ++j) one_tile(Slot<0>{}, j);
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

// Persistent workgroups walk the query blocks (schedule.hpp: persistent_index).
template <int D, int NW, int BN, bool MASK>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_kernel(BwdParams) {
  __shared__ __attribute__((aligned(1024))) char smem[dq_smem_bytes<D, BN>()];
  __shared__ int ticket;
  __shared__ uint16_t vis[MASK ? kMaxMaskTiles : 1];   // block mask: visible key tiles
  __shared__ int vis_n;
  for (int r = 0;; ++r) {
    const BwdParams& p = kernel_args<BwdParams>();
    const int i = next_tile(r, p.ntiles_dq, p.nxcd, p.queue_dq, &ticket);
    if (i < 0) break;
    Tile t;
    if (p.sv.cu_q) {
      t = varlen_tile(i, p.order_dq, p.tile_prefix_dq, p.sv.batch, p.hq, true);
      if (t.seq < 0) {
        if (p.queue_dq) continue;   // a ticket past the last real tile
        break;
      }
    } else {
      t = fwd_tile_fixed(i, p.sv.batch, p.hq, p.nm_dq, p.sec_dq, p.nxcd, p.natural != 0);
    }
    dq_tile<D, NW, BN, MASK>(p, t, smem, vis, &vis_n);
    __syncthreads();   // the next tile's loads reuse the ring slots
  }
}

template <int D, bool MASK>
hipError_t launch_dq_t(const BwdParams& p, int cus, hipStream_t stream) {
  using C = DqCfg<D>;
  static const int occ = resident_per_cu(bwd_dq_kernel<D, C::NW, C::BN, MASK>, C::NW * 64);
  const int grid = persistent_grid(p.ntiles_dq, cus * occ, p.nxcd);
  hipLaunchKernelGGL((bwd_dq_kernel<D, C::NW, C::BN, MASK>), dim3(grid), dim3(C::NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}
template <int D>
hipError_t launch_dq_d(const BwdParams& p, int cus, hipStream_t stream) {
  return p.mask.mask ? launch_dq_t<D, true>(p, cus, stream) : launch_dq_t<D, false>(p, cus, stream);
}

}  // namespace

hipError_t launch_bwd_dq(const BwdParams& p, int d, int cus, hipStream_t stream) {
  if (p.ntiles_dq <= 0) return hipSuccess;
  switch (d) {
    case 64: return launch_dq_d<64>(p, cus, stream);
    case 128: return launch_dq_d<128>(p, cus, stream);
    case 256: return launch_dq_d<256>(p, cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn71
