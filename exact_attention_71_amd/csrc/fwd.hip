// Forward attention kernel for gfx950: O = softmax(alpha Q K^T) V with a
// tiled online softmax, conditional rescaling and a stored LSE.
//
// Method (FlashAttention-4 pages): two GEMMs with a softmax between them
// (blog page, introduction); running row max, rescale of the accumulator only
// when the max jumps by more than tau = log2(256) = 8 (digest page, item 3;
// blog page, forward section equation), decided once per group of rows that
// execute together; final division by the true row sum and optional LSE
// (blog page, correction-warpgroup list).
//
// gfx950 design (our own, not the pages' Blackwell pipeline):
//  * workgroup = 8 wavefronts, two per SIMD (4 at head_dim 256); each wave
//    owns 32*QB query rows and runs both GEMMs on v_mfma_f32_32x32x16_bf16
//    with fp32 accumulation;
//  * S is computed transposed, S^T = K Q^T, so every lane owns one query row
//    (lane % 32) and half of the keys of each 32-key block: the row max needs
//    one exchange with lane ^ 32, the rescale factor is a per-lane scalar, and
//    the accumulator of S^T is already the B operand of O^T = V^T P^T;
//  * K and V tiles stream into an LDS ring (two or three slots) by direct
//    global->LDS loads issued ahead of use, row-major under an XOR row
//    swizzle: ds_read_b128 gives the A operand of S^T (K), and the transposing
//    read ds_read_b64_tr_b16 gives the A operand of O^T += V^T P^T (V^T) with
//    the key order of the S^T accumulator; one barrier per tile;
//  * the rescale decision is one ballot per wavefront (any row over tau);
//  * exp2 runs on v_exp_f32; EMU > 0 moves EMU of every 8 elements to the
//    Cody-Waite + Horner polynomial on the FMA path.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "schedule.hpp"

namespace attn71 {

namespace {

__device__ __forceinline__ void seq_bounds(const SeqView& sv, int seq, int64_t* q0, int* lq,
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

// LDS of one workgroup: [NS] K tiles | [NS] V tiles (three-deep ring when it fits)
template <int D, int BN>
constexpr int fwd_ring_depth() { return (3 * 2 * BN * 2 * D <= 160 * 1024) ? 3 : 2; }
template <int D, int BN>
constexpr int fwd_smem_bytes() { return 2 * fwd_ring_depth<D, BN>() * BN * 2 * D; }

// One tile: query block t.block of (sequence t.seq, query head t.head).
// Tiles follow each other on a workgroup: the K / V ring continues across them
// (key tile n of this tile sits in slot (s0 + n) % NS; s0 is advanced for the
// next tile), and during its last key tile a tile loads the first key tile
// and the Q fragments of `nxt` (when has_nxt), so that the next tile starts
// without waiting for them. `pre` says the previous tile did so for this one;
// the return value says whether this one did for `nxt`.
template <int D, int NW, int QB, int BN, int EMU, bool MASK>
__device__ __forceinline__ bool fwd_tile(const FwdParams& p, const Tile& t, char* smem,
                                         bf16x8 (&qf)[QB][D / 16], int& s0, bool pre,
                                         Tile nxt, bool has_nxt, uint16_t* vis, int* vis_n) {
  // not at head_dim 256, whose scalar registers are already short, and not
  // with a block mask, whose tiles first list their visible key tiles: there
  // every tile starts its ring at slot 0 and loads its own first tiles
  constexpr bool XT = D <= 128 && !MASK;
  if constexpr (!XT) {
    s0 = 0;
    has_nxt = false;
  }
  constexpr int NT = NW * 64;           // threads
  constexpr int BM = NW * 32 * QB;
  constexpr int KS = D / 16;            // MFMA k-steps over the head dim
  constexpr int NKB = BN / 32;          // 32-key blocks per tile
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  constexpr int RB = 2 * D;             // bytes per K / V row in LDS
  constexpr int SPR = D / 8;            // 16-byte slots per row
  constexpr int TILE = BN * RB;         // bytes of one K (or V) tile
  constexpr int NS = fwd_ring_depth<D, BN>();   // ring depth
  constexpr int CH = TILE / (16 * NT);  // dma16 per thread per tile
  static_assert(CH * 16 * NT == TILE, "tile split over the workgroup");
  constexpr int OPS = 2 * CH;           // ring loads per thread per tile (K and V)
  static_assert(OPS < 64, "vmcnt range");
  static_assert(fwd_smem_bytes<D, BN>() == 2 * NS * TILE, "LDS layout");
  const uint32_t lds_k = lds_addr(smem);
  constexpr int VT = NS * TILE;         // V tile offset from the K tile

  int64_t qs, ks0;
  int lq, lk;
  // the tile is wave-uniform (the previous tile carried it); its fields stay in
  // scalar registers for the loads' buffer resources
  seq_bounds(p.sv, __builtin_amdgcn_readfirstlane(t.seq), &qs, &lq, &ks0, &lk);
  const int m0 = __builtin_amdgcn_readfirstlane(t.block) * BM;
  if (m0 >= lq) return false;   // never with pre: the prefetch checks the same bound
  const int h = __builtin_amdgcn_readfirstlane(t.head);
  const int kvh = h / p.group;
  const bool causal = p.causal != 0;
  const int shift = lk - lq;            // causal: row i sees keys j <= i + shift
  const int n_tiles = cdiv(causal ? causal_key_end(m0 + BM, shift, lk) : lk, BN);

  const int tid = tile_tid();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int qw0 = m0 + w * 32 * QB;     // first query row of this wave
  // block mask (MASK): this wave's rows lie in one 128-row block, whose mask
  // row starts at byte mrow of the mask buffer
  const rsrc_t mrs = raw_rsrc(p.mask.mask, MASK ? p.mask.range : 0);
  uint32_t mrow = 0;
  if constexpr (MASK) {
    mrow = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        (int64_t)t.seq * p.mask.sb + (int64_t)h * p.mask.sh + (int64_t)(qw0 / kMaskBlock) * p.mask.nkb));
  }
  // block mask: the key tiles with a set block in some mask row of this
  // workgroup's rows, listed in ascending order by wave 0 (mask_list_tiles);
  // the loop below walks only those. Waves still skip a listed tile whose
  // block their own rows do not see.
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
  // key tile of loop position j (the visible list with a mask)
  auto tile_of = [&](int j) -> int {
    if constexpr (MASK) return __builtin_amdgcn_readfirstlane(static_cast<int>(vis[j]));
    return j;
  };
  const int64_t qstride = (int64_t)p.hq * D, kstride = (int64_t)p.hkv * D;
  const float tau = keep_sgpr(p.tau);
  const bf16* __restrict__ qp = static_cast<const bf16*>(p.q);
  const bf16* __restrict__ kp = static_cast<const bf16*>(p.k);
  const bf16* __restrict__ vp = static_cast<const bf16*>(p.v);

  // ---- Q^T operands: lane holds query row (qb*32 + c), dims 16ks + 8g .. +7,
  // of the query block at row q0_ of head hh_ in the sequence at packed row qs_
  auto load_q = [&](int64_t qs_, int lq_, int hh_, int q0_) {
    const rsrc_t qr = make_rsrc(qp + qs_ * qstride + (int64_t)hh_ * D,
                                ((int64_t)(lq_ - 1) * qstride + D) * 2);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = q0_ + w * 32 * QB + qb * 32 + c;
      const int voff = (row * (int)qstride + 8 * g) * 2;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) qf[qb][kk] = buf_load16(qr, voff + 32 * kk, 0);
    }
  };

  // ---- K / V ring: tile n into slot n % NS, loaded NS - 1 tiles ahead by
  // direct global->LDS loads (row-major, XOR row swizzle dma_swz). Buffers
  // cover exactly this sequence's rows of this KV head: keys past the end
  // read as zero and are masked.
  const int64_t kv_bytes = ((int64_t)(lk - 1) * kstride + D) * 2;
  const bf16* kbase = kp + ks0 * kstride + (int64_t)kvh * D;
  const bf16* vbase = vp + ks0 * kstride + (int64_t)kvh * D;
  int voffs[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int slot = (i * NW + w) * 64 + lane;
    const int r = slot / SPR, pos = slot % SPR;
    voffs[i] = (r * (int)kstride + (pos ^ dma_swz<D>(r)) * 8) * 2;
  }
  // key tile n of the K / V rows at kb_ / vb_ (kvb_ bytes each) into slot st
  auto issue_at = [&](const bf16* kb_, const bf16* vb_, int64_t kvb_, int n, int st) {
    // one resource per tile (scalar math): the range check covers the tail
    const int64_t t0 = (int64_t)n * BN * kstride;
    const rsrc_t kr = make_rsrc(kb_ + t0, kvb_ - 2 * t0);
    const rsrc_t vr = make_rsrc(vb_ + t0, kvb_ - 2 * t0);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t dst = lds_k + st * TILE + (i * NW + w) * 1024;
      dma16(kr, dst, voffs[i]);
      dma16(vr, dst + VT, voffs[i]);
    }
  };
  // loop position j: its key tile into ring slot (s0 + j) % NS
  auto issue = [&](int j) { issue_at(kbase, vbase, kv_bytes, tile_of(j), (s0 + j) % NS); };
  // The next tile: its first key tile goes to slot (s0 + n_tiles) % NS, whose
  // last reader (this tile's key tile n_tiles - NS, or an earlier tile) has
  // passed a workgroup barrier by the start of this tile's last key tile; its
  // Q fragments load into qf after this tile's last S^T product.
  bool nxt_ok = false;
  int nn = 0, nlq = 0, nlk = 0, nm0 = 0, nh = 0;
  int64_t nqs = 0, nks = 0;
  if (has_nxt) {
    // wave-uniform by construction; kept in scalar registers for the loads'
    // buffer resources
    const int nseq = __builtin_amdgcn_readfirstlane(nxt.seq);
    seq_bounds(p.sv, nseq, &nqs, &nlq, &nks, &nlk);
    nm0 = __builtin_amdgcn_readfirstlane(nxt.block) * BM;
    nh = __builtin_amdgcn_readfirstlane(nxt.head);
    nxt_ok = nm0 < nlq;
    if (nxt_ok) nn = cdiv(causal ? causal_key_end(nm0 + BM, nlk - nlq, nlk) : nlk, BN);
  }
  auto prefetch_kv = [&]() {
    if (!nxt_ok || nn == 0) return;
    const int64_t off = nks * kstride + (int64_t)(nh / p.group) * D;
    issue_at(kp + off, vp + off, ((int64_t)(nlk - 1) * kstride + D) * 2, 0, (s0 + n_tiles) % NS);
  };
  // wait until the next tile is in LDS (with NS = 3 the tile after it may
  // still be in flight), then make it visible to the workgroup
  auto wait_next = [&](bool later_issued) {
    if constexpr (NS == 3) {
      if (later_issued) wait_vm<OPS>(); else wait_vm<0>();
    } else {
      (void)later_issued;
      wait_vm<0>();
    }
    __builtin_amdgcn_s_barrier();
  };

  // per-lane LDS addresses in ring slot 0 (see dma_swz): ar[kk] for the A
  // operand of S^T (key row c of each 32-key block, logical chunk 2kk + g),
  // at[db][h] for the transposing reads of V^T (16-lane group (g, dh), lane
  // s16 reads key row 4g + s16/4 (+8 for k slots 4..7), dims
  // 32db + 16dh + 4(s16%4)): the key order matches the registers of the S^T
  // accumulator that become P^T. Row rq + 8 has dma_swz(rq) ^ 2.
  const int a_rm = c * RB + 16 * (g ^ dma_swz<D>(c));
  const int s16 = lane & 15, dh = (lane >> 4) & 1;
  const int rq = 4 * g + (s16 >> 2);
  const int cl = 2 * dh + ((s16 & 3) >> 1);
  const int a_t = rq * RB + 16 * (cl ^ dma_swz<D>(rq)) + 8 * (s16 & 1);
  // The addresses are those of ring slot 0: the key-tile loop holds one copy
  // of the tile per ring slot, whose LDS reads add the slot's offset as an
  // immediate instead of moving the addresses (2 KS VALU adds per tile: the
  // d = 256 forward, one wave per SIMD, 3 % faster, the others 1 %); tiles
  // before the continued ring wraps to slot 0, and the last tile, take their
  // offset at run time. The addresses go through an empty asm so that the
  // compiler keeps them whole: split into a base and a constant, the V tile's
  // offsets of the second slot exceed the 16-bit immediate and cost an add
  // per read.
  uint32_t ar[KS], at[NDB][2];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    ar[kk] = lds_k + (a_rm ^ (32 * kk));
    asm volatile("" : "+v"(ar[kk]));
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    at[db][0] = lds_k + VT + (a_t ^ (64 * db));
    at[db][1] = lds_k + VT + (a_t ^ (64 * db + 32)) + 8 * RB;
    asm volatile("" : "+v"(at[db][0]), "+v"(at[db][1]));
  }

  f32x16 oacc[QB][NDB];
  float mref[QB], lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mref[qb] = neg_inf();
    lsum[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[qb][db] = f32x16{};
  }
  const float sl2 = p.scale_log2;

  // ---- prologue: Q fragments and NS - 1 ring slots. The full wait also
  // retires the Q loads, so the compiler places no wait of its own in the loop
  // (where the ring loads, which it cannot see, would make it stall). After a
  // prefetch, Q and key tile 0 have landed already (waited for by the previous
  // tile, on every path that issued them).
  if (!pre) {
    load_q(qs, lq, h, m0);
#pragma unroll
    for (int n = 0; n < NS - 1; ++n)
      if (n < nv) issue(n);
    wait_vm<0>();
  } else {
#pragma unroll
    for (int n = 1; n < NS - 1; ++n)
      if (n < nv) issue(n);
  }
  __builtin_amdgcn_s_barrier();

  // key tile n; the last one is a separate copy (LAST) that also loads the
  // next tile's first key tile and Q fragments, so that those loads sit
  // outside the loop and the compiler tracks no loop-carried load
  // so: byte offset of the tile's ring slot from slot 0
  auto k_tile = [&](int j, auto last_c, int so) {
    constexpr bool LAST = decltype(last_c)::value;
    if constexpr (LAST) {
      prefetch_kv();
    } else {
      if (j + NS - 1 < nv) issue(j + NS - 1);
    }
    const int k0 = tile_of(j) * BN;
    bool active = !(causal && k0 > qw0 + 32 * QB - 1 + shift);
    // a cleared mask block: this wave skips the tile (no visible key in it)
    if constexpr (MASK) active = active && mask_set(mrs, mrow + static_cast<uint32_t>(k0 / kMaskBlock));
    f32x16 s[NKB][QB];   // S^T, then P^T in place
    if (active) {
      // S^T = K Q^T for this tile, key block by key block; the mask and the
      // row-max work of block kb run between the MFMAs of block kb + 1
      // (operand fragments streamed two ahead)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
      const bool need_mask = (k0 + BN > lk) || (causal && k0 + BN - 1 > qw0 + shift);
      float mx[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mx[qb] = neg_inf();
      auto kb_max = [&](int kb) {
        if (need_mask) {   // the ragged key tail and the causal diagonal
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int qrow = qw0 + qb * 32 + c;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = k0 + kb * 32 + c_row(i, g);
              const bool hide = key >= lk || (causal && key > qrow + shift);
              s[kb][qb][i] = hide ? neg_inf() : s[kb][qb][i];
            }
          }
        }
        // a depth-3 tree of eight v_max3 per 32-key block (a chain would
        // serialise eight dependent instructions)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const f32x16& v = s[kb][qb];
          const float t0 = max3f(v[0], v[1], v[2]), t1 = max3f(v[3], v[4], v[5]);
          const float t2 = max3f(v[6], v[7], v[8]), t3 = max3f(v[9], v[10], v[11]);
          const float t4 = max3f(v[12], v[13], v[14]);
          mx[qb] = max3f(mx[qb], max3f(t0, t1, t2), max3f(t3, t4, v[15]));
        }
      };
      constexpr int NSF = NKB * KS;                 // S^T MFMA fragments
      auto fetch_s = [&](int y) -> bf16x8 {
        const int kb = y / KS, kk = y % KS;
        return lds_ld16(ar[kk] + so + kb * 32 * RB);
      };
      bf16x8 k0f = fetch_s(0), k1f = fetch_s(1);
#pragma unroll
      for (int y = 0; y < NSF; ++y) {
        const int kb = y / KS, kk = y % KS;
        const bf16x8 a = k0f;
        k0f = k1f;
        if (y + 2 < NSF) k1f = fetch_s(y + 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32(a, qf[qb][kk], s[kb][qb]);
        __builtin_amdgcn_sched_barrier(0);
        if (kb > 0 && kk == 1) {
          kb_max(kb - 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      kb_max(NKB - 1);
      // running max and the per-wavefront rescale decision
      float mnew[QB];
      bool big = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m = fmaxf(mx[qb], xor32(mx[qb]));
        mnew[qb] = fmaxf(mref[qb], m);
        big = big || ((mnew[qb] - mref[qb]) * sl2 > tau);
      }
      if (wave_any(big)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float fac = (mref[qb] == neg_inf()) ? 0.0f : fast_exp2((mref[qb] - mnew[qb]) * sl2);
          lsum[qb] *= fac;
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[qb][db] *= fac;
          mref[qb] = mnew[qb];
        }
      }
    }
    // the last key tile's S^T products were the last reads of qf: the next
    // tile's Q fragments load now, under this tile's PV products
    if constexpr (LAST) {
      if (nxt_ok) load_q(nqs, nlq, nh, nm0);
    }
    if (active) {
      // P = 2^(s*alpha*log2e - m_ref*alpha*log2e), row sums from fp32 p, and
      // O^T += V^T P^T (A of the PV product by transposing reads of V). Hand
      // schedule: the P work of each 16-key half (8 elements) runs between
      // the NDB MFMAs of the previous half, whose V^T fragments stream two
      // ahead; only half 0 is computed up front.
      // row sums in two accumulators (even and odd elements): two short
      // dependency chains instead of one through the whole tile
      float nb[QB], acc[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        nb[qb] = (mref[qb] == neg_inf()) ? 0.0f : -mref[qb] * sl2;
        acc[qb][0] = acc[qb][1] = 0.0f;
      }
      auto p_half = [&](int h, int j0, int nj) {   // elements j0 .. j0+nj-1 of half h
        const int kb = h / 2;
        // the exponentials first, then the sums: no sum reads the result of
        // the exponential just before it (a wait state after v_exp_f32)
#pragma unroll
        for (int j = j0; j < j0 + nj; ++j) {
          const int i = 8 * (h % 2) + j;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const float x = __builtin_fmaf(s[kb][qb][i], sl2, nb[qb]);
            float e = ((i & 7) < EMU) ? emu_exp2(x) : fast_exp2(x);
            pin(e);
            s[kb][qb][i] = e;
          }
        }
#pragma unroll
        for (int j = j0; j < j0 + nj; ++j) {
          const int i = 8 * (h % 2) + j;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[qb][j & 1] += s[kb][qb][i];
        }
      };
      constexpr int NH = 2 * NKB, NPV = NH * NDB;   // halves, PV MFMAs
      constexpr int PE = 8 / NDB;                   // P elements per PV MFMA
      static_assert(PE * NDB == 8, "even P slices");
      auto fetch_pv = [&](int x) -> bf16x8 {
        const int h = x / NDB, db = x % NDB;
        const int off = so + (h / 2 * 32 + 16 * (h % 2)) * RB;
        return cat8(ds_read_tr(at[db][0] + off), ds_read_tr(at[db][1] + off));
      };
      bf16x8 v0 = fetch_pv(0), v1 = fetch_pv(1);
      p_half(0, 0, 8);
      bf16x8 pb[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) pb[qb] = pack_half(s[0][qb], 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int x = 0; x < NPV; ++x) {
        const int h = x / NDB, db = x % NDB;
        const bf16x8 a = v0;
        v0 = v1;
        if (x + 2 < NPV) v1 = fetch_pv(x + 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma32(a, pb[qb], oacc[qb][db]);
        __builtin_amdgcn_sched_barrier(0);
        if (h + 1 < NH) {
          p_half(h + 1, db * PE, PE);
          if (db == NDB - 1) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) pb[qb] = pack_half(s[(h + 1) / 2][qb], (h + 1) % 2);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) lsum[qb] += acc[qb][0] + acc[qb][1];
    }
    if constexpr (!LAST) wait_next(j + NS - 1 < nv);
  };
  static_assert(NS == 2 || NS == 3, "one copy per ring slot");
  int j0 = 0;
  // tiles before the ring wraps to slot 0 (the ring continues from the last tile)
  for (; j0 + 1 < nv && (s0 + j0) % NS != 0; ++j0) k_tile(j0, std::false_type{}, (s0 + j0) % NS * TILE);
  for (int j = j0; j + 1 < nv; j += NS) {   // tiles j .. j + NS - 1 in slots 0 .. NS - 1
    k_tile(j, std::false_type{}, 0);
    if (j + 2 < nv) k_tile(j + 1, std::false_type{}, TILE);
    if constexpr (NS == 3) {
      if (j + 3 < nv) k_tile(j + 2, std::false_type{}, 2 * TILE);
    }
  }
  if (nv > 0) k_tile(nv - 1, std::true_type{}, (s0 + nv - 1) % NS * TILE);
  if (nv == 0) {
    prefetch_kv();
    if (nxt_ok) load_q(nqs, nlq, nh, nm0);
  }
  // the next tile's loads land before this tile's stores queue behind them
  // (the vector memory counter also counts stores), so the next tile's
  // prologue need not wait for either; unconditional, so the compiler sees
  // the Q loads retired on every path
  wait_vm<0>();

  // ---- epilogue: O = O_acc / l (true statistics), LSE = alpha*m + ln(l)
  bf16* __restrict__ op = static_cast<bf16*>(p.o);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lsum[qb] + xor32(lsum[qb]);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const int row = qw0 + qb * 32 + c;
    if (row < lq) {
      bf16* dst = op + (qs + row) * qstride + (int64_t)h * D + 4 * g;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16& x = oacc[qb][db];
          *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * j) =
              pack4(x[4 * j] * inv, x[4 * j + 1] * inv, x[4 * j + 2] * inv, x[4 * j + 3] * inv);
        }
      if (g == 0 && p.lse) {
        const float val = lt > 0.0f ? mref[qb] * p.alpha + fast_log2(lt) * 0.69314718055994531f
                                    : neg_inf();
        const int64_t off = p.sv.cu_q ? (int64_t)h * p.sv.total_q + qs + row
                                      : ((int64_t)t.seq * p.hq + h) * p.sv.seqlen_q + row;
        p.lse[off] = val;
      }
    }
  }
  s0 = XT ? (s0 + nv) % NS : 0;
  return nxt_ok;
}

// Persistent workgroups walk the query blocks (schedule.hpp: persistent_index).
// The next tile is drawn before the current one runs, so that its first loads
// can go out during the current tile's last key tile.
template <int D, int NW, int QB, int BN, int EMU, bool MASK>
__global__ __launch_bounds__(NW * 64, 1) void fwd_kernel(FwdParams) {
  __shared__ __attribute__((aligned(1024))) char smem[fwd_smem_bytes<D, BN>()];
  __shared__ int ticket;
  __shared__ uint16_t vis[MASK ? kMaxMaskTiles : 1];   // block mask: visible key tiles
  __shared__ int vis_n;
  auto draw = [&](int& r, Tile& t) -> bool {   // every thread calls it (barriers)
    for (;;) {
      const FwdParams& p = kernel_args<FwdParams>();
      const int i = next_tile(r++, p.ntiles, p.nxcd, p.queue, &ticket);
      if (i < 0) return false;
      if (p.sv.cu_q) {
        t = varlen_tile(i, p.order, p.tile_prefix, p.sv.batch, p.hq, /*reverse=*/true);
        if (t.seq < 0) {
          if (p.queue) continue;   // a ticket past the last real tile
          return false;
        }
      } else {
        t = fwd_tile_fixed(i, p.sv.batch, p.hq, p.nm, p.sec, p.nxcd, p.natural != 0);
      }
      return true;
    }
  };
  bf16x8 qf[QB][D / 16];
  int r = 0, s0 = 0;
  Tile cur, nxt;
  bool have = draw(r, cur), pre = false;
  while (have) {
    const bool have_next = draw(r, nxt);
    const FwdParams& p = kernel_args<FwdParams>();
    pre = fwd_tile<D, NW, QB, BN, EMU, MASK>(p, cur, smem, qf, s0, pre, nxt, have_next, vis,
                                             &vis_n);
    __syncthreads();   // the next tile's loads reuse the ring slots
    cur = nxt;
    have = have_next;
  }
}

template <int D, int EMU, bool MASK>
hipError_t launch_dm(const FwdParams& p, int cus, hipStream_t stream) {
  using C = FwdCfg<D>;
  static const int occ = resident_per_cu(fwd_kernel<D, C::NW, C::QB, C::BN, EMU, MASK>, C::NW * 64);
  const int grid = persistent_grid(p.ntiles, cus * occ, p.nxcd);
  hipLaunchKernelGGL((fwd_kernel<D, C::NW, C::QB, C::BN, EMU, MASK>), dim3(grid),
                     dim3(C::NW * 64), 0, stream, p);
  return hipGetLastError();
}
// block masks only with every exponential on v_exp_f32 (the host refuses the rest)
template <int D, int EMU>
hipError_t launch_d(const FwdParams& p, int cus, hipStream_t stream) {
  if constexpr (EMU == 0) {
    if (p.mask.mask) return launch_dm<D, 0, true>(p, cus, stream);
  } else {
    if (p.mask.mask) return hipErrorInvalidValue;
  }
  return launch_dm<D, EMU, false>(p, cus, stream);
}

}  // namespace

// exp_emulation: 0 = all exp2 on v_exp_f32; E = 1, 2, 4: E of every 8 on the
// FMA path.
hipError_t launch_fwd(const FwdParams& p, int d, int cus, int exp_emulation, hipStream_t stream) {
  if (p.ntiles <= 0) return hipSuccess;
  switch (d * 8 + exp_emulation) {
#define ATTN71_FWD_CASE(D, E) \
    case D * 8 + E: return launch_d<D, E>(p, cus, stream);
    ATTN71_FWD_CASE(64, 0) ATTN71_FWD_CASE(64, 1) ATTN71_FWD_CASE(64, 2) ATTN71_FWD_CASE(64, 4)
    ATTN71_FWD_CASE(128, 0) ATTN71_FWD_CASE(128, 1) ATTN71_FWD_CASE(128, 2) ATTN71_FWD_CASE(128, 4)
    ATTN71_FWD_CASE(256, 0) ATTN71_FWD_CASE(256, 1) ATTN71_FWD_CASE(256, 2) ATTN71_FWD_CASE(256, 4)
#undef ATTN71_FWD_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn71
