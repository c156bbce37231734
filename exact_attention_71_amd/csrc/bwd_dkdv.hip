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
//
// With DS set the kernel also stores every dS it forms (bf16, the values its
// dK^T product uses) for the dQ kernel of bwd_dq_ds.hip, which then runs
// dQ = alpha dS K as its only GEMM instead of recomputing S and dP.
//
// With DQ set (the fused design, head_dim 64 and 128) the kernel runs the
// fifth GEMM itself, dQ += dS K over all 256 keys of the workgroup, and adds
// the result to the fp32 dQ accumulator once per step: one global reduction
// per 256 keys, where a 128-key workgroup would need two (blog page, 2-CTA
// backward section: dQ as an (M/2, 2N) x (2N, d) product halves the global
// atomic reductions; here one workgroup covers the 2N keys, so no exchange
// between workgroups is needed). Each wave writes its bf16 dS fragments
// into an LDS image in the stored-dS sub-tile layout (two buffers, by step
// parity); after the mid-step barrier wave w forms one 32 x 32 unit of dQ
// (queries x dims) from that image and a row-major K tile held in LDS for
// the whole work tile, both read with transposing reads, interleaved with
// its dK^T MFMAs, then adds it with 16 coalesced fp32 buffer atomics. DQ = 2
// is the deterministic mode (blog page, deterministic-mode section): the key
// blocks of a (query block, query head) add in a fixed order, the last key
// block first; a wavefront waits until every wavefront of the earlier key
// blocks has counted its adds done in the pair's semaphore, and counts its
// own once a later mid-step wait has retired them (two steps on; at the end
// of the work tile, after a full wait).
#include "common.hpp"
#include "kernels.hpp"
#include "schedule.hpp"

namespace attn71 {

namespace {

// LDS of one workgroup: [NS] Q tiles | [NS] dO tiles | [NS][LSE BM | D BM] fp32,
// and with DQ (from a 1 KiB boundary) the K tile | [2] dS images
template <int D, int BM>
constexpr int dkdv_ring_bytes() { return 2 * 3 * BM * 2 * D + 3 * 2 * BM * 4; }
template <int D, int BM, int DQ>
constexpr int dkdv_smem_bytes() {
  return DQ ? (dkdv_ring_bytes<D, BM>() + 1023) / 1024 * 1024 + DkdvCfg<D>::BN * 2 * D +
                  2 * BM * DkdvCfg<D>::BN * 2
            : dkdv_ring_bytes<D, BM>();
}

// Block mask: the (query head h < gs, mask row r0 + rr < r0 + nrows) pairs
// whose byte is set in one of the workgroup's ncols key columns (first byte
// at mb0 + h sh + row nkb), head-major, as h << 16 | rr, written to rows[];
// wave-uniform. Each lane tests one pair per round of 64; a ballot and a
// count of the lower lanes place it. Returns the count; *n_first / *n_last:
// listed pairs in row r0 / in row last_row.
__device__ __forceinline__ int mask_list_rows(rsrc_t r, uint32_t mb0, uint32_t sh, uint32_t nkb,
                                              int gs, int r0, int nrows, int ncols, int last_row,
                                              int* rows, int* n_first, int* n_last) {
  const int lane = static_cast<int>(__lane_id());
  const int total = gs * nrows;
  int base = 0, nf = 0, nl = 0;
  for (int e0 = 0; e0 < total; e0 += 64) {
    const int e = e0 + lane;
    bool v = false;
    int h = 0, rr = 0;
    if (e < total) {
      h = e / nrows;
      rr = e - h * nrows;
      const int off = static_cast<int>(mb0 + h * sh + (r0 + rr) * nkb);
      v = __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0) != 0 ||
          (ncols > 1 && __builtin_amdgcn_raw_buffer_load_b8(r, off + 1, 0, 0) != 0);
    }
    const uint64_t bal = __ballot(v);
    if (v) rows[base + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] = h << 16 | rr;
    base += __builtin_popcountll(bal);
    nf += __builtin_popcountll(__ballot(v && rr == 0));
    nl += __builtin_popcountll(__ballot(v && r0 + rr == last_row));
  }
  *n_first = nf;
  *n_last = nl;
  return base;
}

// One tile: the keys of key block t.block of (sequence t.seq, KV head t.head),
// query heads of part `part` of the group (p.hsplit parts). mrows, mstat: LDS
// for the listed mask pairs (kMaxMaskRows) and their count and steps.
template <int D, int KB, int BM, bool DS, bool MASK, int DQ>
__device__ __forceinline__ void dkdv_tile(const BwdParams& p, const Tile& t, int part, char* smem,
                                          int* mrows, int* mstat) {
  static_assert(!(DS && MASK), "block masks run with the recomputing dQ kernel");
  static_assert(!(DS && DQ), "stored dS feeds the dQ kernel; DQ forms dQ here");
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
  static_assert(NS == 3, "loads run two steps ahead: slot (s + 2) % NS == (s - 1) % NS");
  constexpr int CH = TILE / (16 * NT);  // dma16 per thread per tile
  constexpr int NLD = 2 * BM / 64;      // dma4 (LSE and D) per step, waves 0 .. NLD-1
  static_assert(TILE % (16 * NT) == 0 && NLD <= NW, "tile split over the workgroup");
  constexpr int OPS = 2 * CH;           // dma per step by waves >= NLD (one more below)
  static_assert(OPS + 1 < 64, "vmcnt range");
  static_assert(dkdv_ring_bytes<D, BM>() == 2 * NS * TILE + NS * 2 * BM * 4, "LDS layout");
  char* const qtile = smem;
  float* const lsed = reinterpret_cast<float*>(smem + 2 * NS * TILE);
  // DQ: K tile (BN rows of RB bytes, row swizzle dma_swz) and two dS images
  // of BM x BN bf16: per 32-query block qb, 8 sub-tiles of 32 keys (2 KiB,
  // the stored-dS sub-tile layout) in key order
  constexpr int NKC = BN / 32;          // 32-key sub-columns of the workgroup
  constexpr int KT = BN * RB;           // bytes of the K tile
  constexpr int DSB = BM * BN * 2;      // bytes of one dS image
  constexpr int RING = (dkdv_ring_bytes<D, BM>() + 1023) / 1024 * 1024;
  constexpr int NJQ = BN / 16;          // k-steps of the dQ product
  static_assert(!DQ || (dkdv_smem_bytes<D, BM, DQ>() == RING + KT + 2 * DSB &&
                        NQB * NDB == NW && KT % (16 * NT) == 0),
                "LDS layout; one 32 x 32 dQ unit per wavefront");
  static_assert(BN == DkdvCfg<D>::BN && BM == DkdvCfg<D>::BM, "host and kernel tiling agree");

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

  const int tid = tile_tid();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63, g = lane >> 5, c = lane & 31;
  const bool causal = p.causal != 0;
  const int kvh = t.head;
  const int64_t qstride = (int64_t)p.hq * D, kstride = (int64_t)p.hkv * D;
  const float sl2 = p.scale_log2;
  const int nm = cdiv(lq, BM);
  const int shift = lk - lq;            // causal: row i sees keys j <= i + shift
  const int m_first = causal ? imin(causal_row_begin(n0, shift) / BM, nm) : 0;
  const int per_head = nm - m_first;
  const int gs = p.group / p.hsplit;   // query heads of this part
  int n_steps = gs * per_head;
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

  const uint32_t lds_q = lds_addr(qtile), lds_l = lds_addr(lsed);   // LDS byte addresses
  // Steps walk (query head of the group, query block) with the block fastest.
  // Cursors replace a division per step: the issue cursor runs NS - 1 steps
  // ahead of the compute cursor (which only needs the block).
  int i_m = m_first;                          // next step to load (block of the issue cursor)
  int c_m = m_first;                          // step being computed
  const int64_t lse_seq = p.sv.cu_q ? qs : (int64_t)t.seq * p.hq * p.sv.seqlen_q;
  const int64_t lse_head = p.sv.cu_q ? p.sv.total_q : p.sv.seqlen_q;
  // Addresses of the issue cursor (query block i_m of head kvh0 + i_h) as
  // 32-bit offsets from per-tile bases: a step's loads then cost a few scalar
  // operations (one wave per SIMD issues every instruction of the step
  // itself). Within one sequence the Q / dO byte offsets stay below 2^31.
  const int kvh0 = kvh * p.group + part * gs;   // first query head of the part
  int i_h = 0;
  int c_h = 0;                                  // query head of the compute cursor, from kvh0
  // CMP (block mask, no chain): the cursors walk the listed (query head,
  // mask row) pairs, pair i_e / c_e; dense (more pairs than the list holds):
  // pair e is query head e, all its steps
  constexpr bool CMP = MASK && DQ != 2;
  constexpr int RPB = kMaskBlock / BM;          // query blocks per mask row
  static_assert(kMaskBlock % BM == 0 && (RPB & (RPB - 1)) == 0 && (!MASK || kMaskBlock % KPW == 0),
                "mask rows hold whole steps");
  int i_e = 0, c_e = 0, n_ent = 0, m_row0 = 0;  // m_row0: first query block of the first row
  bool m_dense = true;
  // advance a cursor (pair e, query block m, query head h) by one step
  auto walk = [&](int& e, int& m, int& h) {
    ++m;
    if (m == nm || (!m_dense && (m & (RPB - 1)) == 0)) {
      if (++e < n_ent) {
        if (m_dense) {
          h = e;
          m = m_first;
        } else {
          const int v = __builtin_amdgcn_readfirstlane(mrows[e]);
          h = v >> 16;
          m = imax(m_row0 + (v & 0xffff) * RPB, m_first);
        }
      }
    }
  };
  // Stored dS (DS): sub-tiles of 32 queries x 32 keys per (sequence, query
  // head), 2 KiB each, key-block major (DsGeom: this tile's keys lie in one
  // 256-key block, whose column holds 16 KiB per 32-query sub-row from its
  // first written row on): two 1 KiB fragments (16-row halves tt of the
  // sub-tile), each the 64 lanes' packed B operands of dK^T in lane order,
  // except that lanes 32..63 swap 64-byte halves (slot L ^ 4) and the second
  // fragment swaps 128-byte halves (slot ^ 8): the dQ kernel's transposing
  // reads then cover one 128-byte bank window per 16 lanes (L ^ 4) and, for
  // the 16-lane groups serviced together, the two halves of a 256-byte bank
  // line (^ 8), so they are conflict-free. The column of the
  // compute cursor's head starts at ds_col (ds_rng bytes; 0 for a packed
  // sequence whose regions did not fit the area, which drops its stores);
  // its step's sub-rows at byte ds_soff of it. The regions of the group's
  // heads follow each other (ds_reg bytes each).
  const char* ds_col = nullptr;
  int64_t ds_reg = 0;
  int ds_rng = 0, ds_soff = 0, ds_soff0 = 0, ds_sub = 0;
  if constexpr (DS) {
    const DsGeom dsg = ds_geom(lq, lk, causal);
    const int blk = n0 >> 8, r0 = ds_r0(dsg, blk);
    ds_reg = uniform64(ds_region_tiles(dsg) * 2048);
    ds_soff0 = __builtin_amdgcn_readfirstlane((m_first * BM / 32 - r0) * 16384);
    ds_sub = ((n0 & 255) >> 5) * 2048;   // this workgroup's first sub-column in the block
    const int64_t first = p.ds_prefix ? p.ds_prefix[t.seq] : (int64_t)t.seq * p.hq * ds_region_tiles(dsg);
    ds_rng = first < 0 ? 0 : __builtin_amdgcn_readfirstlane((dsg.rows - r0) * 16384);
    ds_col = keep_sgpr(p.ds + uniform64(first < 0 ? 0 : first * 2048 + (int64_t)kvh0 * ds_reg +
                                                       ds_col_start(dsg, blk) * 2048));
    ds_soff = ds_soff0;
  }
  // block mask (MASK): this wave's keys lie in one 128-key block; the byte of
  // (query head kvh0 + c_h, query block mq0 / 128) sits at
  // m_base + c_h * m_sh + (mq0 / 128) * m_nkb of the mask buffer
  const rsrc_t mrs = raw_rsrc(p.mask.mask, MASK ? p.mask.range : 0);
  uint32_t m_base = 0, m_sh = 0, m_nkb = 0;
  if constexpr (MASK) {
    m_base = keep_sgpr(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        (int64_t)t.seq * p.mask.sb + (int64_t)kvh0 * p.mask.sh + wk0 / kMaskBlock)));
    m_sh = keep_sgpr(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p.mask.sh)));
    m_nkb = keep_sgpr(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p.mask.nkb)));
  }
  const int64_t q_tile = (qs * qstride + (int64_t)kvh0 * D) * 2;
  const char* const q_seq = keep_sgpr(static_cast<const char*>(p.q) + q_tile);
  const char* const do_seq = keep_sgpr(static_cast<const char*>(p.dout) + q_tile);
  const int blk_bytes = BM * (int)qstride * 2;
  const int l_step = (int)lse_head;
  const int n_full = clamp_range(((int64_t)(BM - 1) * qstride + D) * 2);
  const int n_last = clamp_range(((int64_t)(lq - (nm - 1) * BM - 1) * qstride + D) * 2);
  // LSE * log2 e rows then D rows: lane idx of the waves below NLD loads row
  // idx % BM of the block from the array its half names
  const int l_idx = 64 * w + lane;
  const float* const l_src = (l_idx < BM ? static_cast<const float*>(p.lse2)
                                         : static_cast<const float*>(p.dsum)) +
                             lse_seq + (int64_t)kvh0 * lse_head;
  // Load the step at the issue cursor into ring slot st and advance the
  // cursor. Rows past the sequence read as zero (buffer range), so their P
  // never reaches dK or dV: both products multiply it by a zero row of Q or
  // dO. Their LSE and D are clamped to the last row to stay finite.
  auto issue = [&](int st) {
    const int n = i_m == nm - 1 ? n_last : n_full;
    const int q_rel = i_m * blk_bytes + i_h * (2 * D);
    const rsrc_t qr = raw_rsrc(q_seq + q_rel, n);
    const rsrc_t orr = raw_rsrc(do_seq + q_rel, n);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int base = (i * NW + w) * 64;          // first slot of this wave's 1 KB
      const int slot = base + lane;
      const int r = slot / SPR, pos = slot % SPR;
      const int voff = (r * (int)qstride + (pos ^ dma_swz<D>(r)) * 8) * 2;
      dma16(qr, lds_q + st * TILE + base * 16, voff);
      dma16(orr, lds_q + (NS + st) * TILE + base * 16, voff);
    }
    if (w < NLD) {
      const int r = imin(i_m * BM + (l_idx & (BM - 1)), lq - 1);
      dma4(l_src + (i_h * l_step + r), lds_l + (st * 2 * BM + 64 * w) * 4);
    }
    if constexpr (CMP) {
      walk(i_e, i_m, i_h);
    } else if (++i_m == nm) {
      i_m = m_first;
      ++i_h;
    }
  };
  // DQ: the dQ adds of a step go out at its end, after the loads of step + 2,
  // and stay in flight through the next step: vector memory operations
  // retire in issue order, so the mid-step wait for the loads of step + 1
  // leaves the last NAT (the previous step's adds) outstanding.
  constexpr int NAT = DQ ? 16 : 0;
  // DQ = 2: the step's semaphore, the count its turn needs and a snapshot of
  // it read before the previous step's adds (complete at the mid-step wait);
  // the semaphores of the two steps before, whose adds are counted once the
  // wait has retired them (rel_a: adds two steps old, complete at that wait).
  int* sem_cur = nullptr;
  int sem_need = 0, sem_seen = 0;
  int* rel_a = nullptr;
  int* rel_b = nullptr;
  int64_t mb0 = 0;
  if constexpr (DQ == 2) mb0 = p.sv.cu_q ? (int64_t)p.mb_prefix[t.seq] : (int64_t)t.seq * p.nm;
  // Ring order. Step s reads slot s % NS. Between its dV^T and dK^T phases
  // every wave waits for its own loads of step s + 1 (the only ones in flight
  // then) and meets the others at a barrier: after it, slot (s + 1) % NS is
  // complete, and every wave is past step s - 1, so the loads of step s + 2
  // may overwrite slot (s - 1) % NS; they go out during the dK^T phase. The
  // barrier sits under a queue of dK^T MFMAs instead of in front of the next
  // step, and the next step's first fragments are read before that step begins.
  auto mid = [&]() {
    wait_vm<NAT>();
    if constexpr (DQ) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // dS image written
    __builtin_amdgcn_s_barrier();
    if constexpr (DQ == 2) {
      // The adds of two steps back have completed (the wait above retired
      // everything but the previous step's adds: the L2 has acknowledged
      // them), so counting them needs no cache fence: no value of the
      // accumulator is read inside the kernel, and a later key block issues
      // its adds only after it has seen the count.
      if (rel_a && lane == 0)
        __hip_atomic_fetch_add(rel_a, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      rel_a = rel_b;
      // this step's turn: every wavefront of the earlier key blocks counted
      int v = __builtin_amdgcn_readfirstlane(sem_seen), it = 0;
      while (v < sem_need) {
        if (++it > p.spin_limit) {   // bounded: report and stop waiting
          if (lane == 0) atomicOr(p.status, 1);
          break;
        }
        if ((it & 255) == 0 && __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                                   p.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0)
          break;
        __builtin_amdgcn_s_sleep(2);
        v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(sem_cur, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      }
      rel_b = sem_cur;
    }
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
  // Absolute LDS addresses in the Q tile of a ring slot (dO at + NS * TILE):
  // ar[kk] for the S / dP operands, at[db][h] for the two transposing reads.
  // UNR: the step loop holds one copy of the step per ring slot, whose reads
  // add the slot's offset (from slot 0) as an immediate, with no per-step
  // address updates (17 VALU adds fewer per step: dK/dV 2-3 % faster at
  // head_dim 128, with or without a block mask); otherwise the addresses
  // move by one slot per step (the copies would spill registers of the
  // fused-dQ variants inside the step loop; at head_dim 256 the dO tile's
  // offsets in the third slot exceed the 16-bit immediate, and the copies
  // measured 0.5-1 % slower). Slot offsets are multiples of TILE, above
  // every bit the XORs touch.
  constexpr bool UNR = D <= 128 && !DQ;
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

  // ---- DQ: the K tile (once per work tile; keys past the sequence read as
  // zero) and the per-lane addresses of the dQ product. Wave w owns dQ unit
  // (query block qb_w, dims 32 db_w .. +31) of every step.
  const int qb_w = DQ ? w / NDB : 0, db_w = DQ ? w % NDB : 0;
  const uint32_t lds_k = lds_q + RING, lds_s = lds_k + KT;
  if constexpr (DQ) {
    const rsrc_t ktr = make_rsrc(static_cast<const bf16*>(p.k) + (ks0 + n0) * kstride + (int64_t)kvh * D,
                                 ((int64_t)(lk - n0 - 1) * kstride + D) * 2);
#pragma unroll
    for (int i = 0; i < KT / (16 * NT); ++i) {
      const int base = (i * NW + w) * 64;
      const int slot = base + lane;
      const int r = slot / SPR, pos = slot % SPR;
      dma16(ktr, lds_k + base * 16, (r * (int)kstride + (pos ^ dma_swz<D>(r)) * 8) * 2);
    }
  }
  // Per-lane addresses of the dQ path, recomputed where they are used from
  // an opaque lane id (kept live across the step they would cost VGPRs the
  // dP and dV^T phases need). dS image writes: this wave's sub-columns
  // w KB .. w KB + KB - 1, in the stored layout (16-byte slot L ^ 4 (L >= 32)
  // ^ 8 tt in half tt; the image's base is 256-byte aligned, so the slot's
  // bit 3 is address bit 7).
  auto dq_write_addr = [&](uint32_t par) -> uint32_t {
    const int ln = opaque_lane_id();
    return lds_s + par + w * KB * 2048 + ((ln ^ ((ln >> 5) << 2)) << 4);
  };
  // dS as the A operand (query on the lane, keys 4g + j and 8 + 4g + j of a
  // 16-key step): the transposing read of the stored sub-tiles; K as the B
  // operand (dim on the lane, the same keys): transposing reads of the
  // row-major K tile, as for Q^T above.
  auto dq_read_addr = [&](uint32_t par, uint32_t& ra, uint32_t& k0, uint32_t& k1) {
    const int ln = opaque_lane_id();
    const int l16 = ln & 15, lh = (ln >> 4) & 1, lg = ln >> 5, sl = l16 & 1;
    ra = lds_s + par + qb_w * NKC * 2048 + lh * 1024 +
         (32 * sl + ((4 * lg + (l16 >> 2)) ^ (4 * sl)) + 8 * lh) * 16 + ((l16 >> 1) & 1) * 8;
    const int lr = 4 * lg + (l16 >> 2), lc = 2 * lh + ((l16 & 3) >> 1);
    const int lt = lr * RB + 16 * (lc ^ dma_swz<D>(lr)) + 8 * (l16 & 1);
    k0 = lds_k + (lt ^ (64 * db_w));
    k1 = lds_k + (lt ^ (64 * db_w + 32)) + 8 * RB;
  };
  // Fragment j (0 or 1) of a step, the Q operands of its first S MFMAs, from
  // the slot at byte offset so from the addresses' slot.
  auto fetch_first = [&](int j, int so) -> bf16x8 {
    const int kk = j / NQB, qb = j % NQB;
    return lds_ld16(ar[kk] + so + qb * 32 * RB);
  };

  // One step for query block mq0. Masking (causal diagonal, key tail) sets
  // S = -inf in a branch of its own on the steps that need it: register i of a
  // tile is query row mq0 + 32 qb + 8 (i / 4) + 4 g + i % 4, so with
  // rel = key - shift - mq0 - 4g the pair is hidden iff rel > 32 qb + 8 (i / 4) + i % 4
  // (rel = INT_MAX for keys past the sequence, -1 where nothing is hidden).
  // Only S crosses that branch; a second copy of the whole body would split
  // the AGPR accumulators over two paths (the allocator answers with spills).
  // slot: Slot<s>, the step's offset from the addresses' ring slot in slots
  // (UNR: its ring slot; else 0). f0, f1: the first two operand fragments of
  // this step on entry (read by the previous step), of the next step (byte
  // offset nxt from the addresses' slot) on return. has_next: a later step
  // exists (mid-step sync); iss >= 0: the ring slot the loads of step + 2
  // go to. par: byte offset of this step's dS image (DQ); dqa: its dQ unit.
  auto step_body = [&](auto slot, int mq0, bool need_mask, bool hid, bf16x8& f0, bf16x8& f1,
                       bool has_next, int iss, int nxt, uint32_t par, f32x16& dqa) {
    constexpr int SO = decltype(slot)::value * TILE;           // Q tile offset
    constexpr int SL = decltype(slot)::value * 2 * BM * 4;     // LSE / D offset
    constexpr int OT = NS * TILE;   // dO tile offset from the Q tile
    uint32_t dsw = 0, dsr = 0, dk0 = 0, dk1 = 0;   // DQ: dS image and K tile addresses
    int rel[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = wk0 + 32 * kb + c;
      rel[kb] = (hid || key >= lk) ? 0x7fffffff : (causal ? key - shift - mq0 - 4 * g : -1);
    }
    // Hand schedule (one wave per SIMD: nothing else hides this wave's VALU
    // work, and issue is in order). The step reads one stream of LDS operand
    // fragments, two ahead of use: NG1 of Q (S), NG1 of dO (dP), NG2 of dO^T
    // (dV^T), NG2 of Q^T (dK^T). After each dP MFMA comes its slice of the
    // P = exp(...) work and after each dV^T MFMA its slice of dS = P o (dP - D),
    // so that VALU runs while the MFMA executes; sched_barrier pins the order.
    constexpr int NG1 = KS * NQB, NG2 = NQB * 2 * NDB, NF = 2 * NG1 + 2 * NG2;
    constexpr int E = NQB * KB * 16;               // P (or dS) elements per lane
    constexpr int PPM = E / (NG1 * KB);            // P elements per dP MFMA
    constexpr int SPM = E / (NG2 * KB);            // dS elements per dV^T MFMA
    static_assert(PPM * NG1 * KB == E && SPM * NG2 * KB == E, "even slices");
    auto fetch = [&](int f) -> bf16x8 {
      if (f < 2 * NG1) {   // Q (then dO): fragment (kk, qb)
        const int x = f % NG1, kk = x / NQB, qb = x % NQB;
        return lds_ld16(ar[kk] + SO + (f < NG1 ? 0 : OT) + qb * 32 * RB);
      }
      const int x = (f - 2 * NG1) % NG2;           // dO^T (then Q^T): (qb, tt, db)
      const int qb = x / (2 * NDB), tt = (x / NDB) % 2, db = x % NDB;
      const int off = SO + (f < 2 * NG1 + NG2 ? OT : 0) + (qb * 32 + 16 * tt) * RB;
      return cat8(ds_read_tr(at[db][0] + off), ds_read_tr(at[db][1] + off));
    };
    f32x16 s[NQB][KB], dp[NQB][KB];
    bf16x8 pb[NQB][KB][2], sb[NQB][KB][2];
    // The rows' -D (stored negated) is the dP accumulators' starting value, so
    // the accumulator ends at dP - D and dS = P o (dP - D) is one multiply.
    // Register 4j + r of a tile is row 8j + 4g + r of its 32-row block.
    f32x16 nd[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = lds_ldf4(al + SL + 4 * (BM + qb * 32 + 8 * j));
#pragma unroll
        for (int r = 0; r < 4; ++r) nd[qb][4 * j + r] = v[r];
      }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) { s[qb][kb] = f32x16{}; dp[qb][kb] = nd[qb]; }
    // element e of the P / dS pass: (qb, j, kb, r) -> register 4j + r of tile (qb, kb).
    // LSE log2 e comes in blocks of 4 rows (qb, j), read one block ahead: LDS
    // returns in order, so a read issued just before its use would make the
    // wait drain the operand fragments prefetched after it.
    constexpr int NJ = 4 * NQB;
    auto row_read = [&](int b) {   // LSE block b
      return lds_ldf4(al + SL + 4 * ((b / 4) * 32 + 8 * (b % 4)));
    };
    f32x4 rv_cur = {}, rv_next = row_read(0);
    auto row_block = [&](int b) {  // entering block b: rotate and prefetch b + 1
      rv_cur = rv_next;
      if (b + 1 < NJ) rv_next = row_read(b + 1);
    };
    auto p_elem = [&](int e) {
      const int qb = e / (KB * 16), rem = e % (KB * 16);
      const int j = rem / (KB * 4), kb = (rem / 4) % KB, r = rem % 4;
      if (kb == 0 && r == 0) row_block(qb * 4 + j);
      float pv = fast_exp2(__builtin_fmaf(s[qb][kb][4 * j + r], sl2, -rv_cur[r]));
      pin(pv);
      s[qb][kb][4 * j + r] = pv;
      if ((j & 1) && kb == KB - 1 && r == 3) {
#pragma unroll
        for (int k2 = 0; k2 < KB; ++k2) {
          pb[qb][k2][j >> 1] = pack_half(s[qb][k2], j >> 1);
          pin8(pb[qb][k2][j >> 1]);
        }
      }
    };
    auto s_elem = [&](int e) {
      const int qb = e / (KB * 16), rem = e % (KB * 16);
      const int j = rem / (KB * 4), kb = (rem / 4) % KB, r = rem % 4;
      float ds = s[qb][kb][4 * j + r] * dp[qb][kb][4 * j + r];
      pin(ds);
      dp[qb][kb][4 * j + r] = ds;
      if ((j & 1) && kb == KB - 1 && r == 3) {
#pragma unroll
        for (int k2 = 0; k2 < KB; ++k2) {
          sb[qb][k2][j >> 1] = pack_half(dp[qb][k2], j >> 1);
          pin8(sb[qb][k2][j >> 1]);
          if constexpr (DQ)
            lds_st16(((j >> 1) ? (dsw ^ 128) : dsw) + qb * NKC * 2048 + k2 * 2048 + (j >> 1) * 1024,
                     sb[qb][k2][j >> 1]);
        }
      }
    };
    // DQ: operands of dQ k-step jq (keys 16 jq .. +15), read two steps ahead
    constexpr int NQ = NJQ / NG2;                  // dQ MFMAs per dK^T fragment
    static_assert(!DQ || NQ * NG2 == NJQ, "even dQ slices");
    bf16x8 qa[3], qk[3];
    auto dq_fetch = [&](int jq) {
      const int kc = jq >> 1, tt = jq & 1;
      const uint32_t so = kc * 2048 + 256 * tt, ko = (kc * 32 + 16 * tt) * RB;
      qa[jq % 3] = cat8(ds_read_tr(dsr + so), ds_read_tr((dsr ^ 128) + so));
      qk[jq % 3] = cat8(ds_read_tr(dk0 + ko), ds_read_tr(dk1 + ko));
    };
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f == 2 * NG1 + NG2) {                       // dV^T done: sync for step + 1
        mid();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DQ) {
          dq_read_addr(par, dsr, dk0, dk1);
          dq_fetch(0);
          dq_fetch(1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (DQ) {
        if (f == 2 * NG1) dsw = dq_write_addr(par);   // dV^T phase: the dS image writes begin
      }
      const bf16x8 cur = f0;
      f0 = f1;
      f1 = f + 2 < NF ? fetch(f + 2) : fetch_first(f + 2 - NF, nxt);
      if (f < NG1) {                                  // S = Q K^T
        const int kk = f / NQB, qb = f % NQB;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[qb][kb] = mfma32(cur, kf[kb][kk], s[qb][kb]);
        __builtin_amdgcn_sched_barrier(0);
        if (f == NG1 - 1 && need_mask) {   // causal diagonal and key tail: S = -inf
#pragma unroll
          for (int q2 = 0; q2 < NQB; ++q2)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i)
                s[q2][kb][i] = rel[kb] > q2 * 32 + 8 * (i >> 2) + (i & 3) ? neg_inf() : s[q2][kb][i];
        }
      } else if (f < 2 * NG1) {                       // dP = dO V^T, with P
        const int x = f - NG1, kk = x / NQB, qb = x % NQB;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          dp[qb][kb] = mfma32(cur, vf[kb][kk], dp[qb][kb]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int e = 0; e < PPM; ++e) p_elem((x * KB + kb) * PPM + e);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else if (f < 2 * NG1 + NG2) {                 // dV^T += dO^T P, with dS
        const int x = f - 2 * NG1;
        const int qb = x / (2 * NDB), tt = (x / NDB) % 2, db = x % NDB;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          mfma32_agpr<false>(dv[kb][db], cur, pb[qb][kb][tt]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int e = 0; e < SPM; ++e) s_elem((x * KB + kb) * SPM + e);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {                                        // dK^T += Q^T dS
        const int x = f - 2 * NG1 - NG2;
        const int qb = x / (2 * NDB), tt = (x / NDB) % 2, db = x % NDB;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mfma32_agpr<false>(dk[kb][db], cur, sb[qb][kb][tt]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DQ) {   // dQ unit += dS (32 queries x 16 keys) K (16 keys x 32 dims)
#pragma unroll
          for (int e = 0; e < NQ; ++e) {
            const int jq = x * NQ + e;
            dqa = mfma32(qa[jq % 3], qk[jq % 3], jq == 0 ? f32x16{} : dqa);
            if (jq + 2 < NJQ) dq_fetch(jq + 2);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (DS) {
          if (db == NDB - 1) {   // last read of sb[qb][*][tt]: store it (waited for a step later)
            const rsrc_t dr = raw_rsrc(ds_col, ds_rng);
            const int so = ds_soff + ds_sub + (KPW >> 5) * w * 2048;
            // lane offset recomputed here from an opaque lane id: kept live
            // across the step it costs a VGPR
            const int ln = opaque_lane_id();
            const int ds_voff = ((ln ^ ((ln >> 5) << 2)) ^ (8 * tt)) << 4;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
              buf_store16_nt(dr, ds_voff, so + qb * 16384 + kb * 2048 + tt * 1024, sb[qb][kb][tt]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (x == 1 && iss >= 0) {
          issue(UNR ? iss : __builtin_amdgcn_readfirstlane(iss));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // DQ = 2: semaphore and needed count of the step at query block mq0, head
  // kvh0 + hh (the key blocks of the pair add from the last one down)
  auto chain_pos = [&](int mq0, int hh) {
    const int nkb = cdiv(lk, BN);
    const int nlast = causal ? imin(nkb - 1, (mq0 + BM - 1 + shift) / BN) : nkb - 1;
    sem_need = 4 * (nlast - t.block);
    sem_cur = p.sem + (mb0 + mq0 / BM) * p.hq + (kvh0 + hh);
    sem_seen = __hip_atomic_load(sem_cur, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // Block mask without the deterministic chain (whose turns count every key
  // block at every step): the walk visits only the (query head, mask row)
  // pairs where one of the workgroup's mask bytes is set; in a listed row a
  // wave whose own byte is clear still computes, with P = 0 (hid). Pairs in
  // list order; the steps of pair (h, row) are the query blocks of the row
  // from m_first on. More pairs than the list holds: every pair, in order.
  if constexpr (CMP) {
    if (n_steps > 0) {
      const int r0 = m_first / RPB, nmr = cdiv(nm, RPB), nrows = nmr - r0;
      const bool dense = (int64_t)gs * nrows > kMaxMaskRows;
      if (!dense && w == 0) {
        int nf, nl;
        // wave 0's column is the workgroup's first
        const int n = mask_list_rows(mrs, m_base, m_sh, m_nkb,
                                     gs, r0, nrows, (BN > kMaskBlock && n0 + kMaskBlock < lk) ? 2 : 1,
                                     nmr - 1, mrows, &nf, &nl);
        if (lane == 0) {
          mstat[0] = n;
          mstat[1] = RPB * n - nf * (m_first - r0 * RPB) - nl * (nmr * RPB - nm);
        }
      }
      __syncthreads();
      m_dense = dense;
      if (!dense) {
        m_row0 = r0 * RPB;
        n_ent = __builtin_amdgcn_readfirstlane(mstat[0]);
        n_steps = __builtin_amdgcn_readfirstlane(mstat[1]);
        if (n_steps > 0) {
          const int v = __builtin_amdgcn_readfirstlane(mrows[0]);
          i_h = c_h = v >> 16;
          i_m = c_m = imax(m_row0 + (v & 0xffff) * RPB, m_first);
        }
      } else {
        n_ent = gs;   // cursors start at (head 0, m_first) as set above
      }
    }
  }

  // ---- prologue: fill NS - 1 ring slots. The full wait also retires the K / V
  // fragment loads: the compiler then knows them complete and places no wait
  // of its own inside the loop (where the outstanding ring loads, which it
  // cannot see, would make such a wait stall on the prefetch).
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < n_steps) issue(s);
  if constexpr (DQ == 2) {
    if (n_steps > 0) chain_pos(m_first * BM, 0);   // step 0's snapshot, retired below
  }
  wait_vm<0>();
  __builtin_amdgcn_s_barrier();

  bf16x8 f0 = fetch_first(0, 0), f1 = fetch_first(1, 0);
  f32x16 dqa;   // DQ: this wave's dQ unit of the step (formed from zero each step)
  int st = 0;   // !UNR: ring slot of the step being computed (step % NS)
  // step `step`; UNR: in ring slot `slot` (= step % NS)
  auto one_step = [&](auto slot, int step) {
    const int mq0 = c_m * BM;
    const int h_step = c_h;
    bool wrap = false;
    if constexpr (CMP) {
      walk(c_e, c_m, c_h);
    } else {
      wrap = ++c_m == nm;
      if (wrap) c_m = m_first;
    }
    // a cleared mask block hides every pair of this wave's step (P = 0)
    bool hid = false;
    if constexpr (MASK)
      hid = !mask_set(mrs, m_base + h_step * m_sh + static_cast<uint32_t>(mq0 / kMaskBlock) * m_nkb);
    if (wrap) ++c_h;
    const bool has_next = step + 1 < n_steps;
    constexpr int ST = decltype(slot)::value;
    const int is_slot = UNR ? (ST + NS - 1) % NS : (st == 0 ? NS - 1 : st - 1);  // (step + 2) % NS
    const int iss = step + NS - 1 < n_steps ? is_slot : -1;
    // the next step's slot, from the addresses' slot
    const int nxt = UNR ? (ST + 1) % NS * TILE : (st == NS - 1 ? -(NS - 1) * TILE : TILE);
    // A wave whose keys all lie above this block's rows computes the step
    // anyway (masked to zero): skipping it would need a second path around
    // the mid-step barrier, and the register allocator answers such a split
    // of the AGPR accumulators with spills.
    const bool need_mask = hid || (wk0 + KPW > lk) || (causal && wk0 + KPW - 1 > mq0 + shift);
    const uint32_t par = (step & 1) * DSB;   // DQ: dS image of this step
    step_body(slot, mq0, need_mask, hid, f0, f1, has_next, iss, nxt, par, dqa);
    if constexpr (DQ) {
      // rows mq0 + 32 qb_w + 8 (r / 4) + 4 g + r % 4 (register r), dims
      // 32 db_w + c; rows past the sequence fall outside the buffer range
      const int r0 = mq0 + 32 * qb_w;
      const int hh = kvh0 + h_step;
      // the next step's snapshot goes out before these adds (c_m, c_h: the next step)
      if constexpr (DQ == 2) {
        if (has_next) chain_pos(c_m * BM, c_h);
      }
      const rsrc_t ar = raw_rsrc(p.dq_acc + ((qs + r0) * qstride + (int64_t)hh * D + 32 * db_w),
                                 clamp_range(((int64_t)(lq - r0 - 1) * qstride + 32) * 4));
      const int qs4 = (int)qstride * 4;
      const int ln = opaque_lane_id();
      const int dq_lane = ((ln >> 5) * 4 * qs4) + (ln & 31) * 4;   // fp32 offset of (row 4g, dim c)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(dqa[r], ar,
                                                        dq_lane + (8 * (r >> 2) + (r & 3)) * qs4, 0, 0);
    }
    if constexpr (DS) {   // the compute cursor's next sub-rows
      if (wrap) {
        ds_col = keep_sgpr(ds_col + ds_reg);
        ds_soff = ds_soff0;
      } else {
        ds_soff += NQB * 16384;
      }
    }
  };
  if constexpr (UNR) {
    for (int step = 0; step < n_steps; step += NS) {
      one_step(Slot<0>{}, step);
      if (step + 1 < n_steps) one_step(Slot<1>{}, step + 1);
      if (step + 2 < n_steps) one_step(Slot<2>{}, step + 2);
    }
  } else {
    for (int step = 0; step < n_steps; ++step) {
      one_step(Slot<0>{}, step);
      advance_slot(st);
      st = st == NS - 1 ? 0 : st + 1;
    }
  }

  if constexpr (DQ == 2) {   // count the last two steps' adds once they have completed
    wait_vm<0>();
    if (rel_a && lane == 0) __hip_atomic_fetch_add(rel_a, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (rel_b) {
      if (lane == 0) __hip_atomic_fetch_add(rel_b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- dK = alpha dK^T, dV = dV^T for this wave's keys
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) { agpr_fence(dk[kb][db]); agpr_fence(dv[kb][db]); }
  // With a head split: fp32 partials of this part (the reduction scales dK).
  // One loop serves both forms, branching on an opaque copy of the flag per
  // store, so that the compiler keeps a single copy of the loop (two would
  // hold the accumulators in VGPRs for both and spill).
  const float a = p.alpha;
  const bool split = p.hsplit > 1;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = wk0 + 32 * kb + c;
    if (key < lk) {
      const int64_t ro = (ks0 + key) * kstride + (int64_t)kvh * D + 4 * g;
      const int64_t rp = (int64_t)part * p.rows_k * kstride + ro;
      bf16* dkp = static_cast<bf16*>(p.dk) + ro;
      bf16* dvp = static_cast<bf16*>(p.dv) + ro;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16& x = dk[kb][db];
          const f32x16& y = dv[kb][db];
          if (opaque_bool(split)) {
            *reinterpret_cast<f32x4*>(p.dk_part + rp + db * 32 + 8 * j) =
                f32x4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
            *reinterpret_cast<f32x4*>(p.dv_part + rp + db * 32 + 8 * j) =
                f32x4{y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]};
          } else {
            *reinterpret_cast<bf16x4*>(dkp + db * 32 + 8 * j) =
                pack4(x[4 * j] * a, x[4 * j + 1] * a, x[4 * j + 2] * a, x[4 * j + 3] * a);
            *reinterpret_cast<bf16x4*>(dvp + db * 32 + 8 * j) =
                pack4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
          }
        }
    }
  }
}

// Persistent workgroups walk the tiles (schedule.hpp: persistent_index); a
// one-shot grid (gridDim.x == ntiles) gives each workgroup one tile.
template <int D, int KB, int BM, bool DS, bool MASK, int DQ>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams) {
  __shared__ __attribute__((aligned(1024))) char smem[dkdv_smem_bytes<D, BM, DQ>()];
  __shared__ int ticket;
  __shared__ int mrows[MASK && DQ != 2 ? kMaxMaskRows : 1];   // listed mask pairs
  __shared__ int mstat[2];                                     // their count, their steps
  for (int r = 0;; ++r) {
    const BwdParams& p = kernel_args<BwdParams>();
    const int i = next_tile(r, p.ntiles, p.nxcd, p.queue, &ticket);
    if (i < 0) break;
    Tile t;
    int part = 0;
    if (p.sv.cu_q) {
      // head split: ticket = base tile * hsplit + part (the tables count base tiles)
      int ib = i;
      if (p.hsplit > 1) {
        ib = i / p.hsplit;
        part = i - ib * p.hsplit;
      }
      if (DQ != 2 && p.key_tiles && p.key_tiles[0]) {
        // one longest-first list of all key blocks, KV heads innermost
        t.seq = -1;
        if (ib < p.tile_prefix[p.sv.batch]) {
          const int e = ib / p.hkv;
          t.head = ib - e * p.hkv;
          t.seq = __builtin_amdgcn_readfirstlane(p.key_tiles[2 + 2 * e]);
          t.block = __builtin_amdgcn_readfirstlane(p.key_tiles[3 + 2 * e]);
          if ((unsigned)t.seq >= (unsigned)p.sv.batch) t.seq = -1;
        }
      } else {
        // deterministic: shortest first, the order of the chain's turns
        t = varlen_tile(ib, p.order, p.tile_prefix, p.sv.batch, p.hkv, /*reverse=*/DQ == 2);
      }
      if (t.seq < 0) {
        if (p.queue) continue;   // a ticket past the last real tile
        break;
      }
    } else {
      // head split: (KV head, part) pairs are the scheduler's heads
      t = bwd_tile_fixed(i, p.sv.batch, p.hkv * p.hsplit, p.nn, p.sec, DQ == 2, p.nxcd,
                         p.natural != 0);
      if (p.hsplit > 1) {
        const int kv = t.head / p.hsplit;
        part = t.head - kv * p.hsplit;
        t.head = kv;
      }
    }
    dkdv_tile<D, KB, BM, DS, MASK, DQ>(p, t, part, smem, mrows, mstat);
    __syncthreads();   // the next tile's loads reuse the ring slots
  }
}

template <int D, bool DS, bool MASK, int DQ>
hipError_t launch_dkdv_t(const BwdParams& p, int cus, hipStream_t stream) {
  using C = DkdvCfg<D>;
  static const int occ = resident_per_cu(bwd_dkdv_kernel<D, C::KB, C::BM, DS, MASK, DQ>, 256);
  const int grid = persistent_grid(p.ntiles, cus * occ, p.nxcd);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, C::KB, C::BM, DS, MASK, DQ>), dim3(grid), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}
template <int D, int DQ>
hipError_t launch_dkdv_q(const BwdParams& p, int cus, hipStream_t stream) {
  return p.mask.mask ? launch_dkdv_t<D, false, true, DQ>(p, cus, stream)
                     : launch_dkdv_t<D, false, false, DQ>(p, cus, stream);
}
template <int D>
hipError_t launch_dkdv_d(const BwdParams& p, int cus, hipStream_t stream) {
  // the host never combines stored dS with a block mask or the fused dQ
  if (p.ds && (p.mask.mask || p.dq_mode)) return hipErrorInvalidValue;
  if constexpr (D <= 128) {
    if (p.dq_mode == 1) return launch_dkdv_q<D, 1>(p, cus, stream);
    if (p.dq_mode == 2) {
      if (!p.queue) return hipErrorInvalidValue;   // the chain needs tickets in turn order
      return launch_dkdv_q<D, 2>(p, cus, stream);
    }
  } else {
    if (p.dq_mode) return hipErrorInvalidValue;
  }
  if (p.ds) return launch_dkdv_t<D, true, false, 0>(p, cus, stream);
  return launch_dkdv_q<D, 0>(p, cus, stream);
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdParams& p, int d, int cus, hipStream_t stream) {
  if (p.ntiles <= 0) return hipSuccess;
  switch (d) {
    case 64: return launch_dkdv_d<64>(p, cus, stream);
    case 128: return launch_dkdv_d<128>(p, cus, stream);
    case 256: return launch_dkdv_d<256>(p, cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn71
