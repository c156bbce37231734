// dQ of the attention backward from the dS the dK/dV kernel stored.
//
// dQ_i = alpha * sum_j dS_ij k_j (FlashAttention-4 blog page, backward
// section: dQ is the product of dS with the key block). The dK/dV kernel
// already forms every dS_ij in bf16 for its dK product; with the stored-dS
// option it writes them out (2 bytes per visible pair), and this kernel runs
// dQ as a single GEMM over them instead of recomputing S, P and dP (two more
// GEMMs and the exponentials). It is bound by the dS stream from HBM: 2 bytes
// per pair against 2 d flops.
//
// Per workgroup: NW wavefronts x 32 query rows of one (sequence, query head).
// Per key tile of BN keys, the K tile (row-major, XOR row swizzle dma_swz)
// streams into a three-deep LDS ring and each wave's own BN x 32 block of dS
// into an NSD-deep one, both by direct global->LDS loads (dS NSD - 1 tiles
// ahead: the HBM latency needs ~100 KiB of it in flight per CU, K comes from
// L2 and needs only two tiles). Both MFMA operands of
// dQ^T += K^T dS^T come from transposing LDS reads (ds_read_b64_tr_b16): K^T
// from the K tile as in bwd_dq.hip, dS^T from the stored sub-tiles, whose
// 8-byte chunks hold four queries of one key. dQ is written once, in bf16, so
// the result is bit-reproducible.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "schedule.hpp"

namespace attn71 {

namespace {

// LDS of one workgroup: [3] K tiles | [NSD][NW] per-wave dS blocks
template <int D>
constexpr int dqds_smem_bytes() {
  using C = DqDsCfg<D>;
  return 3 * C::BN * 2 * D + C::NSD * C::NW * C::BN * 64;
}

// One tile: query block t.block of (sequence t.seq, query head t.head).
template <int D>
__device__ __forceinline__ void dqds_tile(const BwdParams& p, const Tile& t, char* smem) {
  using C = DqDsCfg<D>;
  constexpr int NW = C::NW, NT = NW * 64, BM = C::BM, BN = C::BN;
  constexpr int NKB = BN / 32;          // 32-key sub-tiles per key tile
  constexpr int NDB = D / 32;           // 32-dim blocks of dQ^T
  constexpr int RB = 2 * D;             // bytes per K row
  constexpr int SPR = D / 8;            // 16-byte slots per K row
  constexpr int TILE = BN * RB;         // bytes of one K tile
  constexpr int DSW = BN * 64;          // bytes of one wave's dS block (32 queries x BN keys)
  constexpr int NS = 3;                 // K ring depth
  static_assert(NS == 3, "K loads run two tiles ahead");
  constexpr int NSD = C::NSD;           // dS ring depth
  static_assert(NSD >= 4, "dS loads run at least as far ahead as the K loads");
  constexpr int CH = TILE / (16 * NT);  // K dma16 per thread per tile
  constexpr int CD = DSW / 1024;        // dS dma16 per wave per tile
  static_assert(CH * 16 * NT == TILE && CD * 1024 == DSW, "tile split over the workgroup");
  static_assert(2 * CD + CH < 64 && (NSD - 1) * CD + 2 * CH < 64, "vmcnt range");
  static_assert(dqds_smem_bytes<D>() == NS * TILE + NSD * NW * DSW, "LDS layout");
  const uint32_t lds_k = lds_addr(smem);
  const uint32_t lds_s = lds_k + NS * TILE;

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

  // ---- K ring (as in bwd_dq.hip): keys past the sequence read as zero
  const int64_t kv_bytes = ((int64_t)(lk - 1) * kstride + D) * 2;
  const bf16* kbase = static_cast<const bf16*>(p.k) + ks0 * kstride + (int64_t)kvh * D;
  int voffs[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int slot = (i * NW + w) * 64 + lane;
    const int r = slot / SPR, pos = slot % SPR;
    voffs[i] = (r * (int)kstride + (pos ^ dma_swz<D>(r)) * 8) * 2;
  }
  // ---- this wave's dS: sub-row qw0 / 32 of the head's region (DsGeom,
  // key-block major), NKB sub-tiles (contiguous, 2 KiB each) per key tile.
  // Each 256-key block's column starts at its own base; key tiles are issued
  // in order, so a cursor (block ds_cb, its first sub-tile ds_cs) walks the
  // columns. Reads of sub-rows the block never stored (above its first
  // written row: sub-tiles no row of this wave sees), of rows past the
  // sequence, and of a packed sequence whose regions did not fit give zero.
  const DsGeom dsg = ds_geom(lq, lk, causal);
  const int ds_r = qw0 >> 5;
  const int64_t ds_first = p.ds_prefix ? p.ds_prefix[t.seq]
                                       : (int64_t)t.seq * p.hq * ds_region_tiles(dsg);
  const bool ds_ok = ds_first >= 0 && ds_r < dsg.rows;
  const int64_t ds_head = ds_ok ? ds_first + (int64_t)h * ds_region_tiles(dsg) : 0;
  int ds_cb = 0;
  int64_t ds_cs = 0;
  const int ds_row = lane * 16;
  auto issue_k = [&](int n) {
    const int64_t t0 = (int64_t)n * BN * kstride;
    const rsrc_t kr = make_rsrc(kbase + t0, kv_bytes - 2 * t0);
    const int st = n % NS;
#pragma unroll
    for (int i = 0; i < CH; ++i) dma16(kr, lds_k + st * TILE + (i * NW + w) * 1024, voffs[i]);
  };
  auto issue_ds = [&](int n) {   // n = the previous call's n + 1 (or 0 first)
    const int sd = n % NSD;
    const int k0 = n * NKB, b = k0 >> 3;
    while (ds_cb < b) {
      ds_cs += 8ll * (dsg.rows - ds_r0(dsg, ds_cb));
      ++ds_cb;
    }
    const int r0 = ds_r0(dsg, b);
    const bool live = ds_ok && ds_r >= r0;
    const int64_t base = live ? (ds_head + ds_cs + 8ll * (ds_r - r0)) * 2048 : 0;
    const rsrc_t dsr = raw_rsrc(p.ds + uniform64(base), __builtin_amdgcn_readfirstlane(live ? 16384 : 0));
#pragma unroll
    for (int i = 0; i < CD; ++i)
      dma16_nt(dsr, lds_s + (sd * NW + w) * DSW + i * 1024, ds_row + (k0 & 7) * 2048 + i * 1024);
  };

  // K^T by transposing reads (see bwd_dq.hip): 16-lane group (g, dh), lane
  // s16 reads key row 4g + s16/4 (+8 for k slots 4..7), dims 32db + 16dh +
  // 4(s16%4).
  const int s16 = lane & 15, dh = (lane >> 4) & 1;
  const int rq = 4 * g + (s16 >> 2);
  const int cl = 2 * dh + ((s16 & 3) >> 1);
  const int a_t = rq * RB + 16 * (cl ^ dma_swz<D>(rq)) + 8 * (s16 & 1);
  uint32_t at[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    at[db][0] = lds_k + (a_t ^ (64 * db));
    at[db][1] = lds_k + (a_t ^ (64 * db + 32)) + 8 * RB;
  }
  // dS^T by transposing reads. In a stored sub-tile, 16-row half tt' holds at
  // 16-byte slot L ^ (4 (L >= 32)) ^ (8 tt') the chunks (queries 16tt' + 4g' +
  // 0..3, then + 8) of key c' for lane L = c' + 32g'. The B operand wants, in
  // lane (query 16dh + s16, g), keys 16tt + 4g + j (slots 0..3) and 16tt + 8 +
  // 4g + j (slots 4..7), the k order of K^T above. So lane s16 of the group
  // points at the chunk of key 16tt + 8hh + 4g + s16/4 and queries 16dh +
  // 4(s16%4) .. +3: tt' = dh, chunk (s16 >> 1) & 1, g' = s16 & 1. Per 16-lane
  // group the 16 chunks cover one 128-byte bank window, and the groups dh = 0
  // and 1, which the transposing read services together, cover the two
  // halves of a 256-byte bank line (the ^ 8 of half tt' = 1). The key group
  // hh is slot bit 3 as well: bt reads hh = 0, bt ^ 128 reads hh = 1 (the
  // region's base is 1 KiB aligned).
  const int sl = s16 & 1;
  const int b_t = dh * 1024 + (32 * sl + ((4 * g + (s16 >> 2)) ^ (4 * sl)) + 8 * dh) * 16 +
                  ((s16 >> 1) & 1) * 8;
  const uint32_t bt = lds_s + w * DSW + b_t, bt1 = bt ^ 128;

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  // Key tile in K ring slot st and dS ring slot sd, its first NV sub-tiles
  // (the visible ones): NV * 2 * NDB MFMAs x = ((sub-tile kb, 16-key half tt),
  // dim block db). Operands stream ahead of use (LDS reads return in order):
  // K^T two MFMAs ahead, dS^T one (kb, tt) group ahead, so each MFMA waits
  // only for reads issued two MFMAs earlier.
  auto body = [&](int st, int sd, auto nv) {
    constexpr int NV = decltype(nv)::value;
    constexpr int NX = NV * 2 * NDB;
    const uint32_t ko = st * TILE, so = sd * NW * DSW;
    auto fetch_a = [&](int x) -> bf16x8 {   // K^T of MFMA x
      const int y = x / NDB, db = x % NDB;
      const uint32_t off = ko + ((y >> 1) * 32 + 16 * (y & 1)) * RB;
      return cat8(ds_read_tr(at[db][0] + off), ds_read_tr(at[db][1] + off));
    };
    auto fetch_b = [&](int y) -> bf16x8 {   // dS^T of group y = 2 kb + tt
      const uint32_t bo = so + (y >> 1) * 2048 + 256 * (y & 1);
      return cat8(ds_read_tr(bt + bo), ds_read_tr(bt1 + bo));
    };
    bf16x8 b = fetch_b(0), bn = b;
    bf16x8 a0 = fetch_a(0), a1 = fetch_a(1);
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int y = x / NDB, db = x % NDB;
      const bf16x8 a = a0;
      a0 = a1;
      if (x + 2 < NX) a1 = fetch_a(x + 2);
      if (db == 0 && y + 1 < 2 * NV) bn = fetch_b(y + 1);
      acc[db] = mfma32(a, b, acc[db]);
      __builtin_amdgcn_sched_barrier(0);
      if (db == NDB - 1) b = bn;
    }
  };
  // ---- prologue, in issue order: dS of tiles 0 .. NSD - 2, K of tiles 0
  // and 1; wait for K of tile 0 (and so for everything issued before it).
  // Loads complete in order, so "K of tile n + 1 done" also covers its dS,
  // which went out earlier.
#pragma unroll
  for (int n = 0; n < NSD - 1; ++n)
    if (n < n_tiles) issue_ds(n);
#pragma unroll
  for (int n = 0; n < NS - 1; ++n)
    if (n < n_tiles) issue_k(n);
  if (n_tiles > 1) wait_vm<CH>(); else wait_vm<0>();
  __builtin_amdgcn_s_barrier();

  const bool rows_live = qw0 < lq;
  for (int n = 0; n < n_tiles; ++n) {
    const int st = n % NS, sd = n % NSD;
    // K of tile n + 2 into the slot of tile n - 1, dS of n + NSD - 1 likewise
    // (every wave is past tile n - 1: the barrier that ended it)
    const bool more_k = n + NS - 1 < n_tiles, more_ds = n + NSD - 1 < n_tiles;
    if (more_k) issue_k(n + NS - 1);
    if (more_ds) issue_ds(n + NSD - 1);
    const int k0 = n * BN;
    // sub-tiles with a visible pair for some row of this wave (the dK/dV
    // kernel wrote exactly those; the rest of the tile is never read)
    const int lim = causal ? qw0 + 31 + shift - k0 : BN - 1;
    const int nv = !rows_live || lim < 0 ? 0 : imin(lim / 32 + 1, NKB);
    if (nv == NKB) body(st, sd, std::integral_constant<int, NKB>{});
    else if constexpr (NKB > 1) {
      if (nv == 1) body(st, sd, std::integral_constant<int, 1>{});
    }
    // K (and dS) of tile n + 1 complete in every wave before any reads them.
    // Issued after K of tile n + 1: at n = 0 only this tile's loads; later
    // also the dS load of the previous tile (its K load came first).
    if (n + 1 < n_tiles) {
      if (more_ds) {
        if (n == 0) wait_vm<CH + CD>(); else wait_vm<CH + 2 * CD>();
      } else {
        wait_vm<0>();
      }
      __builtin_amdgcn_s_barrier();
    }
  }

  // ---- dQ = alpha * dQ^T, bf16, this lane's query row
  if (myq < lq) {
    bf16* dst = static_cast<bf16*>(p.dq) + (qs + myq) * qstride + (int64_t)h * D + 4 * g;
    const float a = p.alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& x = acc[db];
        *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * j) =
            pack4(x[4 * j] * a, x[4 * j + 1] * a, x[4 * j + 2] * a, x[4 * j + 3] * a);
      }
  }
}

// Persistent workgroups walk the query blocks (schedule.hpp: persistent_index).
template <int D>
__global__ __launch_bounds__(DqDsCfg<D>::NW * 64, 1) void bwd_dq_ds_kernel(BwdParams) {
  __shared__ __attribute__((aligned(1024))) char smem[dqds_smem_bytes<D>()];
  __shared__ int ticket;
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
    dqds_tile<D>(p, t, smem);
    __syncthreads();   // the next tile's loads reuse the ring slots
  }
}

template <int D>
hipError_t launch_dq_ds_d(const BwdParams& p, int cus, hipStream_t stream) {
  using C = DqDsCfg<D>;
  static const int occ = resident_per_cu(bwd_dq_ds_kernel<D>, C::NW * 64);
  const int grid = persistent_grid(p.ntiles_dq, cus * occ, p.nxcd);
  hipLaunchKernelGGL((bwd_dq_ds_kernel<D>), dim3(grid), dim3(C::NW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq_ds(const BwdParams& p, int d, int cus, hipStream_t stream) {
  if (!p.ds || (p.sv.cu_q && !p.ds_prefix)) return hipErrorInvalidValue;
  if (p.ntiles_dq <= 0) return hipSuccess;
  switch (d) {
    case 64: return launch_dq_ds_d<64>(p, cus, stream);
    case 128: return launch_dq_ds_d<128>(p, cus, stream);
    case 256: return launch_dq_ds_d<256>(p, cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn71
