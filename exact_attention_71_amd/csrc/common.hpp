// Device helpers shared by the gfx950 attention kernels: MFMA fragment types,
// bf16 packing, LDS swizzles, wavefront reductions and the two exp2 paths.
#pragma once

#include <hip/hip_runtime.h>

#include "schedule.hpp"
#include <stdint.h>

namespace attn71 {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// MFMA 32x32x16 bf16 -> fp32.
// Operand layout (lane l, g = l / 32, c = l % 32):
//   A[m][k]: lane holds m = c, k = 8g .. 8g+7
//   B[k][n]: lane holds n = c, k = 8g .. 8g+7
//   C[m][n]: lane holds n = c, register i holds m = 8*(i/4) + 4*g + (i%4)
// Only the C layout is relied on across instructions; A and B use the same
// k slots, so any consistent k-to-slot assignment contracts correctly.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int c_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// The same MFMA with the accumulator pinned to AGPRs, for long-lived
// accumulators in kernels whose VGPRs are full (the compiler's VGPR/AGPR form
// choice is all-or-nothing per function). The compiler does not see hazards
// inside inline asm, so the two cases that apply here are covered by hand:
// an A/B operand written by a VALU instruction needs 2 wait states before an
// MFMA reads it, which WAIT = true provides with s_nop 1, and agpr_fence()
// must separate the last accumulation from any non-MFMA read of the
// accumulator. Back-to-back accumulation into the same registers needs no
// wait states. WAIT = false is for hand-scheduled call sites whose operands
// come from LDS reads or from VALU work issued well before; the
// tests/test_isa_hazards.py scan of the compiled code checks every such MFMA
// for a VALU write of its operands in the 2 wait states before it.
template <bool WAIT = true>
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (WAIT)
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Keeps a value's computation where it stands in the source: sched_barrier
// only orders instructions with side effects, so pure VALU results would
// otherwise be placed next to their (later) uses by instruction selection.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
// The same for a packed MFMA operand: formed here, not sunk next to its use
// (where it would also sit inside the hazard window of an inline-asm MFMA).
__device__ __forceinline__ void pin8(bf16x8& x) { asm volatile("" : "+v"(x)); }

// Zero accumulator defined directly in AGPRs (an MFMA of zero operands with
// C = 0), so a loop-carried accumulator never has a VGPR definition. The
// zero operand is written by VALU just before, hence the same s_nop 1.
__device__ __forceinline__ f32x16 agpr_zero() {
  f32x16 acc;
  const bf16x8 z = {};
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
  return acc;
}

// 16 wait states between the last MFMA that wrote acc and the reads after it
// (the compiler itself places 11 to 12 after this MFMA before a VALU read).
__device__ __forceinline__ void agpr_fence(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+a"(acc));
}

// Eight fp32 -> eight bf16 (round to nearest even) as one MFMA operand.
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4,
                                        float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
  r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
  return r;
}

// C registers 8t .. 8t+7 of a 32x32 accumulator as a bf16 operand.
__device__ __forceinline__ bf16x8 pack_half(const f32x16& x, int t) {
  return pack8(x[8 * t + 0], x[8 * t + 1], x[8 * t + 2], x[8 * t + 3], x[8 * t + 4],
               x[8 * t + 5], x[8 * t + 6], x[8 * t + 7]);
}

__device__ __forceinline__ bf16x4 pack4(float a0, float a1, float a2, float a3) {
  bf16x4 r;
  r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
  return r;
}

// ---------------------------------------------------------------------------
// LDS layouts.
// Row-major tiles [rows][D] of bf16 are stored in 16-byte slots. Slot ch of
// row r goes to slot ch ^ swz(r), chosen so that 16 consecutive rows read at
// the same logical slot land in 16 distinct 16-byte bank groups of a 256-byte
// bank line (and 8 consecutive rows in 8 distinct groups of a 128-byte line).
// ---------------------------------------------------------------------------
template <int ROW_ELEMS>
__device__ __forceinline__ int swz_slot(int row, int ch) {
  if constexpr (ROW_ELEMS * 2 >= 256) {
    return ch ^ (row & 15);
  } else if constexpr (ROW_ELEMS * 2 == 128) {
    return ch ^ ((row >> 1) & 7);
  } else {  // 64-byte rows
    return ch ^ ((row >> 2) & 3);
  }
}

// element offset of (row, 8-element chunk ch) in a swizzled [rows][ROW_ELEMS] tile
template <int ROW_ELEMS>
__device__ __forceinline__ int swz_off(int row, int ch) {
  return row * ROW_ELEMS + swz_slot<ROW_ELEMS>(row, ch) * 8;
}

// Transposed operand tiles hold a key (or query) axis along the row. Within
// every 16 consecutive positions, bits 2 and 3 of the index are swapped so
// that the 8 values one lane needs for an MFMA operand built from a C
// accumulator (indices 16t + 8h + 4g + r, h, r varying) are contiguous.
__device__ __forceinline__ int perm16(int idx) {
  return (idx & ~12) | ((idx & 4) << 1) | ((idx & 8) >> 1);
}

// ---------------------------------------------------------------------------
// Wavefront helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor32(float x) {
  // exchange with lane l ^ 32
  return __shfl_xor(x, 32, kWave);
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

// max of three floats: the compiler folds the pair of fmaxf into one
// v_max3_f32 (and, on MFMA results, adds no quieting step). Plain code rather
// than inline asm, whose outputs the hazard recognizer guards with a wait
// state before every dependent VALU instruction.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Staging-unit mapping for tiles written to LDS both row-major and transposed.
// A unit is 4 rows x 8 columns (four 16-byte global loads). Within a
// wavefront, CL consecutive lanes take CL consecutive column chunks of one row
// group (coalesced loads) and the remaining lane bits take distinct row
// groups, so a transposed 8-byte store spreads over all LDS banks (each bank
// hit twice for 512 bytes, the minimum) instead of hitting a few banks eight
// times.
template <int CPR, int RG>   // CPR column chunks per row, RG row groups per tile
__device__ __forceinline__ void unit_coords(int u, int* rg, int* ch) {
  constexpr int CL = (RG >= 16) ? 4 : 64 / RG;   // consecutive chunks per row group
  static_assert(CPR % CL == 0 && (CL & (CL - 1)) == 0, "unit mapping needs CL | CPR");
  const int lo = u % CL;
  const int g = (u / CL) % RG;
  const int hi = (u / CL) / RG;
  *rg = g;
  *ch = hi * CL + lo;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Software 2^x on the FMA path: Cody-Waite split x = n + f, n = floor(x),
// degree-3 Horner polynomial for 2^f on [0, 1) with p0 = 1 and p1..p3 the
// minimax relative-error fit (max relative error 8.56e-5; the printed
// 4-digit values are 0.6951, 0.2276, 0.0771), then n added into the exponent
// field. Inputs below -126 (including -inf) return 0.
__device__ __forceinline__ float emu_exp2(float x) {
  const float xs = fmaxf(x, -127.0f);
  const float n = __builtin_floorf(xs);
  const float f = xs - n;
  float p = __builtin_fmaf(0.07706713f, f, 0.22764487f);
  p = __builtin_fmaf(p, f, 0.69511682f);
  p = __builtin_fmaf(p, f, 1.0f);
  const int bits = __float_as_int(p) + (static_cast<int>(n) << 23);
  return xs < -126.0f ? 0.0f : __int_as_float(bits);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// The kernel's argument block (the only explicit argument, at offset 0 of the
// kernel argument segment), read through a pointer the compiler cannot see
// through. Called once per iteration of a persistent loop, it keeps the
// argument loads (scalar loads from constant memory) inside the iteration
// instead of hoisting them all in front of the loop, where they would stay
// live in SGPRs for the whole kernel and spill.
template <typename P>
__device__ __forceinline__ const P& kernel_args() {
#if defined(__HIP_DEVICE_COMPILE__)
  auto a = __builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(a));
  return *(const P*)(const __attribute__((address_space(4))) P*)a;
#else
  return *static_cast<const P*>(nullptr);   // host pass: never executed
#endif
}

// A uniform value the compiler must keep in an SGPR from here on: without
// this it may re-load an argument field (a scalar load from constant memory)
// inside a hot loop instead of keeping it live, and the wait for that load
// (lgkmcnt) also waits for every LDS read in flight.
template <typename T>
__device__ __forceinline__ T keep_sgpr(T x) {
  asm volatile("" : "+s"(x));
  return x;
}

// A wave-uniform 64-bit value moved to scalar registers (the compiler cannot
// always prove uniformity, e.g. of a value loaded through a per-tile index).
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Next tile position of a persistent workgroup in round r. queue == null:
// the static walk (schedule.hpp: persistent_index). Otherwise a ticket from a
// device counter, in the schedule's longest-first order — for packed variable
// lengths, whose tiles are too unequal for a static walk. A launch draws
// exactly ntiles + gridDim.x tickets (one past the end per workgroup), so
// counting modulo that keeps a counter cleared once (by the varlen schedule
// pass) valid for repeated launches of the same problem. Returns -1 when the
// workgroup is done; every thread of the workgroup calls it (barriers).
__device__ __forceinline__ int next_tile(int r, int ntiles, int nx, unsigned* queue, int* slot) {
  if (!queue) return persistent_index(blockIdx.x, r, gridDim.x, ntiles, nx);
  if (threadIdx.x == 0)
    *slot = static_cast<int>(atomicAdd(queue, 1u) % static_cast<unsigned>(ntiles + gridDim.x));
  __syncthreads();
  const int i = *slot;
  __syncthreads();   // every thread has read the ticket before the next draw
  return i < ntiles ? i : -1;
}

// Lane id (0..63) read where it is used: the asm cannot be hoisted out of a
// loop, so no register holds it across the loop body.
__device__ __forceinline__ int opaque_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// A wave-uniform flag through an opaque copy: a branch on it inside a loop
// is not hoisted out (no second copy of the loop).
__device__ __forceinline__ bool opaque_bool(bool b) {
  int v = __builtin_amdgcn_readfirstlane(b ? 1 : 0);
  asm volatile("" : "+s"(v));
  return v != 0;
}

// threadIdx.x through an opaque copy: values derived from it inside a
// persistent loop's tile body are then recomputed per tile rather than
// hoisted in front of the loop and kept live (in VGPRs) across all tiles.
__device__ __forceinline__ int tile_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// LSE in log2 units for the backward's P = 2^(S alpha log2 e - LSE log2 e).
// A row that saw no key has LSE = -inf; it maps to +inf so that every P of
// the row is 2^-inf = 0, masked (S = -inf) or not, and never -inf + inf.
__device__ __forceinline__ float lse_log2(float lse) {
  return lse == neg_inf() ? __builtin_inff() : lse * 1.4426950408889634f;
}

// ---------------------------------------------------------------------------
// Buffer resources: raw buffer loads return zero past `bytes`, which handles
// ragged sequence tails without branches. Offsets are 32-bit byte offsets.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Byte range of a buffer resource clamped to [0, 2^31 - 1].
__device__ __forceinline__ int clamp_range(int64_t bytes) {
  return bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : static_cast<int>(bytes));
}
// Resource for a range already clamped by clamp_range (no per-call checks).
__device__ __forceinline__ rsrc_t raw_rsrc(const void* base, int range) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, range, 0x00020000);
}

// One byte of a block mask (nonzero: the block is visible), read by the
// scalar unit from the dword that holds it: a uniform value, waited for in
// the same asm block (the wait also drains the LDS reads in flight). Offsets
// past the resource's range read as zero: hidden.
__device__ __forceinline__ bool mask_set(rsrc_t r, uint32_t byte_off) {
  uint32_t w;
  asm volatile("s_buffer_load_dword %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
               : "=s"(w) : "s"(r), "s"(byte_off & ~3u));
  return ((w >> ((byte_off & 3u) * 8u)) & 0xffu) != 0u;
}

// Block mask, one wavefront: the key tiles (bn keys each, tile n in mask
// column n bn / mblk) in [0, n_tiles) whose block is set in any of the mask
// rows r0 .. r1 (row r0 at byte mb0 of the mask buffer, rows stride bytes
// apart), in ascending order into vis[]; returns their count (every lane).
// Each lane tests one tile per round of 64; a ballot and a count of the
// lower lanes place it. Bytes past the buffer's range read as zero.
__device__ __forceinline__ int mask_list_tiles(rsrc_t r, uint32_t mb0, int stride, int r0, int r1,
                                               int n_tiles, int bn, int mblk, uint16_t* vis) {
  const int lane = static_cast<int>(__lane_id());
  int base = 0;
  for (int c0 = 0; c0 < n_tiles; c0 += 64) {
    const int n = c0 + lane;
    bool v = false;
    if (n < n_tiles) {
      const int col = n * bn / mblk;
      for (int row = r0; row <= r1; ++row)
        v = v || __builtin_amdgcn_raw_buffer_load_b8(
                     r, static_cast<int>(mb0 + (row - r0) * stride + col), 0, 0) != 0;
    }
    const uint64_t bal = __ballot(v);
    if (v) vis[base + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] = static_cast<uint16_t>(n);
    base += __builtin_popcountll(bal);
  }
  return base;
}

__device__ __forceinline__ bf16x8 buf_load16(rsrc_t r, int voff, int soff) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return __builtin_bit_cast(bf16x8, x);
}

// Streaming store (cache policy nt: data written once and read back much
// later by another kernel, kept from displacing reused lines in L2).
__device__ __forceinline__ void buf_store16_nt(rsrc_t r, int voff, int soff, const bf16x8& x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, voff, soff, 2);
}

// Streaming load (cache policy nt: data read once).
__device__ __forceinline__ bf16x8 buf_load16_nt(rsrc_t r, int voff, int soff) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
  return __builtin_bit_cast(bf16x8, x);
}

__device__ __forceinline__ float buf_load_f32(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// ---------------------------------------------------------------------------
// Direct global -> LDS loads (no VGPR staging). One instruction moves 64
// lanes x 16 bytes (or x 4 bytes) into LDS at dst + 16 * lane (4 * lane); dst
// must be the same for the whole wavefront. Completion is tracked by vmcnt
// only, so consumers wait with wait_vm<N>() and then a workgroup barrier.
// ---------------------------------------------------------------------------
// Written as inline asm: given the builtins, the compiler cannot tell which
// LDS bytes a load fills, so it makes later LDS reads wait for every such
// load in flight (vmcnt(0)), including those that prefetch a later step into
// another buffer. Hidden from it, the loads are ordered by the explicit
// wait_vm<N>() + barrier alone; its own vmcnt waits only grow more
// conservative with extra loads outstanding (they complete in order). M0
// carries the LDS address; s_nop 0 is the one wait state between writing M0
// and an LDS-DMA read of it. Nothing else in these kernels uses M0.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t lds_byte, int voff) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :: "v"(voff), "s"(lds_byte), "s"(r) : "memory", "m0");
}

// dma16 with cache policy nt (a stream read once).
__device__ __forceinline__ void dma16_nt(rsrc_t r, uint32_t lds_byte, int voff) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen nt lds"
               :: "v"(voff), "s"(lds_byte), "s"(r) : "memory", "m0");
}

__device__ __forceinline__ void dma4(const float* src, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds_byte) : "memory", "m0");
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Row swizzle of tiles filled by dma16: slot ch (16 bytes) of row r holds
// logical chunk ch ^ dma_swz<D>(r). Chosen so that (a) 16 consecutive rows
// read at one logical chunk (ds_read_b128 of an MFMA operand) and (b) the
// 4 rows x 4 chunks one 32-lane half of a transposing read touches (rows
// 4a .. 4a+3 and 8 + 4a .. 8 + 4a + 3, chunks 4b .. 4b+3) fall in distinct
// 16-byte bank groups. For r < 8, dma_swz(r + 8) == dma_swz(r) ^ 2.
template <int D>
__device__ __forceinline__ int dma_swz(int r) {
  if constexpr (D >= 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {   // 128-byte rows: two rows per 256-byte bank line
    const int t = (r >> 1) & 7;
    return ((t & 1) << 2) | (t >> 1);
  }
}

// gfx950 transposing LDS read of 4 x 16-bit values. Within each group of 16
// lanes, lane i receives element (i % 4) of the 8 bytes read by lanes
// 4j + i / 4 as its element j: if lane 4j + t reads row j, columns 4t .. 4t+3
// of a 16-bit matrix, lane i ends up with column i, rows 0..3.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ bf16x4 ds_read_tr(uint32_t lds_byte) {
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_byte));
  return __builtin_bit_cast(bf16x4, x);
}

// Reads at a 32-bit LDS byte address (no generic-pointer conversion).
// A ring slot as a compile-time constant: loops that run one copy of their
// body per slot of an LDS ring read each slot at immediate offsets.
template <int N> struct Slot { static constexpr int value = N; };

__device__ __forceinline__ bf16x8 lds_ld16(uint32_t lds_byte) {
  return *(const lds_bf16x8*)(lds_byte);
}
__device__ __forceinline__ f32x4 lds_ldf4(uint32_t lds_byte) {
  return *(const lds_f32x4*)(lds_byte);
}
__device__ __forceinline__ void lds_st16(uint32_t lds_byte, const bf16x8& x) {
  *(lds_bf16x8*)(lds_byte) = x;
}
// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)(p);
}

__device__ __forceinline__ bf16x8 cat8(const bf16x4& a, const bf16x4& b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace attn71
