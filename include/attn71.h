/*
 * attn71 — fused exact attention for AMD MI355X (gfx950), C ABI.
 *
 * The operation (FlashAttention-4 pages: digest page, notation table and
 * roofline paragraph; blog page, introduction, forward section and backward
 * section):
 *
 *   forward   S = alpha * Q K^T, P = softmax(S) over the visible keys,
 *             O = P V, and optionally LSE = log sum_j exp(S_j) (natural log),
 *             computed tile by tile with an online softmax whose rescale is
 *             skipped while the row max grows by at most tau = log2(256) = 8
 *             (base-2 units) and a final division by the true row sums;
 *   backward  from Q, K, V, O, dO and the stored LSE: D = rowsum(dO o O),
 *             P = exp(S - LSE), dP = dO V^T, dS = P o (dP - D),
 *             dQ = alpha dS K, dK = alpha dS^T Q, dV = P^T dO.
 *
 * Conventions shared by every call
 *   - q, k, v, o, dout, dq, dk, dv are bfloat16, contiguous, head dim
 *     innermost, 16-byte aligned device pointers.
 *     Fixed length: BSHD, q/o/dout/dq [batch, seqlen_q, num_heads_q, head_dim],
 *     k/v/dk/dv [batch, seqlen_k, num_heads_kv, head_dim].
 *     Packed variable length (the *_varlen calls): THD, q [total_q, Hq, d],
 *     k [total_k, Hkv, d]; sequence s owns rows cu_seqlens[s] ..
 *     cu_seqlens[s+1]-1.
 *   - lse is float32, natural log. Fixed length [batch, Hq, seqlen_q];
 *     varlen [Hq, total_q]. A row that sees no key gets O = 0, LSE = -inf.
 *   - Grouped heads: num_heads_q % num_heads_kv == 0 and query head h reads
 *     KV head h / (num_heads_q / num_heads_kv) (MQA: Hkv = 1, MHA: Hkv = Hq).
 *     dK, dV are summed over the query heads of each group.
 *   - causal: key j is visible to query i iff j <= i (lower triangular:
 *     the causal masking of the digest page's LPT scheduling item). With
 *     unequal lengths (per sequence for varlen) the diagonal is aligned to
 *     the last query and last key: j <= i + (Lk - Lq). The pages show only
 *     the square case; this alignment is the reading taken (a query block
 *     appended to a key cache). With Lq > Lk the first Lq - Lk queries see
 *     no key: O = 0, LSE = -inf, dQ = 0.
 *   - softmax_scale (alpha) is finite and > 0, typically 1/sqrt(head_dim).
 *   - head_dim is 64, 128 or 256; the device must be gfx950.
 *
 * Ownership and errors
 *   - The caller owns all device memory, including the workspace (size from
 *     the *_workspace_size calls). The library allocates and frees nothing
 *     and keeps no pointer after a call returns. Host structs are read during
 *     the call only.
 *   - Every argument is validated before anything is enqueued: a status other
 *     than ATTN_OK means no kernel was launched. ATTN_ERR_HIP reports a launch
 *     error from the HIP runtime. Calls are asynchronous on `stream` (NULL =
 *     the default stream); faults surface at the caller's next
 *     synchronisation. Nothing is thrown across the ABI.
 *   - Reentrant; the only global state is a per-device attribute cache and
 *     the process-wide tuning knobs of attn_set_tuning.
 */
#ifndef ATTN71_H
#define ATTN71_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN71_VERSION 100 /* 0.1.0 */

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARGUMENT = 1,    /* null pointer, bad shape/scale/flag, misalignment */
  ATTN_ERR_UNSUPPORTED = 2,         /* head_dim not in {64,128,256}, not gfx950, too large */
  ATTN_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the *_workspace_size value */
  ATTN_ERR_HIP = 4                  /* the HIP runtime refused a query or a launch */
} attn_status;

typedef struct attn_params {
  int32_t batch;         /* fixed: B. varlen: number of packed sequences */
  int32_t seqlen_q;      /* fixed: Sq. varlen: max query length (upper bound) */
  int32_t seqlen_k;      /* fixed: Sk. varlen: max key length (upper bound) */
  int32_t total_q;       /* varlen only: rows of q/o/dout/dq (ignored for fixed) */
  int32_t total_k;       /* varlen only: rows of k/v/dk/dv (ignored for fixed) */
  int32_t num_heads_q;   /* Hq >= 1 */
  int32_t num_heads_kv;  /* Hkv >= 1, divides Hq */
  int32_t head_dim;      /* 64, 128 or 256 */
  float softmax_scale;   /* alpha */
  int32_t causal;        /* 0 or 1 */
  int32_t deterministic; /* backward only, 0 or 1. The default split backward
                            writes every output once and is bit-identical across
                            runs either way; with bwd_fused_dq = 1, 0 = fp32
                            atomics for dQ, 1 = fixed accumulation order,
                            bit-identical dQ/dK/dV across runs (blog page,
                            deterministic-mode section) */
} attn_params;

/* "OK", "invalid argument", ... ; never NULL. */
const char* attn_status_string(attn_status status);
/* ATTN71_VERSION of the built library. */
int attn_version(void);

/* Workspace bytes for a forward / backward call with these parameters
 * (varlen = 1 for the *_varlen calls). 0 means no workspace is needed.
 * Returns (size_t)-1 for parameters that the calls would reject. */
size_t attn_fwd_workspace_size(const attn_params* p, int32_t varlen);
size_t attn_bwd_workspace_size(const attn_params* p, int32_t varlen);

/* 1 if a backward call with these parameters, under the current tuning
 * (attn_set_tuning "bwd_store_ds", "bwd_fused_dq"), has its dK/dV kernel store
 * dS into the workspace and computes dQ = alpha dS K from it; 0 if its dQ
 * kernel recomputes S and dP (or dQ is fused); -1 for parameters the calls
 * would reject. The stored dS takes B * Hq * ceil(Sq/64)*2 * ceil(Sk/256)*8
 * * 2 KiB of the workspace (about 2 bytes per query-key pair); for packed
 * lengths the workspace holds Hq * 2 (ceil(total_q/64) + batch) *
 * ceil(seqlen_k/256)*8 * 2 KiB, a bound from the total and the longest key
 * length (seqlen_k must bound every sequence's key length). */
int32_t attn_bwd_stores_ds(const attn_params* p, int32_t varlen);

/* Forward, fixed length. lse may be NULL (the LSE is optional on the pages:
 * blog page, correction-warpgroup list, "optionally compute and store LSE"). */
attn_status attn_fwd(const attn_params* p, const void* q, const void* k, const void* v, void* o,
                     float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Forward, packed variable length. cu_seqlens_q / cu_seqlens_k: device int32
 * [batch + 1], non-decreasing, starting at 0, ending at total_q / total_k.
 * A pre-pass orders the sequences longest first (blog page, scheduling
 * section, varlen sort and virtual-to-actual batch map). */
attn_status attn_fwd_varlen(const attn_params* p, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, const void* q, const void* k,
                            const void* v, void* o, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Backward, fixed length: dq, dk, dv from q, k, v, the forward's o and lse
 * (required) and dout. Launches on `stream`: preprocess (D = rowsum(dO o O));
 * main; postprocess. Two designs, chosen by attn_set_tuning("bwd_fused_dq"):
 *   0 (default) main = a dK/dV kernel (one workgroup per key block, four
 *     GEMMs) plus a dQ kernel (one workgroup per query block, S and dP
 *     recomputed): no atomics, bit-reproducible whatever `deterministic` says;
 *   1 main = one kernel that also adds each tile's dQ into an fp32 buffer with
 *     atomics (blog page, 2-CTA backward, dQ atomic accumulation), or, with
 *     deterministic = 1, in a fixed order behind per-block semaphores (blog
 *     page, deterministic mode); postprocess converts dQ to bf16.
 * In the split design the dQ kernel either recomputes S and dP from q, k, v,
 * dout and lse, or (attn_bwd_stores_ds = 1) reads the dS that
 * the dK/dV kernel wrote into the workspace and runs dQ = alpha dS K, its
 * only GEMM (blog page, backward section: dQ is dS times the key block).
 * Both write dQ once: bit-reproducible either way. */
attn_status attn_bwd(const attn_params* p, const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse, void* dq, void* dk,
                     void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward, packed variable length (same conventions as attn_fwd_varlen). */
attn_status attn_bwd_varlen(const attn_params* p, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, const void* q, const void* k,
                            const void* v, const void* o, const void* dout, const float* lse,
                            void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* The backward split into its phases, for callers that schedule or time them
 * separately. `phases` is a mask of ATTN_BWD_*; running the masks in the
 * order PREPROCESS, MAIN, DQ, POSTPROCESS on one stream with the same
 * workspace equals attn_bwd(_varlen) (with the recomputing dQ kernel MAIN and
 * DQ are independent of each other and may also run in either order).
 * cu_seqlens_q/k NULL = fixed length. Arguments a phase does not read may
 * be NULL only if no selected phase reads them. Every MAIN phase needs a
 * PREPROCESS phase of the same workspace before it: it clears the dQ
 * accumulator and, in deterministic mode, the ordering state. A MAIN phase
 * run without it still terminates and stays in bounds, but dQ accumulates on
 * the previous values and the deterministic order is not guaranteed. When
 * the call stores dS (attn_bwd_stores_ds), the DQ phase reads what the MAIN
 * phase of the same workspace wrote: run MAIN before DQ. */
#define ATTN_BWD_PREPROCESS 1  /* D = rowsum(dO o O); fused design: clear dQ accumulator, semaphores */
#define ATTN_BWD_MAIN 2        /* key-block kernel: dK, dV (fused design: + dQ accumulation) */
#define ATTN_BWD_POSTPROCESS 4 /* fused design: dQ = bf16(alpha * accumulator); else nothing */
#define ATTN_BWD_DQ 8          /* split design: the query-block dQ kernel; else nothing */
#define ATTN_BWD_ALL 15
attn_status attn_bwd_phases(const attn_params* p, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t phases, const void* q,
                            const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Diagnostics of the deterministic backward: the error word of the last
 * backward that used this workspace (0 = fine; 1 = a bounded wait of the
 * ordered dQ chain expired and the ordering was abandoned). Synchronous:
 * waits for `stream`. */
attn_status attn_bwd_status(const attn_params* p, int32_t varlen, const void* workspace,
                            int32_t* status_out, hipStream_t stream);

/* Tile order of the fixed-length kernels, evaluated on the host with the
 * same arithmetic the kernels use (scheduling section of the blog page:
 * longest first, L2-sized batch-head sections; here also one contiguous range
 * per XCD). which = 0: forward, out[3*i..3*i+2] = (batch, query head,
 * query block) of workgroup i; which = 1: dK/dV (or fused) backward,
 * which = 2: fused deterministic backward in ticket order, (batch, KV head,
 * key block); which = 3: dQ kernel, (batch, query head, query block).
 * *count receives the grid size; at most `capacity` triples are written.
 * No GPU is needed. */
attn_status attn_tile_order(const attn_params* p, int32_t which, int32_t* out, int64_t capacity,
                            int64_t* count);

/* Persistent launches (forward, dK/dV and dQ kernels): `grid` workgroups, as
 * many as fit on the device at once, loop over the `ntiles` positions of the
 * tile order above. Returns the position that workgroup g takes in round r,
 * or -1 when it has no more (host evaluation of the kernels' arithmetic:
 * workgroup g stays on XCD g % nx; rounds alternate direction). Requires
 * grid >= min(ntiles, nx). No GPU is needed. */
int32_t attn_persistent_tile(int32_t g, int32_t r, int32_t grid, int32_t ntiles, int32_t nx);

/* Process-wide tuning knobs (not synchronised with launches in flight):
 *   "bwd_fused_dq"  0 = dK/dV kernel + dQ kernel (default), 1 = one kernel with
 *                   dQ atomics / semaphore-ordered adds (see attn_bwd);
 *   "fwd_pingpong"  1 = forward with two wave groups offset by one phase so
 *                   MFMA and softmax overlap (head_dim <= 128; measured slower on
 *                   MI355X so far), 0 = one phase per key tile (default);
 *   "tile_order"    0 = longest first + XCD ranges (default), 1 = natural
 *                   (batch-head major, blocks ascending, no remap);
 *   "persistent"    1 = resident workgroups loop over the tiles (default: a
 *                   static walk for fixed lengths, tickets from a workspace
 *                   counter for packed variable lengths); 0 = one workgroup
 *                   per tile;
 *   "exp_emulation" -1 = automatic (default: 0, the fastest measured at
 *                   every head_dim); 0 = every exp2 on
 *                   v_exp_f32; 1, 2 or 4 = that many of every 8 on the
 *                   Cody-Waite + Horner FMA path (blog page, faster exponential
 *                   section);
 *   "tau"           forward rescale threshold on the running-max jump, in
 *                   log2 units, 0..64 (default 8 = log2 256: digest page item
 *                   3; blog page, forward section). 0 rescales on every
 *                   increase of the row max;
 *   "spin_limit"    bound on each wait of the deterministic chain (default
 *                   2^26 polls);
 *   "bwd_store_ds"  split backward: -1 = automatic (default:
 *                   stored dS at head_dim 128 and 256, where it measured 5 %
 *                   and 11 % faster per fwd+bwd step; recomputation at 64,
 *                   where the dK/dV kernel's extra writes cost more than the
 *                   dQ kernel saves), 1 = the dK/dV kernel stores dS and dQ = alpha dS K,
 *                   0 = the dQ kernel recomputes S and dP. Heads whose
 *                   stored dS would exceed 2 GiB (at the longest lengths)
 *                   always recompute.
 * Returns ATTN_ERR_INVALID_ARGUMENT for unknown keys or values. */
attn_status attn_set_tuning(const char* key, int32_t value);

#ifdef __cplusplus
}
#endif

#endif /* ATTN71_H */
