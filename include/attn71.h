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
 *     innermost, 16-byte aligned device pointers. A tensor with no elements
 *     (no query rows: q, o, dout, dq, lse; no keys: k, v, dk, dv) may be
 *     null: no kernel touches it. Rows that see no key get O = 0, LSE =
 *     -inf and dQ = 0; keys that no row sees get dK = dV = 0.
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
 *   - Reentrant. Every design choice and tuning value travels with the call
 *     (attn_params.opt); the only global state is a once-initialised
 *     per-device attribute cache (architecture, compute units). Workspace
 *     sizes are pure functions of the parameters.
 */
#ifndef ATTN71_H
#define ATTN71_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN71_VERSION 202 /* 0.2.2: + longest-first packed key-block order */

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARGUMENT = 1,    /* null pointer, bad shape/scale/flag, misalignment */
  ATTN_ERR_UNSUPPORTED = 2,         /* head_dim not in {64,128,256}, not gfx950, too large */
  ATTN_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the *_workspace_size value */
  ATTN_ERR_HIP = 4                  /* the HIP runtime refused a query or a launch */
} attn_status;

/* Backward designs (attn_options.bwd_design). All compute the same
 * gradients; they differ in how dQ is formed (blog page, backward, 2-CTA
 * backward and deterministic-mode sections):
 *   ATTN_BWD_AUTO        stored dS at head_dim 128 and 256 when the dS area
 *                        fits opt.ds_budget, else recomputing dQ;
 *   ATTN_BWD_RECOMPUTE   a dK/dV kernel (one workgroup per key block, four
 *                        GEMMs) plus a dQ kernel (one workgroup per query
 *                        block) that recomputes S and dP; no atomics, every
 *                        output written once: bit-reproducible;
 *   ATTN_BWD_STORED_DS   the dK/dV kernel also writes the bf16 dS it forms
 *                        into the workspace and the dQ kernel runs
 *                        dQ = alpha dS K as its only GEMM; bit-reproducible;
 *                        needs the dS area to fit opt.ds_budget
 *                        (ATTN_ERR_UNSUPPORTED otherwise);
 *   ATTN_BWD_FUSED_DQ    one key-block kernel for all five GEMMs that adds
 *                        each step's dQ into an fp32 buffer with atomics
 *                        (head_dim 64, 128: once per 256 keys; 256: once per
 *                        128), or, with deterministic = 1, in a fixed order
 *                        (the last key block first) behind per-(query block,
 *                        query head) semaphores; a postprocess converts dQ.
 *                        Bound by the device's fp32 atomic rate, 2 bytes of
 *                        adds per visible (query, key) pair at head_dim 128. */
#define ATTN_BWD_AUTO 0
#define ATTN_BWD_RECOMPUTE 1
#define ATTN_BWD_STORED_DS 2
#define ATTN_BWD_FUSED_DQ 3

/* Per-call options. An all-zero struct selects every default. */
typedef struct attn_options {
  int32_t bwd_design;    /* ATTN_BWD_* above (default ATTN_BWD_AUTO) */
  int32_t tile_order;    /* 0 (default): longest first over L2-sized batch-head
                            sections, one contiguous range per XCD (blog page,
                            scheduling section); 1: natural order (batch-head
                            major, blocks ascending) */
  int32_t one_shot_grid; /* 0 (default): as many workgroups as fit at once loop
                            over the tiles (packed lengths: tickets from a
                            workspace counter); 1: one workgroup per tile */
  int32_t exp_emulation; /* 0 (default): every exp2 on v_exp_f32; 1, 2 or 4:
                            that many of every 8 on the Cody-Waite + Horner FMA
                            path (blog page, faster exponential section) */
  float tau;             /* forward rescale threshold on the running-max jump,
                            log2 units: 0 selects the default 8 = log2 256
                            (digest page item 3; blog page, forward section);
                            a value in (0, 64] is used as given; -1 selects 0
                            (rescale on every increase of the row max) */
  int32_t spin_limit;    /* deterministic fused backward: bound on each wait of
                            the ordered dQ chain in polls (0: default 2^26) */
  int64_t ds_budget;     /* bytes of stored dS the backward may place in its
                            workspace (0: default ATTN_DS_BUDGET_DEFAULT) */
  int32_t head_split;    /* backward key-block tiles: 0 (default) automatic:
                            when the (sequence, KV head, key block) tiles
                            would not fill the device (few KV heads, few or
                            short sequences; fewer than ATTN_SPLIT_TARGET
                            tiles), the query heads of each KV group are split
                            over n workgroups (the largest divisor n of
                            Hq / Hkv that keeps the tiles within the target),
                            each writing fp32 dK / dV partials that a
                            reduction adds in a fixed order; 1: never split;
                            n >= 2: n parts (n must divide Hq / Hkv; not with
                            the fused design at head_dim 256) */
  int32_t reserved;      /* must be zero */
} attn_options;

#define ATTN_DS_BUDGET_DEFAULT (4ll << 30)
#define ATTN_SPLIT_TARGET 512 /* key-block tiles the automatic head split aims at */

/* A varlen plan: the schedule tables of one packed batch (the order of the
 * sequences longest first, tile and block prefix sums, stored-dS offsets,
 * the longest-first list of all key blocks (attn_varlen_key_order),
 * tile-ticket counters) for every kernel, built once by
 * attn_varlen_plan_build and reused by any number of attn_fwd_varlen /
 * attn_bwd_varlen / attn_bwd_phases calls on the same sequences (blog page,
 * scheduling section: the metadata can be cached, so the sort costs
 * nothing). The caller owns `data` (attn_varlen_plan_size bytes of device
 * memory). The fields below `bytes` record the parameters the plan was built
 * for; a call whose parameters differ in any of them is rejected
 * (ATTN_ERR_INVALID_ARGUMENT). The cu_seqlens contents cannot be checked:
 * a plan is valid for the cu_seqlens values it was built from. Calls that
 * use one plan must not overlap in time (they share its tile counters). */
typedef struct attn_varlen_plan {
  void* data;
  size_t bytes;
  int32_t batch, seqlen_q, seqlen_k, total_q, total_k, num_heads_q, num_heads_kv, head_dim,
      causal;
} attn_varlen_plan;

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
  int32_t deterministic; /* backward only, 0 or 1: bit-identical dQ/dK/dV across
                            runs (blog page, deterministic-mode section). The
                            recomputing and stored-dS designs write every output
                            once and are bit-identical either way; the fused
                            design orders its dQ additions when set */
  attn_options opt;      /* per-call design and tuning options (zero: defaults) */
  const attn_varlen_plan* varlen_plan; /* varlen calls: the cached schedule (NULL: each
                                          call computes it in its workspace) */
  /* Block-sparse mask (fixed length; NULL: none), the reading taken of the
   * synthesis page's block-sparse attention on the FA4 framework: one byte
   * per 128 x 128 block of (query, key) pairs, at byte
   *   b * block_mask_stride_b + h * block_mask_stride_h + i * ceil(seqlen_k / 128) + j
   * for batch b, query head h, query block i < ceil(seqlen_q / 128), key
   * block j; 0 hides every pair of the block, ANDed with the causal rule.
   * Rows that see no key get O = 0, LSE = -inf, dQ = 0. Strides may be 0 (one
   * mask shared by the batches or heads). The pointer must be 4-byte aligned;
   * the mask is read in 4-byte words, so the buffer must hold its span rounded
   * up to a multiple of 4 bytes, at most 2^31 - 1; packed variable lengths, the
   * stored-dS design (ATTN_BWD_AUTO then recomputes dQ), exp_emulation and
   * seqlen_k above 4096 * 64 keys (the length of the visible-tile lists the
   * forward and dQ kernels keep) are refused with a mask
   * (ATTN_ERR_UNSUPPORTED). The forward and dQ kernels skip hidden key tiles;
   * the dK/dV kernel skips the (query head, 128-row block) pairs hidden for
   * all of its keys, except in the deterministic fused design, whose ordered
   * dQ chain steps through them (masked to zero). */
  const uint8_t* block_mask;
  int64_t block_mask_stride_b, block_mask_stride_h;
} attn_params;

/* "OK", "invalid argument", ... ; never NULL. */
const char* attn_status_string(attn_status status);
/* ATTN71_VERSION of the built library. */
int attn_version(void);

/* Workspace bytes for a forward / backward call with these parameters
 * (varlen = 1 for the *_varlen calls), a pure function of its arguments.
 * 0 means no workspace is needed. Returns (size_t)-1 for parameters that the
 * calls would reject. Packed lengths are sized from the totals, the batch
 * count and the maxima seqlen_q / seqlen_k (the lengths themselves live on
 * the device; the sizing variants of a spec that takes num_seqs and the
 * maxima need the totals as well, for the per-row statistics). */
size_t attn_fwd_workspace_size(const attn_params* p, int32_t varlen);
size_t attn_bwd_workspace_size(const attn_params* p, int32_t varlen);

/* The backward design a call with these parameters runs (ATTN_BWD_RECOMPUTE,
 * ATTN_BWD_STORED_DS or ATTN_BWD_FUSED_DQ: opt.bwd_design with AUTO
 * resolved), or -1 for parameters the calls would reject (including an
 * explicit ATTN_BWD_STORED_DS whose dS does not fit opt.ds_budget).
 * Stored dS keeps only the sub-tiles the causal mask leaves visible: per
 * (sequence, query head) the 32-query rows of a 256-query group hold the
 * 32 x 32 sub-tiles (2 KiB) of every 256-key block that reaches into the
 * group, about 1 byte per query-key pair under a causal mask and 2 without
 * (B2 H16 S8192 causal d128: 2.06 GiB). Packed lengths are sized by
 * Hq * 2 (ceil(total_q/64) + batch) * ceil(seqlen_k/256) * 8 sub-tiles,
 * a bound from the totals and the longest key length (seqlen_k must bound
 * every sequence's key length; sequences beyond it drop stores rather than
 * write past the workspace). */
int32_t attn_bwd_design(const attn_params* p, int32_t varlen);

/* Query-head parts per KV group the backward's key-block kernel runs with
 * (opt.head_split resolved; 1: unsplit), -1 if the parameters are invalid
 * or the design request cannot be met. With n > 1 each (sequence, KV head,
 * key block) tile becomes n workgroups, part j walking query heads
 * j Hq/(Hkv n) .. (j+1) Hq/(Hkv n) - 1 of the group and writing fp32 dK / dV
 * partials that a reduction kernel adds in part order (deterministic). Pure
 * function of the arguments. */
int32_t attn_bwd_head_split(const attn_params* p, int32_t varlen);

/* Bytes of device memory a varlen plan for these parameters needs (they
 * depend on the sequence count, and through the key-block list on total_k
 * and head_dim); (size_t)-1 for parameters the varlen calls would reject. */
size_t attn_varlen_plan_size(const attn_params* p);

/* Builds a varlen plan for the packed batch described by p and the device
 * arrays cu_seqlens_q / cu_seqlens_k (as for attn_fwd_varlen): fills *plan
 * (host) and enqueues one schedule kernel on `stream` that writes the tables
 * into `data` (`bytes` >= attn_varlen_plan_size). Calls that then pass the
 * plan in attn_params.varlen_plan launch no schedule pass of their own, and
 * their workspaces hold no tables (the workspace sizes drop accordingly). */
attn_status attn_varlen_plan_build(const attn_params* p, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, void* data, size_t bytes,
                                   attn_varlen_plan* plan, hipStream_t stream);

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
 * (required) and dout. Launches on `stream`: preprocess (D = rowsum(dO o O)),
 * then the kernels of opt.bwd_design (see ATTN_BWD_*): dK/dV and dQ kernels,
 * or the fused kernel and its postprocess. */
attn_status attn_bwd(const attn_params* p, const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse, void* dq, void* dk,
                     void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward, fixed length, allocating nothing: for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments and results as attn_bwd
 * with the recomputing design (opt.bwd_design must be ATTN_BWD_AUTO or
 * ATTN_BWD_RECOMPUTE, else ATTN_ERR_UNSUPPORTED), but no workspace argument:
 * the workspace lives in a library-owned static device array of
 * ATTN_NOALLOC_SCRATCH_BYTES, which each GPU the library runs on holds until
 * the process ends. Calls whose workspace (attn_bwd_workspace_size with the
 * recomputing design: 8 bytes per (query row, query head) plus a few
 * hundred) exceeds it return ATTN_ERR_UNSUPPORTED before launching
 * anything. The first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress); no call allocates or frees memory. All calls
 * on one GPU share its array, and each call rewrites what it needs, so calls
 * that overlap in time on one GPU (other streams, other host threads) race:
 * serialize them. */
#define ATTN_NOALLOC_SCRATCH_BYTES (32ll << 20)
attn_status attn_bwd_noalloc(const attn_params* p, const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse, void* dq,
                             void* dk, void* dv, hipStream_t stream);

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
 * the call stores dS (attn_bwd_design), the DQ phase reads what the MAIN
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

/* Tile order of the fixed-length kernels under p->opt.tile_order, evaluated
 * on the host with the same arithmetic the kernels use (scheduling section
 * of the blog page: longest first, L2-sized batch-head sections; here also
 * one contiguous range per XCD). which = 0: forward, out[3*i..3*i+2] = (batch, query head,
 * query block) of workgroup i; which = 1: dK/dV (or fused) backward,
 * which = 2: fused deterministic backward in ticket order (key blocks of
 * 256 at head_dim 64 and 128, 128 at 256), (batch, KV head, key block),
 * or with a head split of n (attn_bwd_head_split) (batch, KV head * n +
 * part, key block);
 * which = 3: dQ kernel, (batch, query head, query block).
 * *count receives the grid size; at most `capacity` triples are written.
 * No GPU is needed. */
attn_status attn_tile_order(const attn_params* p, int32_t which, int32_t* out, int64_t capacity,
                            int64_t* count);

/* Packed lengths: the order in which the dK/dV kernel of the recomputing
 * and stored-dS designs (and of the fused design at head_dim 64 and 128,
 * unless deterministic) takes its key-block tiles. The FlashAttention-4 blog
 * page (scheduling section) puts the longest tiles first; here every key
 * block of every sequence is ranked by its work (the query-block steps it
 * visits: all of them without a causal mask, those from its diagonal on
 * with one), ties by sequence then block, and the KV heads of one key block
 * follow each other. cu_q / cu_k: host copies of the packed offsets
 * (batch + 1 entries each, non-decreasing). Writes (sequence, key block)
 * pairs in that order to out[2 r], out[2 r + 1] for the first `capacity`
 * ranks; *count receives the number of key blocks. ATTN_ERR_UNSUPPORTED
 * when the call keeps the per-sequence order instead (the order of
 * attn_tile_order's packed analogue: sequences longest first), which it
 * does past 2^17 (key-block bound x batch) ranking steps. Evaluated on the
 * host with the schedule pass's arithmetic; no GPU is needed. */
attn_status attn_varlen_key_order(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k,
                                  int32_t* out, int64_t capacity, int64_t* count);

/* Stored-dS layout, evaluated on the host with the kernels' arithmetic: the
 * index of the 32 x 32 sub-tile (sub-row row32 = queries 32 row32 ..,
 * sub-column col32 = keys 32 col32 ..) inside the region of one (sequence,
 * query head) with p->seqlen_q queries and p->seqlen_k keys (p->causal), or
 * -1 when the layout keeps no such sub-tile. The region holds
 * *region_tiles sub-tiles (2 KiB each). Key-block major: each 256-key block
 * keeps the sub-rows from the first one its dK/dV step writes, 8 sub-tiles
 * per sub-row. No GPU is needed. */
int64_t attn_bwd_ds_subtile(const attn_params* p, int32_t row32, int32_t col32,
                            int64_t* region_tiles);

/* Persistent launches (forward, dK/dV and dQ kernels): `grid` workgroups, as
 * many as fit on the device at once, loop over the `ntiles` positions of the
 * tile order above. Returns the position that workgroup g takes in round r,
 * or -1 when it has no more (host evaluation of the kernels' arithmetic:
 * workgroup g stays on XCD g % nx; rounds alternate direction). Requires
 * grid >= min(ntiles, nx). No GPU is needed. */
int32_t attn_persistent_tile(int32_t g, int32_t r, int32_t grid, int32_t ntiles, int32_t nx);

#ifdef __cplusplus
}
#endif

#endif /* ATTN71_H */
