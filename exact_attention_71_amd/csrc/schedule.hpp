// Tile order: which (sequence, head, block) a workgroup processes.
//
// Causal masking and variable lengths give tiles different amounts of work.
// The FlashAttention-4 blog page (scheduling section) orders tiles
// longest-processing-time first: batch-heads are grouped into sections whose
// K/V fit in L2, and inside a section the m-blocks are visited in reverse
// (longest first), batch-heads innermost. For packed variable lengths a
// pre-pass sorts the sequences by their longest tile and the kernel walks
// them through a virtual-to-actual map.
//
// MI355X form of the same idea: workgroup i is dispatched to XCD i % 8 and each
// XCD has its own L2, so the workgroup index is first remapped so that each
// XCD receives one contiguous range of the section order (its own batch-heads,
// longest tiles first). The deterministic backward takes SPT order instead
// (shortest first, see the backward kernel).
//
// Everything here is plain integer arithmetic usable on host and device, so
// the host test entry point evaluates exactly what the kernels evaluate.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define A71_HD __host__ __device__ __forceinline__
#else
#define A71_HD inline
#endif

namespace attn71 {

struct Tile {
  int seq;    // sequence (batch index, or actual packed-sequence index)
  int head;   // query head (forward) or KV head (backward)
  int block;  // m-block (forward) or n-block (backward)
};

A71_HD int imin(int a, int b) { return a < b ? a : b; }
A71_HD int imax(int a, int b) { return a > b ? a : b; }
A71_HD int cdiv(int a, int b) { return (a + b - 1) / b; }

// Causal mask with the diagonal aligned to the last query and the last key:
// query i of a sequence with lq queries and lk keys sees key j iff
// j <= i + shift, shift = lk - lq (equal lengths: lower triangular).
// Keys visible to any of the rows below row_end: [0, causal_key_end).
A71_HD int causal_key_end(int row_end, int shift, int lk) {
  return imax(0, imin(row_end + shift, lk));
}
// First query row that sees key n0 (rows before it see no key >= n0).
A71_HD int causal_row_begin(int n0, int shift) { return imax(0, n0 - shift); }

// Position of workgroup i among the contiguous ranges given to each XCD.
// XCD x (receiving workgroups x, x + nx, x + 2nx, ...) owns positions
// [x*q + min(x, r), ...) with q = n / nx, r = n % nx. A bijection on [0, n).
A71_HD int xcd_remap(int i, int n, int nx) {
  if (nx <= 1) return i;
  const int x = i % nx, j = i / nx;
  const int q = n / nx, r = n % nx;
  return x * q + imin(x, r) + j;
}

// Persistent workgroups. Dispatch hands workgroups to the XCDs round-robin
// and, inside an XCD, to its shader engines in turn. With a one-shot grid of
// unequal causal tiles that leaves CUs idle: in a timeline of the dK/dV kernel
// at B2 H16 S8192 (one workgroup per CU), later workgroups started in groups
// of four, one per shader engine, each group only once every engine had a
// free CU, so a CU sat idle ~20 us on average before each new tile. Instead G workgroups,
// as many as can be resident, loop over the n tiles of the schedule order in
// rounds. Workgroup g stays on XCD x = g % nx as the j-th of its J_x
// workgroups; in round r it takes the tile that workgroup x + nx * p of a
// one-shot grid would take, with p = r * J_x + j in even rounds and
// r * J_x + (J_x - 1 - j) in odd rounds. Going back and forth pairs the
// longest tiles of one round with the shortest of the next, and every tile
// keeps the XCD (and L2) it has in the one-shot grid. With G = n this is
// exactly the one-shot grid. Requires G >= min(n, nx) so that every residue
// class of tiles has a workgroup. Returns -1 past the last tile.
A71_HD int persistent_index(int g, int r, int G, int n, int nx) {
  if (nx < 1) nx = 1;
  const int x = g % nx, j = g / nx;
  const int J = (G - x + nx - 1) / nx;
  const int64_t pos = (int64_t)r * J + ((r & 1) ? (J - 1 - j) : j);
  const int64_t i = x + (int64_t)nx * pos;
  return i < n ? (int)i : -1;
}

// Section order over a regular grid of nbh batch-heads x nblk blocks:
// sections of `sec` batch-heads; inside a section blocks are visited from
// `first` in the direction given by `reverse`, batch-heads innermost.
// Requires 0 <= v < nbh * nblk (callers check).
A71_HD void section_decode(int v, int nbh, int nblk, int sec, bool reverse, int* bh, int* blk) {
  const int per_sec = sec * nblk;
  const int s = v / per_sec;
  const int u = v - s * per_sec;
  const int width = imin(sec, nbh - s * sec);   // last section may be narrower
  const int b = u / width;
  *bh = s * sec + (u - b * width);
  *blk = reverse ? (nblk - 1 - b) : b;
}

// Forward, fixed length: grid = B * Hq * nm. Longest first for causal (high
// m-blocks first); the XCD remap applies when the batch-heads split evenly.
// natural = true gives the plain order (batch-head major, blocks ascending).
A71_HD Tile fwd_tile_fixed(int wg, int batch, int heads, int nm, int sec, int nxcd,
                           bool natural) {
  const int nbh = batch * heads;
  const int n = nbh * nm;
  int bh, blk;
  if (natural) {
    bh = wg / nm;
    blk = wg - bh * nm;
  } else {
    const int v = (nbh % nxcd == 0) ? xcd_remap(wg, n, nxcd) : wg;
    section_decode(v, nbh, nm, sec, /*reverse=*/true, &bh, &blk);
  }
  Tile t;
  t.seq = bh / heads;
  t.head = bh - t.seq * heads;
  t.block = blk;
  return t;
}

// Backward, fixed length: one workgroup per (batch, KV head, n-block).
// Non-deterministic: longest first (n-block 0 sees the most query blocks
// under the causal mask). Deterministic: shortest first, the order in which
// the semaphore chain hands out turns (see the backward kernel).
// natural = true (non-deterministic only) gives batch-head major, blocks ascending.
A71_HD Tile bwd_tile_fixed(int v, int batch, int heads_kv, int nn, int sec, bool shortest_first,
                           int nxcd, bool natural) {
  const int nbh = batch * heads_kv;
  const int n = nbh * nn;
  int bh, blk;
  if (natural && !shortest_first) {
    bh = v / nn;
    blk = v - bh * nn;
  } else {
    if (!shortest_first && nbh % nxcd == 0) v = xcd_remap(v, n, nxcd);
    section_decode(v, nbh, nn, sec, /*reverse=*/shortest_first, &bh, &blk);
  }
  Tile t;
  t.seq = bh / heads_kv;
  t.head = bh - t.seq * heads_kv;
  t.block = blk;
  return t;
}

// Packed variable lengths: sequences in the order written by the varlen
// schedule pass (longest first), tile_prefix[vs] = first tile of virtual
// sequence vs, tiles of one sequence ordered block-major (reverse when
// `reverse`) with heads innermost. Returns seq = -1 past the last tile.
A71_HD Tile varlen_tile(int v, const int* order, const int* tile_prefix, int nseq, int heads,
                        bool reverse) {
  Tile t;
  t.seq = -1; t.head = 0; t.block = 0;
  if (nseq <= 0 || v >= tile_prefix[nseq]) return t;
  int lo = 0, hi = nseq - 1;  // last vs with tile_prefix[vs] <= v
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_prefix[mid] <= v) lo = mid; else hi = mid - 1;
  }
  const int u = v - tile_prefix[lo];
  const int nblk = (tile_prefix[lo + 1] - tile_prefix[lo]) / heads;
  const int b = u / heads;
  t.seq = order[lo];
  t.head = u - b * heads;
  t.block = reverse ? (nblk - 1 - b) : b;
  return t;
}

// Key-block tiles of packed sequences in one global longest-first order. The
// work of key block b of a sequence (query rows lq, keys lk, query blocks of
// bm rows, key blocks of bn keys) is its number of query-block steps: all of
// them without a causal mask, those from the block's diagonal on with one
// (bottom-right aligned).
A71_HD int key_block_work(int lq, int lk, int bm, int bn, bool causal, int b) {
  const int nm = cdiv(lq, bm);
  if (!causal) return nm;
  return nm - imin(causal_row_begin(b * bn, lk - lq) / bm, nm);
}
// Number of key blocks b < nkb with work >= w (work > w when strict). The
// work never grows with b: under the causal mask, work >= w (1 <= w <= nm)
// holds iff the block's first visible row, max(0, b bn - shift), lies below
// (nm - w + 1) bm, i.e. iff b bn < (nm - w + 1) bm + shift.
A71_HD int key_blocks_above(int lq, int lk, int bm, int bn, bool causal, int nkb, int w,
                            bool strict) {
  if (strict) ++w;
  const int nm = cdiv(lq, bm);
  if (w <= 0) return imax(nkb, 0);
  if (w > nm) return 0;
  if (!causal) return imax(nkb, 0);
  const int n = cdiv((nm - w + 1) * bm + (lk - lq), bn);
  return imax(0, imin(n, nkb));
}
// Position of key block b of sequence s in the longest-first order of all
// blocks (ties: sequence, then block, ascending): the blocks with more work,
// plus the blocks with equal work that come first. len_q / len_k: the
// sequences' query and key lengths; a permutation of [0, total blocks).
A71_HD int key_block_rank(const int* len_q, const int* len_k, int nseq, int bm, int bn,
                          bool causal, int s, int b) {
  const int w = key_block_work(len_q[s], len_k[s], bm, bn, causal, b);
  int r = b;   // this sequence's earlier blocks (their work is >= w)
  for (int t = 0; t < nseq; ++t) {
    if (t == s) continue;
    r += key_blocks_above(len_q[t], len_k[t], bm, bn, causal, cdiv(len_k[t], bn), w,
                          /*strict=*/t > s);
  }
  return r;
}

// Key block e of the natural order (sequence-major, blocks of bn keys
// ascending): *s = its sequence, *b = its block; *s = -1 past the last.
A71_HD void key_block_at(const int* len_k, int nseq, int bn, int e, int* s, int* b) {
  *s = -1; *b = 0;
  for (int t = 0; t < nseq; ++t) {
    const int n = cdiv(len_k[t], bn);
    if (n > 0 && e < n) { *s = t; *b = e; return; }
    if (n > 0) e -= n;
  }
}

// Host/device reference of the varlen schedule pass (also run by the single
// workgroup schedule kernel): sequences sorted by decreasing length (ties by
// index), tile prefix over ceil(len / blk) * heads, and the per-sequence
// prefix of query blocks (for semaphores) in natural order.
A71_HD int varlen_rank(const int* cu, int nseq, int s) {
  const int ls = cu[s + 1] - cu[s];
  int r = 0;
  for (int t = 0; t < nseq; ++t) {
    const int lt = cu[t + 1] - cu[t];
    r += (lt > ls) || (lt == ls && t < s);
  }
  return r;
}

}  // namespace attn71
