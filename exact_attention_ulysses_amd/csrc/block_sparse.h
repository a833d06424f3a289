// Walking a block layout from inside a kernel (internal).
//
// Block-sparse attention (paper-graph summary of arXiv 2309.14509, section
// 3.4 and Figs 6-7: "blocked sparse attention" runs after the same
// all-to-all; pinyu.ai: each rank holds the full sequence of its heads and can
// apply the whole pattern locally) takes a per-head uint8 layout
// [heads][nb][nb]: entry (i, j) != 0 lets query block i attend key block j
// (128 tokens each). A kernel visits the active blocks of one layout row (the
// key blocks of a query block) or one column (the query blocks of a key
// block) in ascending order: the wave reads 64 entries at a time, one byte
// per lane, and keeps the 64-bit ballot of the non-zero ones, so the scan
// state is wave-uniform and lives in scalar registers.
#pragma once

#include "common.h"

namespace ulysses {

constexpr int kSparseBlock = 128;   // tokens per layout block
// The dK/dV kernel lists a key block's active (query head, query block) pairs
// in LDS as g * 8192 + i: at most 8192 of them, query blocks below 8192 and at
// most 8 query heads per K/V head.
constexpr int kMaxSparsePairs = 8192;
constexpr int kMaxSparseGroup = 8;
// Heavily attended key block columns are cut into chunks of this many
// (query head, query block) pairs, using at most kSparseSlots partial-sum
// slots of [2][128][d_h] fp32 each; a split column has at least two chunks.
constexpr int kSparseChunk = 32;
constexpr int kSparseSlots = 512;
constexpr int kMaxSplitColumns = kSparseSlots / 2;

// The backward pass's work plan for block layouts, in the workspace. A layout
// column is (K/V head hk, key block kb), index hk * nb + kb, shared by the
// batch; a work column adds the batch: (b * H_kv + hk) * nb + kb.
struct SparsePlan {
  int* cnt;               // [H_kv * nb] active pairs of each layout column
  uint16_t* colpairs;     // [H_kv * nb][G * nb] those pairs, g * 8192 + i, ascending
  int* header;            // [0]: dK/dV work items, [1]: split work columns
  int4* items;            // (work column, chunk, chunks of the column, first slot)
  int* split_col;         // [kMaxSplitColumns] work column of each split
  int* split_slot;        // its first slot
  int* split_nch;         // its chunks (= slots)
  float* partials;        // [kSparseSlots][2][128][d_h]
};

struct LayoutScan {
  const uint8_t* p;   // entry 0 of the row or column
  int stride;         // bytes between consecutive entries (1 for a row, nb for a column)
  int lim;            // entries [0, lim) are visited
  int base;           // first entry of the current 64-entry window
  uint64_t bits;      // active entries of the window not yet returned

  __device__ void reset(const uint8_t* p_, int stride_, int start, int lim_) {
    p = p_;
    stride = stride_;
    lim = lim_;
    base = start - 64;
    bits = 0;
  }

  // next active entry (ascending), or -1 when none is left
  __device__ int next(int lane) {
    while (bits == 0) {
      base += 64;
      if (base >= lim) return -1;
      const int e = base + lane;
      bits = __ballot(e < lim && p[(size_t)e * stride] != 0);
    }
    const int e = base + __builtin_ctzll(bits);
    bits &= bits - 1;
    return e;
  }
};

}  // namespace ulysses
