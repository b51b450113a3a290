// Row and item mapping shared by the indexer's score and top-k kernels: the
// sequence and visible entries of a query row, and the position (entry or
// block id) behind each item a row walks in flat, block, pool and candidate
// mode.
#pragma once

#include "csa2_dev.h"
#include "csa2_launch.h"

namespace csa2 {

// ---------------------------------------------------------------------------
// item <-> position mapping
// ---------------------------------------------------------------------------

// Entries visible to row r: n_valid clamped to [0, n_ent]; none if the row's
// sequence (row_seq[r], or row_base + r) is not in the cache.  The row's
// sequence goes to *seq_out when asked for.
__device__ __forceinline__ int64_t row_valid(const ItemMap& im, int r, int64_t* seq_out = nullptr) {
  int32_t vs, vn;
  scalar_words2(row_word_ptr(im.row_seq, r, im.any), row_word_ptr(im.n_valid, r, im.any), vs, vn);
  const int64_t seq = im.row_seq ? (int64_t)vs : im.row_base + r;
  if (seq_out) *seq_out = seq;
  const int64_t nv = im.n_valid ? (int64_t)vn : im.n_ent;
  const int64_t c = nv < 0 ? 0 : (nv > im.n_ent ? im.n_ent : nv);
  return (seq < 0 || seq >= im.n_seq) ? 0 : c;
}

// Items row walks.  A row that sees no entry (n_valid 0, or a sequence
// outside the cache) walks none in every mode: pool and candidate items
// would otherwise be addressed from an invalid sequence's keys.
__device__ __forceinline__ int64_t row_items(const ItemMap& im, int64_t nv) {
  if (nv <= 0) return 0;
  if (im.mode == kItemsFlat) return nv;
  if (im.mode == kItemsBlocks) return (nv + kBlockPos - 1) / kBlockPos;
  return im.n_items;
}

// Position (entry or block id) of item i of row r, or -1 if the item is not
// visible to the row.
__device__ __forceinline__ int64_t item_pos(const ItemMap& im, int r, int64_t i, int64_t nv) {
  if (im.mode == kItemsFlat || im.mode == kItemsBlocks) return i;
  if (im.mode == kItemsPool) {
    const int32_t b = im.list[(int64_t)r * im.list_len + (i >> 3)];
    const int64_t p = (int64_t)b * kBlockPos + (i & 7);
    return (b >= 0 && p < nv) ? p : -1;
  }
  const int32_t c = im.list[(int64_t)r * im.list_len + i];
  return (c >= 0 && (int64_t)c < nv) ? (int64_t)c : -1;
}

}  // namespace csa2
