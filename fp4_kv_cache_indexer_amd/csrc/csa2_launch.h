// Host-side launchers of the CSA2 kernels (internal to libcsa2.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

hipError_t launch_kv_compress_quantize(const void* x, const void* z, int64_t n_seq, int64_t n_ent,
                                       int32_t m, int64_t x_seq_stride, uint8_t* codes,
                                       uint8_t* scales, int64_t out_seq_stride, hipStream_t stream);

hipError_t launch_index_key_quantize(const void* k, int64_t n_seq, int64_t n_ent, int64_t k_seq_stride,
                                     uint8_t* codes, uint8_t* scales, int64_t out_seq_stride,
                                     hipStream_t stream);
hipError_t launch_block_summary_fp4(const uint8_t* codes, const uint8_t* scales, int64_t n_seq,
                                    int64_t n_ent, int64_t blk_begin, int64_t blk_end, uint8_t* summ,
                                    hipStream_t stream);
hipError_t launch_block_summary(const uint8_t* keys, int64_t n_seq, int64_t n_ent,
                                int64_t blk_begin, int64_t blk_end, uint8_t* summ,
                                hipStream_t stream);


// Which items a row of the score/select kernels walks and how they map to
// cache positions.
enum ItemMode : int32_t {
  kItemsFlat = 0,    // item i = entry i, rows walk [0, n_valid)
  kItemsBlocks = 1,  // item i = block i, rows walk [0, ceil(n_valid/8))
  kItemsPool = 2,    // item i = position blocks[i/8]*8 + i%8 (invalid -> NaN score)
  kItemsCand = 3,    // item i = cand[i] (invalid -> NaN score)
};

struct ItemMap {
  // A row's two words come from these arrays; the kernels load both at once
  // and unconditionally, an absent array reading the word at `any` (a
  // readable address; the value is discarded).  Kept together at the front
  // so that one scalar load fetches the three pointers.
  const int32_t* row_seq;   // [R] or null (row r reads sequence row_base + r)
  const int32_t* n_valid;   // [R] or null
  const void* any;          // readable stand-in address (non-null)
  int32_t mode;
  int32_t n_items;          // item stride per row (scores row length)
  int64_t n_seq;            // rows whose sequence is outside [0, n_seq) see nothing
  int64_t row_base;         // first row of this launch among the call's rows
  int64_t n_ent;            // default n_valid
  const int32_t* list;      // kept blocks [R][list_len] or cand [R][list_len]
  int32_t list_len;
};

constexpr int kFiltChunk = 4096;          // items per filter workgroup
constexpr int64_t kMaxItems = 1LL << 24;  // items one top-k stage walks per row

// One new token per row: window ring, pending group or a completed entry
// with its index key and block summary.
struct AppendArgs {
  int32_t n_rows;
  int64_t n_seq;
  const int32_t* row_seq;
  const int64_t* pos;
  int32_t m;
  const uint16_t* x;
  const uint16_t* gate;
  uint16_t* pend_x;
  uint16_t* pend_gate;
  int64_t n_ent;
  uint8_t* codes;
  uint8_t* scales;
  const uint16_t* key;
  bool key_fp4;
  uint8_t* keys;
  uint8_t* key_scales;
  uint8_t* block_keys;
  uint8_t* swa;
  int32_t swa_cap;
};

struct ScoreArgs {
  ItemMap im;
  int32_t row_stride;       // floats between score rows (multiple of 4)
  int32_t n_rows;
  int64_t n_seq;
  const int32_t* row_seq;
  const uint8_t* keys;      // key rows (index keys, or block keys in kItemsBlocks mode)
  const uint8_t* key_scales;// FP4 index keys: [S][seq_rows][4] E4M3 scales
  int32_t key_fp4;          // index keys are FP4 (codes in `keys`, 64 B per row)
  int64_t seq_rows;         // key rows per sequence in `keys`
  const uint8_t* q;         // [R][32][128]
  const float* w;           // [R][32] or null
  float* scores;            // [R][n_items]
  uint32_t* hist;           // [R][kHistBins]
  int32_t chunk;            // items per workgroup
  // The decode step's append (coarse stage only): row r's token is appended
  // by an extra workgroup of row r (the grid's last column), and the
  // workgroup whose chunk holds the block of the entry the token completes
  // scores that block's refreshed summary, computed in its own registers.
  int32_t fuse_append;      // 0 or 1
  AppendArgs app;
};

struct SelectArgs {
  ItemMap im;
  int32_t n_rows;
  int32_t k;
  int32_t row_stride;       // floats between score rows (multiple of 4)
  const float* scores;      // [R][row_stride]
  uint32_t* hist;           // [R][kHistBins], zeroed after use
  uint64_t* cand;           // [R][n_chunks][kFiltChunk] candidate composite keys, or null
                            // (then a row select never spills its candidates to memory)
  uint32_t* cand_count;     // [R][n_chunks], or null with cand
  int32_t n_chunks;         // ceil(n_items / kFiltChunk)
  int32_t* out_idx;         // [R][k]
  float* out_score;         // [R][k] or null
};

hipError_t launch_index_score(const ScoreArgs& a, hipStream_t stream);
// Flat E4M3 scans of many rows over a one-sequence cache (a prefill chunk)
// score groups of rows per key tile (index_score_rows_kernel).
constexpr int32_t kScoreRowsMin = 256;
bool score_rows_path(const ScoreArgs& a);
int score_resident_wgs();
hipError_t launch_topk_filter(const SelectArgs& a, hipStream_t stream);
hipError_t launch_topk_select(const SelectArgs& a, hipStream_t stream);
// whole-row top-k (filter + select in one workgroup per row); preferred up to
// kRowMaxItems items per row or from kRowMinRows rows
constexpr int64_t kRowMaxItems = 1 << 15;
constexpr int32_t kRowMinRows = 256;
hipError_t launch_topk_row(const SelectArgs& a, hipStream_t stream);
// Zero n 32-bit words with a fill kernel (no memset node: the call may be
// captured into a graph).
hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t stream);

struct AttnArgs {
  // the per-row arrays (each [R] or null) and Q, whose first word stands in
  // for an absent row word (a row's words are loaded at once, unconditionally)
  const int32_t* row_seq;
  const int32_t* swa_start;
  const int32_t* swa_len;
  const uint16_t* q;
  int32_t n_rows, n_heads;
  int64_t n_seq;
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t n_ent;
  const int32_t* idx;
  int32_t top_k;
  const uint8_t* swa;
  int32_t swa_cap;
  int32_t swa_max;          // window lengths are clamped to this (<= swa_cap)
  float sm_scale_log2;      // sm_scale * log2(e)
  float* out;
  float* lse;
  int32_t heads_per_wg;     // heads one workgroup owns: 16 or 64
  int32_t n_split;          // key splits per row
  int32_t keys_per_split;   // multiple of the key chunk
  float* part_o;            // [n_split][R][H][512] when n_split > 1
  float* part_ml;           // [n_split][R][H][2]
  int32_t xcd_block;        // set by the launcher of the 16-head kernel: work items per XCD
};

hipError_t launch_decode_append(const AppendArgs& a, hipStream_t stream);

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream);
hipError_t launch_sparse_attn_narrow(const AttnArgs& a, hipStream_t stream);   // 16 heads per workgroup
hipError_t launch_sparse_attn_tile(const AttnArgs& a, hipStream_t stream);     // 64 heads, 32x32 MFMA tiles
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t stream);
hipError_t launch_mfma_dot_probe(const uint8_t* q, const uint8_t* k, int32_t n_q, int32_t n_k, float* out16,
                                 float* out8, hipStream_t stream);
hipError_t launch_scan_read_probe(const uint8_t* keys, int32_t n_rows, int32_t n_keys, int32_t chunk, bool full,
                                  bool nt, uint32_t* out, hipStream_t stream);
hipError_t launch_mfma_valu_probe(int32_t n_valu, int32_t threads, int32_t iters, int32_t n_wg, float* out,
                                  hipStream_t stream);
hipError_t launch_gather_probe(const uint8_t* codes, const uint8_t* scales, int64_t n_ent, const int32_t* ids,
                               int32_t n_rows, int32_t n_wg, bool whole, uint32_t* out, hipStream_t stream);

}  // namespace csa2
