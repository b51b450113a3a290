/*
 * csa2.h -- C ABI of the CSA2 decode hot path on MI355X (gfx950).
 *
 * CSA2 (Compressed Sparse Attention 2) keeps one 512-channel latent per
 * global KV entry, shared by every query head and used as both key and value,
 * stored as FP4 E2M1 with one FP8 E4M3 scale per 16 channels and no second
 * level scale; a 32-head x 128-dim sparse indexer picks the top 512 entries
 * (optionally coarse-to-fine through 8-position blocks) and attention runs
 * over them jointly with a 128-token FP8 sliding window.  Sources (web pages):
 *   [0539edu §3]  http://www.0539edu.com/news/5732216/ , section 3: the
 *                 inference configuration (cache dtypes, scale granularity,
 *                 window, indexer heads/dim/top-k, hierarchical blocks and
 *                 candidate pool, layer groups and compression ratios).
 *   [nxbn §4.2]   http://m.nxbn.cn/news/78290 , §4.2: the main key
 *                 compressor pools m tokens with context-dependent weights.
 *   [daiw]        https://daiw.net/manual/deepseek-v4-flash/million-token-cost ,
 *                 "four factors" table: one 512-dim latent shared by all
 *                 query heads; encoder m = 2, decoder m = 1.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  Scratch space is a caller-owned
 *     device workspace whose size the matching *_workspace call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; results are ready after the stream is
 *     synchronised.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     non-zero status nothing was enqueued and csa2_last_error() (per calling
 *     thread) describes the problem.  Device faults surface at the caller's
 *     next synchronisation.
 *   - Pointers must be 16-byte aligned except where noted.
 *   - No C++ exception crosses this boundary.  Calls are re-entrant; two
 *     calls that share a workspace must be ordered on one stream.
 *
 * Layouts (row-major, innermost last; S = sequences, N = entries per
 * sequence, R = query rows, H = attention heads):
 *   FP4 codes   uint8 [S][N][256]  byte j holds channel 2j in its low nibble
 *                                  and channel 2j+1 in its high nibble
 *   FP4 scales  uint8 [S][N][32]   E4M3FN scale of channels 16g..16g+15
 *   index keys  uint8 [S][N][128]  E4M3FN, one 128-dim key per entry shared
 *                                  by the 32 indexer heads
 *   block keys  uint8 [S][ceil(N/8)][128] E4M3FN block summaries
 *   SWA tokens  uint8 [S][cap][512] E4M3FN ring buffer
 * E4M3 is the OCP "FN" variant (max 448, no inf); values rounded into it use
 * round-to-nearest-even, saturate at +-448 and never produce -0.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 2

/* Status codes. */
#define CSA2_OK 0
#define CSA2_EINVAL 1        /* null/misaligned pointer, bad size or shape      */
#define CSA2_EUNSUPPORTED 2  /* valid request outside what the kernels support  */
#define CSA2_EWORKSPACE 3    /* workspace smaller than *_workspace reported     */
#define CSA2_EHIP 4          /* the HIP runtime refused a launch                */

/* Fixed dimensions of the method [0539edu §3; daiw]. */
#define CSA2_LATENT_DIM 512
#define CSA2_SCALE_GROUP 16
#define CSA2_IDX_HEADS 32
#define CSA2_IDX_DIM 128
#define CSA2_BLOCK_POS 8
#define CSA2_MAX_TOPK 2048

/* Version of this ABI (CSA2_ABI_VERSION of the built library). */
int32_t csa2_abi_version(void);

/* Static text for a status code. */
const char* csa2_status_string(int32_t status);

/* Detail of the last non-zero status returned on the calling thread
 * ("" if none).  The pointer stays valid until the thread's next call. */
const char* csa2_last_error(void);

/*
 * Cache write [0539edu §3 (fp4_e2m1, e4m3_per_16_channel, compression_ratio);
 * nxbn §4.2 (context-weighted pooling)].
 *
 * For every sequence s and group g of m consecutive tokens, per channel c:
 *   y_c = sum_j softmax_j(gate[s][g*m+j][c]) * x[s][g*m+j][c]   (m > 1)
 *   y_c = x[s][g][c]                                            (m = 1)
 * with equal weights (the mean) when gate is NULL; pooling runs in float32.
 * Then per 16-channel group: scale = E4M3(amax / 6) (float32 division),
 * each value rounded to the nearest of {0,.5,1,1.5,2,3,4,6} * scale with ties
 * to the even code, sign kept except on zero; a zero scale gives zero codes.
 *
 *   x_bf16, gate_bf16 : bf16 [n_seq][x_seq_stride tokens][512]; gate may be NULL
 *   n_tok             : tokens per sequence to consume; a trailing group of
 *                       fewer than m tokens is not emitted (n_tok/m entries)
 *   m                 : 1, 2 or 4
 *   x_seq_stride      : tokens between consecutive sequences in x/gate
 *                       (0 = n_tok)
 *   codes, scales     : entry e of sequence s goes to
 *                       codes + (s*out_seq_stride + e)*256 and
 *                       scales + (s*out_seq_stride + e)*32
 *   out_seq_stride    : entries between consecutive sequences in the output
 *                       (0 = n_tok/m); lets a decode step append in place.
 * codes/scales need only 8-byte alignment.
 */
int32_t csa2_kv_compress_quantize(const void* x_bf16, const void* gate_bf16, int64_t n_seq,
                                  int64_t n_tok, int32_t m, int64_t x_seq_stride,
                                  uint8_t* codes, uint8_t* scales, int64_t out_seq_stride,
                                  void* stream);

/*
 * Block summaries of the index keys for the hierarchical indexer
 * [0539edu §3, positions_per_block = 8]: block b of sequence s gets the mean
 * of the decoded keys of its members [8b, min(8b+8, n_ent)) (exact float32
 * sum divided by the member count in float32), rounded to E4M3.
 * Only blocks [blk_begin, blk_end) are written, so a decode step can refresh
 * the one block its new entry falls in.
 *   keys : uint8 [n_seq][n_ent][128];  summ : uint8 [n_seq][ceil(n_ent/8)][128]
 */
int32_t csa2_index_block_summary(const uint8_t* keys, int64_t n_seq, int64_t n_ent,
                                 int64_t blk_begin, int64_t blk_end, uint8_t* summ,
                                 void* stream);

/*
 * FP4 index keys [daiw "four generations" table: 890 B/token of global
 * cache = 2.5 entries/token x (288 B main entry + 68 B index key)]: each
 * 128-dim key is stored as 128 E2M1 codes (64 B, channel 2j in the low nibble
 * of byte j) and one E4M3 scale per 32 channels (4 B), quantised by the
 * main-KV rule (scale = E4M3(amax/6), nearest grid point, ties to the even
 * code, saturate at 6*scale, no -0).
 *   k_bf16       : bf16 [n_seq][k_seq_stride][128]; k_seq_stride 0 = n_ent
 *   codes        : uint8 [n_seq][out_seq_stride][64]   (16-byte aligned)
 *   scales       : uint8 [n_seq][out_seq_stride][4];   out_seq_stride 0 = n_ent
 * The indexer reads them with key_format = CSA2_KEY_FP4.
 */
int32_t csa2_index_key_quantize(const void* k_bf16, int64_t n_seq, int64_t n_ent, int64_t k_seq_stride,
                                uint8_t* codes, uint8_t* scales, int64_t out_seq_stride, void* stream);

/*
 * Block summaries of FP4 index keys: as csa2_index_block_summary, from the
 * decoded FP4 members (float32 mean, E4M3 rounding; E4M3 block keys).
 *   codes : uint8 [n_seq][n_ent][64];  scales : uint8 [n_seq][n_ent][4]
 *   summ  : uint8 [n_seq][ceil(n_ent/8)][128]
 */
int32_t csa2_index_block_summary_fp4(const uint8_t* codes, const uint8_t* scales, int64_t n_seq,
                                     int64_t n_ent, int64_t blk_begin, int64_t blk_end, uint8_t* summ,
                                     void* stream);

/*
 * Decode-time append: one generated token per row, written into a sequence's
 * caches in one launch [0539edu §3: compression_ratio 2 in the encoder and
 * 1 in the decoder, swa_window_size 128, FP8 window; nxbn §4.2 pooling].
 * For row r, sequence s = row_seq[r] (identity when NULL), position p = pos[r]:
 *   * window ring (when swa != NULL): swa[s][p % swa_cap] = E4M3 of the token
 *     (round to nearest even, saturating), as the prefill window reads it;
 *   * p % m < m-1: the group is still open; the token (and its gate logits)
 *     go to pend_x[s][p % m] (pend_gate[s][p % m]);
 *   * p % m == m-1: entry e = p / m completes from pend_x[s][0..m-2] and the
 *     token, pooled and quantised exactly as csa2_kv_compress_quantize
 *     (codes/scales[s][e]); its index key key_bf16[r] is stored as E4M3
 *     (round to nearest even, saturating) or FP4 (as csa2_index_key_quantize)
 *     in keys/key_scales[s][e]; with block_keys != NULL the summary of block
 *     e/8 is recomputed over its entries written so far, [8*(e/8), e], as
 *     csa2_index_block_summary(_fp4) with n_ent = e + 1.
 * With codes == NULL the call only writes windows (layers with no global
 * cache of their own): swa, swa_cap, pos and x are used, the rest ignored.
 * Rows whose sequence is outside [0, n_seq), whose position is negative or
 * whose entry would be at or past n_ent are skipped.  Two rows of one
 * sequence in one call race.  The pending buffers are the caller's but their
 * contents are the library's (bf16 tokens); keep them per cache.
 *   n_rows              : rows (tokens) in this call
 *   n_seq               : sequences in the caches
 *   row_seq, pos        : device int32 [R] (nullable), int64 [R]
 *   m                   : 1, 2 or 4
 *   x_bf16, gate_bf16   : bf16 [R][512]; gate nullable (equal weights)
 *   pend_x, pend_gate   : bf16 [n_seq][m-1][512]; pend_x required for m > 1,
 *                         pend_gate when gate_bf16 is given
 *   n_ent               : entries per sequence in codes/scales/keys
 *   codes, scales       : [n_seq][n_ent][256], [n_seq][n_ent][32]
 *   key_bf16            : bf16 [R][128]: the index key of the entry the row
 *                         completes (read only then)
 *   key_format          : CSA2_KEY_E4M3 (keys [n_seq][n_ent][128]) or
 *                         CSA2_KEY_FP4 (keys [n_seq][n_ent][64] codes,
 *                         key_scales [n_seq][n_ent][4])
 *   block_keys          : nullable, [n_seq][ceil(n_ent/8)][128] E4M3
 *   swa, swa_cap        : nullable, [n_seq][swa_cap][512] E4M3 ring
 * Alignment: x, gate, pending buffers 16 bytes; codes, keys 8; swa 4.
 * Status: EUNSUPPORTED for m or key_format outside the sets above, EINVAL
 * for missing or misaligned buffers and negative sizes.
 */
typedef struct {
  int32_t n_rows;
  int64_t n_seq;
  const int32_t* row_seq;
  const int64_t* pos;
  int32_t m;
  const void* x_bf16;
  const void* gate_bf16;
  void* pend_x;
  void* pend_gate;
  int64_t n_ent;
  uint8_t* codes;
  uint8_t* scales;
  const void* key_bf16;
  int32_t key_format;
  uint8_t* keys;
  uint8_t* key_scales;
  uint8_t* block_keys;
  uint8_t* swa;
  int32_t swa_cap;
} csa2_append_args;

int32_t csa2_decode_append(const csa2_append_args* args, void* stream);

/*
 * Indexer + top-k [0539edu §3, csa2.indexer and its hierarchical block].
 *
 * Row r scores entries of sequence row_seq[r] (r if NULL) that are visible to
 * it, t < n_valid[r] (n_ent if NULL):
 *   I_t = sum_{h<32} head_w[r][h] * max(0, sum_{i<128} q[r][h][i] * key[t][i])
 * (E4M3 x E4M3 products, float32 accumulation), and keeps the top_k entries
 * ordered by score descending then index ascending.  out_idx[r] receives the
 * kept indices in ascending order, padded with -1 when fewer than top_k are
 * visible; out_score (optional) the matching float32 scores (0 for padding).
 *
 * Modes (exactly one):
 *   flat          block_keys == NULL and cand == NULL.
 *   hierarchical  block_keys != NULL: score the ceil(n_valid/8) blocks,
 *                 keep the top min(keep_blocks, #blocks) (ties to the lower
 *                 block id), expand each to its positions below n_valid and
 *                 select among those.
 *   candidate     cand != NULL: select among cand[r][0..n_cand) (distinct
 *                 entry ids; -1 and ids >= n_valid are skipped), e.g. a pool
 *                 kept from an earlier layer.
 *   block pool    cand_blocks != NULL: select among the positions below
 *                 n_valid of the blocks cand_blocks[r][0..n_cand_blocks)
 *                 (block b covers entries 8b..8b+7; -1 skipped) -- the fine
 *                 stage of the hierarchical mode on a given block list.  With
 *                 the pool of a Full layer (its out_blocks) this restricts a
 *                 Reindex layer to that pool [0539edu §3: the candidate pool
 *                 bounds the indexer's work].  Output is ascending when the
 *                 list is (out_blocks is); otherwise it follows the list.
 * Supported: 1 <= top_k <= 2048, 1 <= keep_blocks <= 2048, and at most
 * 2^24 items per row in one stage (entries in flat mode, blocks in the
 * coarse stage, candidates in candidate mode, 8 per block in block-pool
 * mode).
 */
typedef struct {
  int32_t n_rows;           /* R >= 1                                           */
  int64_t n_seq;            /* S, sequences in keys (rows whose row_seq is
                               outside [0, S) see no entry)                     */
  const int32_t* row_seq;   /* [R] sequence of each row, or NULL (identity)     */
  const int32_t* n_valid;   /* [R] visible entries per row (clamped to
                               [0, n_ent]), or NULL (n_ent)                     */
  int64_t n_ent;            /* N, entries per sequence in keys                  */
  int32_t top_k;            /* k                                                */
  const uint8_t* q;         /* [R][32][128] E4M3 indexer queries                */
  const float* head_w;      /* [R][32] head weights, or NULL (all 1)            */
  const uint8_t* keys;      /* [S][N][128] E4M3 index keys                      */
  const uint8_t* block_keys;/* [S][ceil(N/8)][128] summaries, or NULL           */
  int32_t keep_blocks;      /* blocks kept by the coarse stage (e.g. 2048)      */
  const int32_t* cand;      /* [R][n_cand] candidate entry ids, or NULL         */
  int32_t n_cand;           /* candidates per row when cand != NULL             */
  int32_t* out_idx;         /* [R][k] kept entry ids, ascending, -1 padded      */
  float* out_score;         /* [R][k] their scores, or NULL                     */
  int32_t* out_blocks;      /* [R][keep_blocks] kept blocks (hierarchical mode,
                               ascending, -1 padded), or NULL                   */
  const int32_t* cand_blocks;/* [R][n_cand_blocks] block ids, or NULL           */
  int32_t n_cand_blocks;    /* blocks per row when cand_blocks != NULL          */
  int32_t key_format;       /* CSA2_KEY_E4M3 (keys [S][N][128]) or CSA2_KEY_FP4
                               (keys = codes [S][N][64], key_scales [S][N][4],
                               see csa2_index_key_quantize); block_keys are
                               E4M3 in both                                     */
  const uint8_t* key_scales;/* FP4 keys: [S][N][4] E4M3 scales, else NULL       */
} csa2_indexer_args;

#define CSA2_KEY_E4M3 0
#define CSA2_KEY_FP4 1

/* Workspace bytes csa2_indexer_topk needs for these arguments (0 on error).
 * Reads only the sizes and which of block_keys/cand/cand_blocks are set; data pointers
 * may still be NULL.
 *
 * The indexer workspace must be ZERO-FILLED before its first use.  It holds
 * per-row score histograms that each call builds up from zero and leaves at
 * zero when its kernels complete, so later calls
 * with the same n_rows and the same mode (flat, hierarchical or candidate)
 * can reuse it without clearing it again, also from a captured HIP graph.
 * Zero it again before a call with another n_rows or mode, and after a call
 * that returned CSA2_EHIP or a device fault.
 *
 * Size: score histograms and a float32 score block of one row per row, plus
 * a candidate area where a stage selects through the candidate filter (rows
 * over 32768 items in calls of fewer than 256 rows).  A one-stage call (flat,
 * cand or cand_blocks) whose score block would exceed 512 MiB runs its rows in
 * passes of equal size, at least 256 rows each, through one block of that
 * many rows: e.g. 4096 rows over 524,288 entries take 16 passes of 256 rows
 * and about 0.52 GB.  The passes give the results one pass of all rows gives. */
size_t csa2_indexer_topk_workspace(const csa2_indexer_args* args);

int32_t csa2_indexer_topk(const csa2_indexer_args* args, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * One decode step's cache append and selection [0539edu §3: the candidate
 * pool bounds the indexer's work; daiw "decode reads": decode is bound by
 * the bytes each step reads]: exactly csa2_decode_append(app) followed by
 * csa2_indexer_topk(idx) on the same stream, with the same validation,
 * results and errors (nothing is enqueued when either is invalid), and the
 * workspace of csa2_indexer_topk.  When the two describe the same rows of the
 * same caches with row r being sequence r -- idx hierarchical, app->codes
 * set, the same keys, key_scales, key format, block_keys, n_seq, n_ent and
 * n_rows, both row_seq NULL, m 1 or 2 -- the append runs inside the coarse
 * scan's launch (one extra workgroup per row), and the scan scores the block
 * the new entry falls in from its refreshed summary, computed by the
 * workgroup that owns it with the arithmetic of the append; the append then
 * costs no step of its own.  Otherwise (e.g. rows mapped by row_seq, where
 * one row may read a sequence another row appends to) the two run one after
 * the other.
 */
int32_t csa2_append_indexer_topk(const csa2_append_args* app, const csa2_indexer_args* idx, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Indexer + top-k that allocates nothing and takes no workspace: for callers
 * that cannot call hipMalloc (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Arguments, modes, results and
 * errors are those of csa2_indexer_topk.  Its scratch lives in a static
 * device array of CSA2_STATIC_SCRATCH_BYTES inside the library; each GPU the
 * library runs on holds its own copy until the process ends.
 *   - A call whose csa2_indexer_topk_workspace() exceeds
 *     CSA2_STATIC_SCRATCH_BYTES returns CSA2_EWORKSPACE before anything is
 *     enqueued (e.g. hierarchical rows over 2^20 entries need about 1.6 MiB
 *     each, so up to ~38 such rows fit).
 *   - Every call first clears the part of the array that must start at zero
 *     (the score histograms) with a small fill kernel on `stream`, then runs
 *     the kernels of csa2_indexer_topk.
 *   - All calls on one GPU share that GPU's array: calls that overlap on one
 *     GPU (unordered streams, several host threads) race and give wrong
 *     results.  Order them on one stream.
 */
#define CSA2_STATIC_SCRATCH_BYTES (64u << 20)

int32_t csa2_indexer_topk_static(const csa2_indexer_args* args, void* stream);

/*
 * Joint sparse + sliding-window attention for one decode step per row
 * [daiw "four factors" (one 512-dim latent shared by all heads);
 *  0539edu §3 (top_k, swa_window_size, fp8 SWA)].
 *
 * Keys = values = the latent: for row r the key set is the dequantised FP4
 * entries idx[r][0..top_k) of sequence row_seq[r] (entries < 0 skipped)
 * followed by the SWA tokens in slots (swa_start[r] + j) mod swa_cap,
 * j < min(swa_len[r], swa_max).  For every head h:
 *   s_t = sm_scale * q[r][h] . K_t,   out[r][h] = sum_t softmax(s)_t K_t,
 *   lse[r][h] = log(sum_t exp(s_t))   (natural log)
 * one softmax over all keys, float32 accumulation.  With no key the output
 * is 0 and lse = -inf.
 *   q_bf16 : bf16 [R][H][512];  out : float32 [R][H][512];  lse : [R][H] or NULL
 *   H in {16, 32, 64, 128};  sm_scale <= 0 selects 1/sqrt(512).
 *   swa may be NULL when every swa_len is 0 (swa_len NULL = no window).
 *   swa_max bounds the window of every row: the key splits are planned for
 *   top_k + swa_max keys per row (0 selects swa_cap).  A caller whose window
 *   buffer is larger than any one row's window (prefill rows reading one
 *   shared run of tokens, each its own 128) passes the window length here;
 *   without it every row is planned for swa_cap keys.
 */
typedef struct {
  int32_t n_rows;           /* R                                                */
  int32_t n_heads;          /* H                                                */
  int64_t n_seq;            /* S, sequences in the caches (rows whose row_seq
                               is outside [0, S) attend to nothing)             */
  const int32_t* row_seq;   /* [R] or NULL                                      */
  const void* q_bf16;       /* [R][H][512]                                      */
  const uint8_t* codes;     /* [S][N][256]                                      */
  const uint8_t* scales;    /* [S][N][32]                                       */
  int64_t n_ent;            /* N                                                */
  const int32_t* idx;       /* [R][top_k] selected entries, -1 skipped          */
  int32_t top_k;            /* 0..2048                                          */
  const uint8_t* swa;       /* [S][swa_cap][512] E4M3 or NULL                   */
  int32_t swa_cap;          /* ring capacity (>= max swa_len)                   */
  const int32_t* swa_start; /* [R] first slot, or NULL (0)                      */
  const int32_t* swa_len;   /* [R] tokens in the window, or NULL (none)         */
  float sm_scale;           /* softmax scale, <= 0 -> 1/sqrt(512)               */
  float* out;               /* [R][H][512] float32                              */
  float* lse;               /* [R][H] float32, or NULL                          */
  int32_t swa_max;          /* largest swa_len used, 0..swa_cap (0 = swa_cap);
                               longer windows are clamped to it                 */
} csa2_attn_args;

/*
 * Attention plan override, for tests and benchmarks that pin the geometry of
 * the attention kernels (every geometry computes the same function to the
 * precision stated above).  heads_per_wg: 16 (one 16-head group per
 * workgroup) or 64 (up to 64 heads per workgroup), 0 = chosen per call;
 * n_split: key splits per row, 1..64, 0 = chosen per call, raised to the
 * least count the chosen kernel supports (512 selected entries per split
 * with 16 heads, 1024 keys with 64).  Process-wide, for calls of csa2_sparse_attn_workspace and
 * csa2_sparse_attn_decode made after it; (0, 0) restores the automatic plan.
 * Returns CSA2_EINVAL for other values and changes nothing then.
 */
int32_t csa2_attn_plan_override(int32_t heads_per_wg, int32_t n_split);

/* Workspace bytes csa2_sparse_attn_decode needs (0 on error or if none).
 * Reads only the sizes and whether swa_len is set. */
size_t csa2_sparse_attn_workspace(const csa2_attn_args* args);

int32_t csa2_sparse_attn_decode(const csa2_attn_args* args, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Instrumentation (for benchmarks and profiling; not needed for computing).
 *
 * csa2_kernel_timer_start(site, max_launches) arms a timer on one launch
 * site: each of the next `max_launches` launches made from that site is
 * bracketed by two HIP events recorded on the stream the kernel is launched
 * on (created with hipEventDisableSystemFence: they order nothing beyond the
 * stream and only measure).  csa2_kernel_timer_stop() waits for those events,
 * returns how many
 * launches were timed and their summed duration in milliseconds, and
 * disarms the timer.  One timer per process; arm it outside HIP graph
 * capture.  Sites:
 */
#define CSA2_SITE_KV_QUANT 1       /* cache write                               */
#define CSA2_SITE_BLOCK_SUMMARY 2  /* block summaries                           */
#define CSA2_SITE_SCORE_FLAT 3     /* indexer scan, flat mode                   */
#define CSA2_SITE_SCORE_COARSE 4   /* indexer scan over block summaries         */
#define CSA2_SITE_SCORE_POOL 5     /* indexer scan over the kept blocks' pool   */
#define CSA2_SITE_SCORE_CAND 6     /* indexer scan over a candidate list        */
#define CSA2_SITE_SELECT 7         /* top-k exact selection (every stage)       */
#define CSA2_SITE_ATTN 8           /* sparse + window attention                 */
#define CSA2_SITE_ATTN_COMBINE 9   /* merge of the attention key splits         */
#define CSA2_SITE_FILTER 10        /* top-k candidate filter (every stage)      */
#define CSA2_SITE_APPEND 11        /* decode-time append                        */

int32_t csa2_kernel_timer_start(int32_t site, int32_t max_launches);
int32_t csa2_kernel_timer_stop(int32_t* n_launches, float* total_ms);

/*
 * Matrix-core precision probe (diagnostics) [0539edu §3: the indexer's head
 * scores are q . k over 128 dims with E4M3 operands and float32 accumulation].
 * For every pair (i, j) of q [n_q][128] and k [n_k][128] (E4M3 bytes, device
 * memory, 16-byte aligned) writes, on `stream`, the 128-term dot product
 * computed two ways: out_f16[i][j] by widening to fp16 and summing with
 * v_mfma_f32_16x16x32_f16 in four steps (the indexer's arithmetic), and
 * out_f8[i][j] by one v_mfma_scale_f32_16x16x128_f8f6f4 on the E4M3 bytes
 * with unit scales.  n_q and n_k: positive multiples of 16, at most 2^20.
 * Outputs float32 [n_q][n_k], caller-owned.  Returns CSA2_EINVAL for other
 * sizes or null/misaligned pointers, CSA2_EHIP if the launch fails.
 */
int32_t csa2_mfma_dot_probe(const uint8_t* q, const uint8_t* k, int32_t n_q, int32_t n_k, float* out_f16,
                            float* out_f8, void* stream);

/*
 * Timing probes (diagnostics).  Each launches one read-only or arithmetic
 * kernel on `stream` whose only output is one word per thread (XOR of the
 * data read, or the accumulators), so that a caller can time the shape of
 * work a hot kernel is built from; `bench.py --probe` prints their tables.
 * Null or misaligned pointers and sizes outside the stated ranges return
 * CSA2_EINVAL before any launch; a failed launch returns CSA2_EHIP.
 *
 * csa2_probe_scan_read [0539edu §3: the coarse stage streams the 128-byte
 * E4M3 block summaries of each row]: reads keys [n_rows][n_keys][128] in
 * chunks of `chunk` keys per 256-thread workgroup (n_rows * ceil(n_keys /
 * chunk) <= 2^20 workgroups, 16 <= chunk, n_keys <= 2^24), four 16-key tiles
 * per wave and two groups in flight; full_lines = 0: each lane reads 32
 * bytes of one key (two loads, each touching half of 16 lines), else each
 * load reads 8 whole keys; nontemporal != 0: non-temporal loads.  keys
 * 16-byte aligned; out uint32 [workgroups * 256].
 *
 * csa2_probe_mfma_valu: n_wg workgroups of `threads` (256 or 512) threads,
 * each wave running `iters` x 8 dependent v_mfma_f32_32x32x16_f16 with n_valu
 * (0, 4, 8, 12 or 16) independent float FMAs after each; iters in [1, 2^20],
 * n_wg in [1, 65536]; out float [n_wg * threads].
 *
 * csa2_probe_gather [0539edu §3: the attention gathers the selected entries,
 * 256 FP4 code bytes and 32 E4M3 scale bytes each]: n_wg 128-thread
 * workgroups (at most 65536) walk rows blockIdx, blockIdx + n_wg, ... of ids
 * [n_rows][512] (clamped into [0, n_ent), n_ent <= 2^31), 32 ids per chunk,
 * four chunks of loads in flight; whole_lines = 0: the attention kernels'
 * lane mapping (4 x 16 code bytes and 8 scale bytes of a quarter entry per
 * lane), else 16 lanes read one entry's 256 code bytes (whole lines) and 4
 * scale bytes each.  codes [n_ent][256] and scales [n_ent][32] 16-byte
 * aligned, ids 4-byte aligned; out uint32 [n_wg * 128].
 */
int32_t csa2_probe_scan_read(const uint8_t* keys, int32_t n_rows, int32_t n_keys, int32_t chunk, int32_t full_lines,
                             int32_t nontemporal, uint32_t* out, void* stream);
int32_t csa2_probe_mfma_valu(int32_t n_valu, int32_t threads, int32_t iters, int32_t n_wg, float* out, void* stream);
int32_t csa2_probe_gather(const uint8_t* codes, const uint8_t* scales, int64_t n_ent, const int32_t* ids,
                          int32_t n_rows, int32_t n_wg, int32_t whole_lines, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
