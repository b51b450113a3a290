// C ABI of libcsa2.so: argument validation, workspace layout and launch
// order.  Every check runs on the host before anything is enqueued; a
// non-zero status means nothing was launched (see include/csa2.h).
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "csa2.h"
#include "csa2_dev.h"
#include "csa2_launch.h"

namespace {

thread_local std::string g_err;

int32_t fail(int32_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(CSA2_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- launch-site timer -----------------------------------------------------

struct SiteTimer {
  int32_t site = 0;
  int32_t used = 0;
  std::vector<hipEvent_t> ev;   // begin/end pairs
};
SiteTimer g_timer;

void timer_mark(int32_t site, hipStream_t s, bool end) {
  if (g_timer.site != site) return;
  const size_t i = 2 * (size_t)g_timer.used + (end ? 1 : 0);
  if (i >= g_timer.ev.size()) return;
  (void)hipEventRecord(g_timer.ev[i], s);   // a failed record shows up when the timer is read
  if (end) ++g_timer.used;
}

// Launch through f() with the site's timer events around it.
template <class F>
hipError_t timed(int32_t site, hipStream_t s, F f) {
  timer_mark(site, s, false);
  hipError_t e = f();
  timer_mark(site, s, true);
  return e;
}

// 16-head attention workgroups that run at once (two per CU of MI355X), and
// the most keys one of them takes.
#ifndef CSA2_RESIDENT_ATTN_WGS
#define CSA2_RESIDENT_ATTN_WGS 512
#endif
// (measured with the combine: 32 rows x 64 heads in 5-chunk narrow splits
// 27.6 + 7.9 us against 24.2 + 10.1 us wide; 64 rows in 10-chunk splits
// 40.5 + 10.6 against 32.6 + 11.7; 8 rows in 2-chunk splits 14.3 + 5.7
// against 19.9 + 5.6)
#define CSA2_NARROW_MAX_SPLIT_KEYS 128

// Fewest keys one attention workgroup takes when a row is split.
#ifndef CSA2_MIN_SPLIT_KEYS
#define CSA2_MIN_SPLIT_KEYS 64
#endif
// 16-head splits are not made shorter than this many keys (three chunks)
// just to have more workgroups than compute units (MI355X: 256).  Measured
// on 8 rows x 64 heads x 640 keys: 7 splits of 96 keys against 10 of 64,
// attention + combine 15.6 against 16.2 us and the 40-layer step 0.985
// against 1.029 ms; one 16-head row keeps its 10 splits (10 workgroups).
#define CSA2_ATTN_CUS 256
#define CSA2_NARROW_CU_SPLIT_KEYS 96
// 64-head splits take at least this many keys (four chunks: the pipeline's
// depth).  Measured on 32 rows x 64 heads x 640 keys: 5 splits of 128 keys
// against 7 of 96, step 110.6 against 112.6 us (the combine reads fewer
// partials); 64 rows keep 4 splits of 160.
#define CSA2_WIDE_MIN_SPLIT_KEYS 128

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- indexer workspace layout ---------------------------------------------

struct IndexerPlan {
  int mode;                 // 0 flat, 1 hierarchical, 2 candidate, 3 block pool
  int64_t R, N, NB;
  int32_t keep;
  int32_t items0, items1;   // items a row walks in stage 0 / 1
  int32_t stride0, stride1; // score row strides (floats, multiple of 4)
  int32_t chunks;           // filter chunks per row (max over stages)
  int64_t group_rows;       // rows per pass of a one-stage call (R if a single pass)
  size_t off_hist0, off_hist1, off_scores0, off_scores1, off_blocks, off_cand, off_count, total;
  bool has_cand;            // the candidate area exists (some stage filters)
};

// Score rows of a one-stage call held at once: a call whose score block
// would exceed this runs its rows in passes of at least kRowMinRows rows
// (the row-group scan and the long-row select still apply to every pass).
constexpr size_t kScoreBlockBudget = (size_t)512 << 20;

// Whether a stage of `rows` rows over `items` items selects through the
// candidate filter (and needs its candidate area).
bool uses_filter(int64_t items, int64_t rows) {
  return items > csa2::kRowMaxItems && rows < csa2::kRowMinRows;
}

int32_t check_indexer(const csa2_indexer_args* a, IndexerPlan* p, bool check_ptrs) {
  if (!a) return fail(CSA2_EINVAL, "indexer: args is NULL");
  if (a->n_rows < 0) return fail(CSA2_EINVAL, "indexer: n_rows < 0");
  if (a->n_seq < 0) return fail(CSA2_EINVAL, "indexer: n_seq < 0");
  if (a->n_ent < 0 || a->n_ent > 0x7FFFFFF0LL) return fail(CSA2_EINVAL, "indexer: n_ent out of range");
  if (a->top_k < 1 || a->top_k > CSA2_MAX_TOPK)
    return fail(CSA2_EUNSUPPORTED, "indexer: top_k %d outside [1, %d]", a->top_k, CSA2_MAX_TOPK);
  if ((a->block_keys != nullptr) + (a->cand != nullptr) + (a->cand_blocks != nullptr) > 1)
    return fail(CSA2_EINVAL, "indexer: block_keys, cand and cand_blocks are exclusive");
  if (a->key_format != CSA2_KEY_E4M3 && a->key_format != CSA2_KEY_FP4)
    return fail(CSA2_EUNSUPPORTED, "indexer: key_format %d unknown", a->key_format);
  if (check_ptrs && a->n_rows > 0 && a->key_format == CSA2_KEY_FP4 &&
      (!a->key_scales || !aligned(a->key_scales, 4)))
    return fail(CSA2_EINVAL, "indexer: FP4 keys need 4-byte aligned key_scales");
  if (a->n_rows > 0 && check_ptrs) {
    if (!a->q || !a->keys || !a->out_idx) return fail(CSA2_EINVAL, "indexer: q, keys and out_idx are required");
    if (!aligned(a->q, 16) || !aligned(a->keys, 16)) return fail(CSA2_EINVAL, "indexer: q/keys not 16-byte aligned");
    if (!aligned(a->out_idx, 4) || (a->out_score && !aligned(a->out_score, 4)) ||
        (a->head_w && !aligned(a->head_w, 4)))
      return fail(CSA2_EINVAL, "indexer: out_idx/out_score/head_w not 4-byte aligned");
  }
  p->R = a->n_rows;
  p->N = a->n_ent;
  p->NB = (a->n_ent + CSA2_BLOCK_POS - 1) / CSA2_BLOCK_POS;
  p->keep = 0;
  p->items1 = 0;
  if (a->block_keys) {
    if (a->keep_blocks < 1 || a->keep_blocks > CSA2_MAX_TOPK)
      return fail(CSA2_EUNSUPPORTED, "indexer: keep_blocks %d outside [1, %d]", a->keep_blocks, CSA2_MAX_TOPK);
    if (check_ptrs && !aligned(a->block_keys, 16)) return fail(CSA2_EINVAL, "indexer: block_keys not 16-byte aligned");
    if (check_ptrs && a->out_blocks && !aligned(a->out_blocks, 4)) return fail(CSA2_EINVAL, "indexer: out_blocks not aligned");
    p->mode = 1;
    p->keep = a->keep_blocks;
    p->items0 = (int32_t)p->NB;
    p->items1 = a->keep_blocks * CSA2_BLOCK_POS;
  } else if (a->cand_blocks) {
    if (a->n_cand_blocks < 1 || a->n_cand_blocks > csa2::kMaxItems / CSA2_BLOCK_POS)
      return fail(CSA2_EINVAL, "indexer: n_cand_blocks %d outside [1, %lld]", a->n_cand_blocks,
                  (long long)(csa2::kMaxItems / CSA2_BLOCK_POS));
    if (check_ptrs && !aligned(a->cand_blocks, 4)) return fail(CSA2_EINVAL, "indexer: cand_blocks not 4-byte aligned");
    p->mode = 3;
    p->items0 = a->n_cand_blocks * CSA2_BLOCK_POS;
  } else if (a->cand) {
    if (a->n_cand < 1) return fail(CSA2_EINVAL, "indexer: n_cand < 1 with cand set");
    if (check_ptrs && !aligned(a->cand, 4)) return fail(CSA2_EINVAL, "indexer: cand not 4-byte aligned");
    p->mode = 2;
    p->items0 = a->n_cand;
  } else {
    p->mode = 0;
    p->items0 = (int32_t)p->N;
  }
  if (p->items0 > csa2::kMaxItems)
    return fail(CSA2_EUNSUPPORTED, "indexer: %d items per row in one stage exceed %lld",
                p->items0, (long long)csa2::kMaxItems);
  p->stride0 = (int32_t)round_up((size_t)p->items0, 4);
  p->stride1 = (int32_t)round_up((size_t)p->items1, 4);
  const int64_t imax = p->items0 > p->items1 ? p->items0 : p->items1;
  p->chunks = (int32_t)((imax + csa2::kFiltChunk - 1) / csa2::kFiltChunk);
  // rows per pass: every row at once unless a one-stage call's score block
  // exceeds the budget; then passes of ceil(R / n) rows, n as small as keeps
  // them within the budget but no pass below kRowMinRows rows
  p->group_rows = p->R;
  const size_t row_bytes = (size_t)p->stride0 * 4;
  if (p->mode != 1 && p->R > 0 && (size_t)p->R * row_bytes > kScoreBlockBudget) {
    const int64_t target = std::max<int64_t>(csa2::kRowMinRows, (int64_t)(kScoreBlockBudget / row_bytes));
    int64_t passes = (p->R + target - 1) / target;
    passes = std::min<int64_t>(passes, std::max<int64_t>(1, p->R / csa2::kRowMinRows));
    p->group_rows = (p->R + passes - 1) / passes;
  }
  const int64_t G = p->group_rows;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = round_up(off + bytes, 256); return o; };
  const size_t hist = (size_t)G * csa2::kHistBins * 4;
  p->off_hist0 = take(hist);
  p->off_hist1 = p->mode == 1 ? take(hist) : 0;
  p->off_scores0 = take((size_t)G * p->stride0 * 4);
  p->off_scores1 = p->mode == 1 ? take((size_t)G * p->stride1 * 4) : 0;
  p->off_blocks = p->mode == 1 ? take((size_t)G * p->keep * 4) : 0;
  // the candidate area only where a stage goes through the filter
  const bool filt = uses_filter(p->items0, G) || (p->mode == 1 && uses_filter(p->items1, G));
  p->has_cand = filt;
  p->off_cand = take(filt ? (size_t)G * p->chunks * csa2::kFiltChunk * 8 : 0);
  p->off_count = take(filt ? (size_t)G * p->chunks * 4 : 0);
  p->total = off;
  return CSA2_OK;
}

int32_t score_chunk(int64_t n_items, int64_t rows, int extra_per_row = 0) {
  // one full round of resident workgroups: as many chunks as fit on the
  // device at once (no tail round), in whole 16-item tiles, so that every
  // slot gets a chunk and no compute unit takes a third more work than
  // another (a wave's last group of tiles may be partial); extra_per_row
  // slots per row are left to other workgroups of the same launch
  const int64_t slots = csa2::score_resident_wgs();
  int64_t per_row_wgs = rows >= slots ? 1 : slots / rows - extra_per_row;
  if (per_row_wgs < 1) per_row_wgs = 1;
  int64_t c = (n_items + per_row_wgs - 1) / per_row_wgs;
  c = (c + 15) / 16 * 16;
  if (c < 256) c = 256;
  return (int32_t)c;
}

// ---- attention plan --------------------------------------------------------

struct AttnPlan {
  int32_t n_split, keys_per_split, heads_per_wg;
  size_t off_o, off_ml, total;
};

// Plan override for tests and benchmarks (csa2_attn_plan_override): heads per
// workgroup and key splits, 0 = chosen per call.
std::atomic<int32_t> g_attn_hpw{0}, g_attn_split{0};

int32_t check_attn(const csa2_attn_args* a, AttnPlan* p, bool check_ptrs) {
  if (!a) return fail(CSA2_EINVAL, "attn: args is NULL");
  if (a->n_rows < 0) return fail(CSA2_EINVAL, "attn: n_rows < 0");
  if (a->n_seq < 0) return fail(CSA2_EINVAL, "attn: n_seq < 0");
  if (a->n_heads != 16 && a->n_heads != 32 && a->n_heads != 64 && a->n_heads != 128)
    return fail(CSA2_EUNSUPPORTED, "attn: n_heads %d not in {16, 32, 64, 128}", a->n_heads);
  if (a->top_k < 0 || a->top_k > CSA2_MAX_TOPK)
    return fail(CSA2_EUNSUPPORTED, "attn: top_k %d outside [0, %d]", a->top_k, CSA2_MAX_TOPK);
  if (a->n_ent < 0) return fail(CSA2_EINVAL, "attn: n_ent < 0");
  const bool has_swa = a->swa_len != nullptr;
  if (has_swa && (a->swa_cap < 1 || a->swa_cap > 65536))
    return fail(CSA2_EINVAL, "attn: swa_cap %d outside [1, 65536] with swa_len set", a->swa_cap);
  if (has_swa && (a->swa_max < 0 || a->swa_max > a->swa_cap))
    return fail(CSA2_EINVAL, "attn: swa_max %d outside [0, swa_cap %d]", a->swa_max, a->swa_cap);
  if (a->n_rows > 0 && check_ptrs) {
    if (!a->q_bf16 || !a->out) return fail(CSA2_EINVAL, "attn: q_bf16 and out are required");
    if (!aligned(a->q_bf16, 16) || !aligned(a->out, 16)) return fail(CSA2_EINVAL, "attn: q/out not 16-byte aligned");
    if (a->top_k > 0 && (!a->idx || !a->codes || !a->scales))
      return fail(CSA2_EINVAL, "attn: idx, codes and scales are required when top_k > 0");
    if (a->top_k > 0 && (!aligned(a->codes, 16) || !aligned(a->scales, 16) || !aligned(a->idx, 4)))
      return fail(CSA2_EINVAL, "attn: codes/scales/idx misaligned");
    if (has_swa && (!a->swa || !aligned(a->swa, 16))) return fail(CSA2_EINVAL, "attn: swa missing or misaligned");
    if (a->lse && !aligned(a->lse, 4)) return fail(CSA2_EINVAL, "attn: lse misaligned");
  }
  const int64_t nk = (int64_t)a->top_k + (has_swa ? (a->swa_max > 0 ? a->swa_max : a->swa_cap) : 0);
  const int64_t max_split = (nk + CSA2_MIN_SPLIT_KEYS - 1) / CSA2_MIN_SPLIT_KEYS;   // keys per split at least
  // Few rows: one 16-head group per workgroup (the narrow kernel: a short
  // chain of dependent steps, two workgroups per CU), as long as every such
  // workgroup of the full key split runs at once; each of them gathers the
  // row's keys (mostly from L2).  Otherwise up to 64 heads per workgroup
  // share one gather and dequantisation.
  const int64_t wg16 = (int64_t)a->n_rows * ((a->n_heads + 15) / 16);
  const int64_t ns16 = wg16 > 0 ? std::min(max_split, (int64_t)CSA2_RESIDENT_ATTN_WGS / wg16) : 0;
  p->heads_per_wg = (ns16 >= 1 && (nk + ns16 - 1) / ns16 <= CSA2_NARROW_MAX_SPLIT_KEYS) ? 16 : 64;
  const int32_t hpw_forced = g_attn_hpw.load(std::memory_order_relaxed);
  if (hpw_forced) p->heads_per_wg = hpw_forced;
  const int64_t hg = (a->n_heads + p->heads_per_wg - 1) / p->heads_per_wg;
  const int64_t wgs = (int64_t)a->n_rows * hg;
  int64_t ns = wgs > 0 ? (256 + wgs - 1) / wgs : 1;
  if (p->heads_per_wg == 64) ns = std::min<int64_t>(ns, std::max<int64_t>(1, nk / CSA2_WIDE_MIN_SPLIT_KEYS));
  if (p->heads_per_wg == 16) {
    // as many splits as run at once, but no more workgroups than compute
    // units where splits of up to three chunks already fill them
    const int64_t fit = std::max<int64_t>(1, (int64_t)CSA2_ATTN_CUS / std::max<int64_t>(wgs, 1));
    const int64_t at_least = (nk + CSA2_NARROW_CU_SPLIT_KEYS - 1) / CSA2_NARROW_CU_SPLIT_KEYS;
    ns = std::max<int64_t>(1, std::min(ns16, std::max(fit, at_least)));
  }
  if (ns > max_split) ns = max_split;
  const int32_t split_forced = g_attn_split.load(std::memory_order_relaxed);
  if (split_forced) ns = split_forced;
  // at most 512 selected ids staged per 16-head workgroup, 1024 keys per
  // 64-head workgroup
  const int64_t min_split = p->heads_per_wg == 16 ? (a->top_k + 511) / 512 : (nk + 1023) / 1024;
  if (ns < min_split) ns = min_split;
  if (ns < 1) ns = 1;
  int64_t kps = (nk + ns - 1) / ns;
  kps = (kps + 31) / 32 * 32;
  if (kps < 32) kps = 32;
  ns = (nk + kps - 1) / kps;
  if (ns < 1) ns = 1;
  p->n_split = (int32_t)ns;
  p->keys_per_split = (int32_t)kps;
  size_t off = 0;
  if (ns > 1) {
    const size_t rh = (size_t)a->n_rows * a->n_heads;
    p->off_o = off;
    off = round_up(off + (size_t)ns * rh * CSA2_LATENT_DIM * 4, 256);
    p->off_ml = off;
    off = round_up(off + (size_t)ns * rh * 2 * 4, 256);
  } else {
    p->off_o = p->off_ml = 0;
  }
  p->total = off;
  return CSA2_OK;
}

// Validates an append and fills the kernel arguments (k->n_rows = 0 when
// there is nothing to launch).
int32_t check_append(const csa2_append_args* a, csa2::AppendArgs* out) {
  if (!a) return fail(CSA2_EINVAL, "decode_append: NULL args");
  if (!a->codes) {                // window-only rows
    if (a->n_rows < 0 || a->n_seq < 0) return fail(CSA2_EINVAL, "decode_append: negative size");
    if (a->n_rows == 0) { out->n_rows = 0; return CSA2_OK; }
    if (!a->swa || a->swa_cap < 1 || !a->pos || !a->x_bf16)
      return fail(CSA2_EINVAL, "decode_append: window-only rows need swa, swa_cap >= 1, pos and x");
    if (!aligned(a->x_bf16, 16) || !aligned(a->pos, 8) || !aligned(a->swa, 4) ||
        (a->row_seq && !aligned(a->row_seq, 4)))
      return fail(CSA2_EINVAL, "decode_append: x/pos/swa/row_seq misaligned");
    csa2::AppendArgs k{};
    k.n_rows = a->n_rows;
    k.n_seq = a->n_seq;
    k.row_seq = a->row_seq;
    k.pos = a->pos;
    k.m = 1;
    k.x = static_cast<const uint16_t*>(a->x_bf16);
    k.swa = a->swa;
    k.swa_cap = a->swa_cap;
    *out = k;
    return CSA2_OK;
  }
  if (a->m != 1 && a->m != 2 && a->m != 4) return fail(CSA2_EUNSUPPORTED, "decode_append: m=%d not in {1,2,4}", a->m);
  if (a->key_format != CSA2_KEY_E4M3 && a->key_format != CSA2_KEY_FP4)
    return fail(CSA2_EUNSUPPORTED, "decode_append: key_format %d unknown", a->key_format);
  if (a->n_rows < 0 || a->n_seq < 0 || a->n_ent < 0) return fail(CSA2_EINVAL, "decode_append: negative size");
  if (a->n_rows == 0) { out->n_rows = 0; return CSA2_OK; }
  if (!a->pos || !a->x_bf16 || !a->scales || !a->key_bf16 || !a->keys)
    return fail(CSA2_EINVAL, "decode_append: pos, x, scales, key and keys are required with codes");
  if (a->m > 1 && !a->pend_x) return fail(CSA2_EINVAL, "decode_append: m > 1 needs pend_x");
  if (a->m > 1 && a->gate_bf16 && !a->pend_gate) return fail(CSA2_EINVAL, "decode_append: a gate needs pend_gate");
  if (a->key_format == CSA2_KEY_FP4 && !a->key_scales) return fail(CSA2_EINVAL, "decode_append: FP4 keys need key_scales");
  if (a->swa && a->swa_cap < 1) return fail(CSA2_EINVAL, "decode_append: swa_cap %d < 1", a->swa_cap);
  if (!aligned(a->x_bf16, 16) || (a->gate_bf16 && !aligned(a->gate_bf16, 16)) ||
      (a->pend_x && !aligned(a->pend_x, 16)) || (a->pend_gate && !aligned(a->pend_gate, 16)) ||
      !aligned(a->key_bf16, 8) || !aligned(a->pos, 8) || (a->row_seq && !aligned(a->row_seq, 4)))
    return fail(CSA2_EINVAL, "decode_append: x/gate/pending/key/pos misaligned");
  if (!aligned(a->codes, 8) || !aligned(a->keys, 8) || (a->block_keys && !aligned(a->block_keys, 4)) ||
      (a->swa && !aligned(a->swa, 4)))
    return fail(CSA2_EINVAL, "decode_append: codes/keys/block_keys/swa misaligned");
  csa2::AppendArgs k;
  k.n_rows = a->n_rows;
  k.n_seq = a->n_seq;
  k.row_seq = a->row_seq;
  k.pos = a->pos;
  k.m = a->m;
  k.x = static_cast<const uint16_t*>(a->x_bf16);
  k.gate = a->m > 1 ? static_cast<const uint16_t*>(a->gate_bf16) : nullptr;
  k.pend_x = static_cast<uint16_t*>(a->pend_x);
  k.pend_gate = static_cast<uint16_t*>(a->pend_gate);
  k.n_ent = a->n_ent;
  k.codes = a->codes;
  k.scales = a->scales;
  k.key = static_cast<const uint16_t*>(a->key_bf16);
  k.key_fp4 = a->key_format == CSA2_KEY_FP4;
  k.keys = a->keys;
  k.key_scales = a->key_scales;
  k.block_keys = a->block_keys;
  k.swa = a->swa;
  k.swa_cap = a->swa ? a->swa_cap : 1;
  *out = k;
  return CSA2_OK;
}

// ---- static scratch of csa2_indexer_topk_static ---------------------------

// One array per GPU (each device holds its own copy at its own address).  In
// host code `scratch` names a host-side stand-in: only the device address
// from hipGetSymbolAddress, kept per device, is ever passed to a kernel.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices];

int32_t static_scratch(char** out);
int32_t run_indexer(const csa2_indexer_args* a, const IndexerPlan& p, char* w, hipStream_t s,
                    const csa2::AppendArgs* fused = nullptr);

}  // namespace

static __device__ __align__(256) unsigned char scratch[CSA2_STATIC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current.
int32_t static_scratch(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "indexer_topk_static: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CSA2_EUNSUPPORTED, "indexer_topk_static: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e, "indexer_topk_static: hipGetSymbolAddress(scratch)");
    if (!aligned(ptr, 256)) return fail(CSA2_EHIP, "indexer_topk_static: scratch not 256-byte aligned");
    g_scratch_dev[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_dev[dev];
  return CSA2_OK;
}

}  // namespace

extern "C" {

int32_t csa2_abi_version(void) { return CSA2_ABI_VERSION; }

const char* csa2_status_string(int32_t st) {
  switch (st) {
    case CSA2_OK: return "ok";
    case CSA2_EINVAL: return "invalid argument";
    case CSA2_EUNSUPPORTED: return "unsupported configuration";
    case CSA2_EWORKSPACE: return "workspace too small";
    case CSA2_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* csa2_last_error(void) { return g_err.c_str(); }

int32_t csa2_kv_compress_quantize(const void* x_bf16, const void* gate_bf16, int64_t n_seq,
                                  int64_t n_tok, int32_t m, int64_t x_seq_stride,
                                  uint8_t* codes, uint8_t* scales, int64_t out_seq_stride,
                                  void* stream) {
  g_err.clear();
  if (m != 1 && m != 2 && m != 4) return fail(CSA2_EUNSUPPORTED, "kv_compress_quantize: m=%d not in {1,2,4}", m);
  if (n_seq < 0 || n_tok < 0) return fail(CSA2_EINVAL, "kv_compress_quantize: negative size");
  const int64_t n_ent = n_tok / m;
  if (x_seq_stride == 0) x_seq_stride = n_tok;
  if (out_seq_stride == 0) out_seq_stride = n_ent;
  if (x_seq_stride < n_tok) return fail(CSA2_EINVAL, "kv_compress_quantize: x_seq_stride < n_tok");
  if (out_seq_stride < n_ent) return fail(CSA2_EINVAL, "kv_compress_quantize: out_seq_stride < n_tok/m");
  if (n_seq == 0 || n_ent == 0) return CSA2_OK;
  if (!x_bf16 || !codes || !scales) return fail(CSA2_EINVAL, "kv_compress_quantize: NULL pointer");
  if (!aligned(x_bf16, 16) || (gate_bf16 && !aligned(gate_bf16, 16)))
    return fail(CSA2_EINVAL, "kv_compress_quantize: x/gate not 16-byte aligned");
  if (!aligned(codes, 8)) return fail(CSA2_EINVAL, "kv_compress_quantize: codes not 8-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(CSA2_SITE_KV_QUANT, s, [&] {
    return csa2::launch_kv_compress_quantize(x_bf16, gate_bf16, n_seq, n_ent, m, x_seq_stride,
                                             codes, scales, out_seq_stride, s);
  });
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "kv_compress_quantize launch");
}

int32_t csa2_decode_append(const csa2_append_args* a, void* stream) {
  g_err.clear();
  csa2::AppendArgs k{};
  const int32_t st = check_append(a, &k);
  if (st != CSA2_OK || k.n_rows == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(CSA2_SITE_APPEND, s, [&] { return csa2::launch_decode_append(k, s); });
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "decode_append launch");
}

int32_t csa2_index_block_summary(const uint8_t* keys, int64_t n_seq, int64_t n_ent,
                                 int64_t blk_begin, int64_t blk_end, uint8_t* summ,
                                 void* stream) {
  g_err.clear();
  if (n_seq < 0 || n_ent < 0) return fail(CSA2_EINVAL, "index_block_summary: negative size");
  const int64_t nb = (n_ent + CSA2_BLOCK_POS - 1) / CSA2_BLOCK_POS;
  if (blk_begin < 0 || blk_end < blk_begin || blk_end > nb)
    return fail(CSA2_EINVAL, "index_block_summary: block range [%lld, %lld) outside [0, %lld)",
                (long long)blk_begin, (long long)blk_end, (long long)nb);
  if (n_seq == 0 || blk_end == blk_begin) return CSA2_OK;
  if (!keys || !summ) return fail(CSA2_EINVAL, "index_block_summary: NULL pointer");
  if (!aligned(keys, 4) || !aligned(summ, 4)) return fail(CSA2_EINVAL, "index_block_summary: misaligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(CSA2_SITE_BLOCK_SUMMARY, s, [&] {
    return csa2::launch_block_summary(keys, n_seq, n_ent, blk_begin, blk_end, summ, s);
  });
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "index_block_summary launch");
}

int32_t csa2_index_key_quantize(const void* k_bf16, int64_t n_seq, int64_t n_ent, int64_t k_seq_stride,
                                uint8_t* codes, uint8_t* scales, int64_t out_seq_stride, void* stream) {
  g_err.clear();
  if (n_seq < 0 || n_ent < 0) return fail(CSA2_EINVAL, "index_key_quantize: negative size");
  if (k_seq_stride == 0) k_seq_stride = n_ent;
  if (out_seq_stride == 0) out_seq_stride = n_ent;
  if (k_seq_stride < n_ent || out_seq_stride < n_ent)
    return fail(CSA2_EINVAL, "index_key_quantize: a sequence stride is below n_ent");
  if (n_seq == 0 || n_ent == 0) return CSA2_OK;
  if (!k_bf16 || !codes || !scales) return fail(CSA2_EINVAL, "index_key_quantize: NULL pointer");
  if (!aligned(k_bf16, 16) || !aligned(codes, 16))
    return fail(CSA2_EINVAL, "index_key_quantize: keys/codes not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(CSA2_SITE_KV_QUANT, s, [&] {
    return csa2::launch_index_key_quantize(k_bf16, n_seq, n_ent, k_seq_stride, codes, scales, out_seq_stride, s);
  });
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "index_key_quantize launch");
}

int32_t csa2_index_block_summary_fp4(const uint8_t* codes, const uint8_t* scales, int64_t n_seq,
                                     int64_t n_ent, int64_t blk_begin, int64_t blk_end, uint8_t* summ,
                                     void* stream) {
  g_err.clear();
  if (n_seq < 0 || n_ent < 0) return fail(CSA2_EINVAL, "index_block_summary_fp4: negative size");
  const int64_t nb = (n_ent + CSA2_BLOCK_POS - 1) / CSA2_BLOCK_POS;
  if (blk_begin < 0 || blk_end < blk_begin || blk_end > nb)
    return fail(CSA2_EINVAL, "index_block_summary_fp4: block range [%lld, %lld) outside [0, %lld)",
                (long long)blk_begin, (long long)blk_end, (long long)nb);
  if (n_seq == 0 || blk_end == blk_begin) return CSA2_OK;
  if (!codes || !scales || !summ) return fail(CSA2_EINVAL, "index_block_summary_fp4: NULL pointer");
  if (!aligned(codes, 4) || !aligned(summ, 4)) return fail(CSA2_EINVAL, "index_block_summary_fp4: misaligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(CSA2_SITE_BLOCK_SUMMARY, s, [&] {
    return csa2::launch_block_summary_fp4(codes, scales, n_seq, n_ent, blk_begin, blk_end, summ, s);
  });
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "index_block_summary_fp4 launch");
}

size_t csa2_indexer_topk_workspace(const csa2_indexer_args* a) {
  IndexerPlan p;
  if (check_indexer(a, &p, false) != CSA2_OK) return 0;
  return p.total;
}

int32_t csa2_indexer_topk(const csa2_indexer_args* a, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  IndexerPlan p;
  int32_t st = check_indexer(a, &p, true);
  if (st != CSA2_OK) return st;
  if (a->n_rows == 0) return CSA2_OK;
  if (ws_bytes < p.total || (p.total && !ws))
    return fail(CSA2_EWORKSPACE, "indexer: workspace %zu bytes < %zu needed", ws_bytes, p.total);
  if (!aligned(ws, 256)) return fail(CSA2_EINVAL, "indexer: workspace not 256-byte aligned");
  return run_indexer(a, p, static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

int32_t csa2_indexer_topk_static(const csa2_indexer_args* a, void* stream) {
  g_err.clear();
  IndexerPlan p;
  int32_t st = check_indexer(a, &p, true);
  if (st != CSA2_OK) return st;
  if (a->n_rows == 0) return CSA2_OK;
  if (p.total > (size_t)CSA2_STATIC_SCRATCH_BYTES)
    return fail(CSA2_EWORKSPACE, "indexer_topk_static: %zu scratch bytes needed, the static array holds %zu",
                p.total, (size_t)CSA2_STATIC_SCRATCH_BYTES);
  char* w = nullptr;
  if ((st = static_scratch(&w)) != CSA2_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the histograms (the plan's first bytes, up to the first score row) must
  // start at zero; the array keeps whatever the last call on this GPU left
  const size_t n_words = p.off_scores0 / 4;
  hipError_t e = csa2::launch_zero_words(reinterpret_cast<uint32_t*>(w), n_words, s);
  if (e != hipSuccess) return hip_fail(e, "indexer_topk_static: clearing the histograms");
  return run_indexer(a, p, w, s);
}

int32_t csa2_append_indexer_topk(const csa2_append_args* ap, const csa2_indexer_args* a, void* ws,
                                 size_t ws_bytes, void* stream) {
  g_err.clear();
  csa2::AppendArgs k{};
  int32_t st = check_append(ap, &k);
  if (st != CSA2_OK) return st;
  IndexerPlan p;
  if ((st = check_indexer(a, &p, true)) != CSA2_OK) return st;
  if (a->n_rows > 0 && (ws_bytes < p.total || (p.total && !ws)))
    return fail(CSA2_EWORKSPACE, "append_indexer: workspace %zu bytes < %zu needed", ws_bytes, p.total);
  if (a->n_rows > 0 && !aligned(ws, 256)) return fail(CSA2_EINVAL, "append_indexer: workspace not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one launch for the append and the coarse scan when they describe the
  // same rows of the same caches, row r being sequence r (no row_seq): each
  // row's scan then reads only the block summaries its own append refreshes
  const bool fuse = p.mode == 1 && k.n_rows > 0 && ap->codes && ap->block_keys == a->block_keys &&
                    ap->keys == a->keys && ap->key_format == a->key_format &&
                    (a->key_format == CSA2_KEY_E4M3 || ap->key_scales == a->key_scales) &&
                    ap->n_rows == a->n_rows && !ap->row_seq && !a->row_seq && ap->n_seq == a->n_seq &&
                    ap->n_ent == a->n_ent && (ap->m == 1 || ap->m == 2);
  if (!fuse) {
    if (k.n_rows > 0) {
      hipError_t e = timed(CSA2_SITE_APPEND, s, [&] { return csa2::launch_decode_append(k, s); });
      if (e != hipSuccess) return hip_fail(e, "decode_append launch");
    }
    if (a->n_rows == 0) return CSA2_OK;
    return run_indexer(a, p, static_cast<char*>(ws), s);
  }
  return run_indexer(a, p, static_cast<char*>(ws), s, &k);
}

}  // extern "C"

namespace {

int32_t run_indexer(const csa2_indexer_args* a, const IndexerPlan& p, char* w, hipStream_t s,
                    const csa2::AppendArgs* fused) {
  int32_t st;

  csa2::ItemMap im0{};
  im0.n_seq = a->n_seq;
  im0.row_seq = a->row_seq;
  im0.n_valid = a->n_valid;
  im0.any = a->q;
  im0.n_ent = a->n_ent;
  im0.n_items = p.items0;

  csa2::ScoreArgs sa{};
  sa.n_rows = a->n_rows;
  sa.n_seq = a->n_seq;
  sa.q = a->q;
  sa.w = a->head_w;
  sa.key_fp4 = a->key_format == CSA2_KEY_FP4;
  sa.key_scales = a->key_scales;

  csa2::SelectArgs se{};
  se.n_rows = a->n_rows;
  // no candidate area: the row select keeps its candidates in LDS, and a
  // threshold bin too large for LDS is resolved from the stored scores
  se.cand = p.has_cand ? reinterpret_cast<uint64_t*>(w + p.off_cand) : nullptr;
  se.cand_count = p.has_cand ? reinterpret_cast<uint32_t*>(w + p.off_count) : nullptr;
  se.n_chunks = p.chunks;

  // histograms start at zero (the caller zeroes the workspace once) and the
  // select kernel leaves them zeroed again
  uint32_t* hist0 = reinterpret_cast<uint32_t*>(w + p.off_hist0);
  float* scores0 = reinterpret_cast<float*>(w + p.off_scores0);

  // one top-k stage: score -> filter -> select
  auto stage = [&](int site, const csa2::ItemMap& im, const uint8_t* keys, int64_t seq_rows, int32_t stride,
                   float* scores, uint32_t* hist, int32_t k, int32_t* out_idx, float* out_score) -> int32_t {
    hipError_t e2;
    sa.im = im;
    sa.keys = keys;
    sa.seq_rows = seq_rows;
    sa.row_stride = stride;
    sa.scores = scores;
    sa.hist = hist;
    // the coarse stage of a fused decode step also runs the append, in one
    // extra workgroup per row (its slots are kept free)
    sa.fuse_append = (fused && im.mode == csa2::kItemsBlocks) ? 1 : 0;
    if (sa.fuse_append) sa.app = *fused;
    sa.chunk = score_chunk(im.n_items, sa.n_rows, sa.fuse_append);
    if ((e2 = timed(site, s, [&] { return csa2::launch_index_score(sa, s); })) != hipSuccess)
      return hip_fail(e2, "indexer score");
    se.im = im;
    se.k = k;
    se.row_stride = stride;
    se.scores = scores;
    se.hist = hist;
    se.out_idx = out_idx;
    se.out_score = out_score;
    // the plan's decision: a last pass of fewer rows than the plan sized the
    // workspace for still selects per row when no candidate area exists
    if (!(p.has_cand && uses_filter(im.n_items, se.n_rows))) {
      if ((e2 = timed(CSA2_SITE_SELECT, s, [&] { return csa2::launch_topk_row(se, s); })) != hipSuccess)
        return hip_fail(e2, "indexer top-k");
      return CSA2_OK;
    }
    if ((e2 = timed(CSA2_SITE_FILTER, s, [&] { return csa2::launch_topk_filter(se, s); })) != hipSuccess)
      return hip_fail(e2, "indexer filter");
    if ((e2 = timed(CSA2_SITE_SELECT, s, [&] { return csa2::launch_topk_select(se, s); })) != hipSuccess)
      return hip_fail(e2, "indexer select");
    return CSA2_OK;
  };

  if (p.mode != 1) {
    // one stage: flat, candidate list or candidate blocks, rows in passes of
    // p.group_rows through one score block (stream-ordered: a pass's select
    // has read the block before the next pass scores into it)
    const int site = p.mode == 0 ? CSA2_SITE_SCORE_FLAT : p.mode == 2 ? CSA2_SITE_SCORE_CAND : CSA2_SITE_SCORE_POOL;
    im0.mode = p.mode == 0 ? csa2::kItemsFlat : p.mode == 2 ? csa2::kItemsCand : csa2::kItemsPool;
    const int32_t* list = p.mode == 2 ? a->cand : p.mode == 3 ? a->cand_blocks : nullptr;
    im0.list_len = p.mode == 2 ? a->n_cand : p.mode == 3 ? a->n_cand_blocks : 0;
    for (int64_t g0 = 0; g0 < p.R; g0 += p.group_rows) {
      const int32_t rows = (int32_t)std::min<int64_t>(p.group_rows, p.R - g0);
      csa2::ItemMap img = im0;
      img.row_seq = a->row_seq ? a->row_seq + g0 : nullptr;
      img.row_base = g0;
      img.n_valid = a->n_valid ? a->n_valid + g0 : nullptr;
      img.list = list ? list + g0 * im0.list_len : nullptr;
      sa.n_rows = se.n_rows = rows;
      sa.q = a->q + g0 * CSA2_IDX_HEADS * CSA2_IDX_DIM;
      sa.w = a->head_w ? a->head_w + g0 * CSA2_IDX_HEADS : nullptr;
      if ((st = stage(site, img, a->keys, a->n_ent, p.stride0, scores0, hist0, a->top_k, a->out_idx + g0 * a->top_k,
                      a->out_score ? a->out_score + g0 * a->top_k : nullptr)) != CSA2_OK)
        return st;
    }
    return CSA2_OK;
  }

  // hierarchical: coarse blocks -> kept blocks -> pool positions -> top-k
  uint32_t* hist1 = reinterpret_cast<uint32_t*>(w + p.off_hist1);
  float* scores1 = reinterpret_cast<float*>(w + p.off_scores1);
  int32_t* blocks = a->out_blocks ? a->out_blocks : reinterpret_cast<int32_t*>(w + p.off_blocks);
  im0.mode = csa2::kItemsBlocks;
  if ((st = stage(CSA2_SITE_SCORE_COARSE, im0, a->block_keys, p.NB, p.stride0, scores0, hist0, p.keep,
                  blocks, nullptr)) != CSA2_OK)
    return st;
  csa2::ItemMap im1 = im0;
  im1.mode = csa2::kItemsPool;
  im1.n_items = p.items1;
  im1.list = blocks;
  im1.list_len = p.keep;
  return stage(CSA2_SITE_SCORE_POOL, im1, a->keys, a->n_ent, p.stride1, scores1, hist1, a->top_k,
               a->out_idx, a->out_score);
}

}  // namespace

extern "C" {

int32_t csa2_attn_plan_override(int32_t heads_per_wg, int32_t n_split) {
  g_err.clear();
  if (heads_per_wg != 0 && heads_per_wg != 16 && heads_per_wg != 64)
    return fail(CSA2_EINVAL, "attn plan: heads_per_wg %d not 0, 16 or 64", heads_per_wg);
  if (n_split < 0 || n_split > 64) return fail(CSA2_EINVAL, "attn plan: n_split %d outside [0, 64]", n_split);
  g_attn_hpw.store(heads_per_wg, std::memory_order_relaxed);
  g_attn_split.store(n_split, std::memory_order_relaxed);
  return CSA2_OK;
}

size_t csa2_sparse_attn_workspace(const csa2_attn_args* a) {
  AttnPlan p;
  if (check_attn(a, &p, false) != CSA2_OK) return 0;
  return p.total;
}

int32_t csa2_sparse_attn_decode(const csa2_attn_args* a, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  AttnPlan p;
  int32_t st = check_attn(a, &p, true);
  if (st != CSA2_OK) return st;
  if (a->n_rows == 0) return CSA2_OK;
  if (ws_bytes < p.total || (p.total && !ws))
    return fail(CSA2_EWORKSPACE, "attn: workspace %zu bytes < %zu needed", ws_bytes, p.total);
  if (p.total && !aligned(ws, 256)) return fail(CSA2_EINVAL, "attn: workspace not 256-byte aligned");
  csa2::AttnArgs k{};
  k.n_rows = a->n_rows;
  k.n_heads = a->n_heads;
  k.n_seq = a->n_seq;
  k.row_seq = a->row_seq;
  k.q = static_cast<const uint16_t*>(a->q_bf16);
  k.codes = a->codes;
  k.scales = a->scales;
  k.n_ent = a->n_ent;
  k.idx = a->idx;
  k.top_k = a->top_k;
  k.swa = a->swa_len ? a->swa : nullptr;
  k.swa_cap = a->swa_len ? a->swa_cap : 0;
  k.swa_max = a->swa_len ? (a->swa_max > 0 ? a->swa_max : a->swa_cap) : 0;
  k.swa_start = a->swa_start;
  k.swa_len = a->swa_len;
  const float sm = a->sm_scale > 0.0f ? a->sm_scale : 0.044194173824159216f;   // 1/sqrt(512)
  k.sm_scale_log2 = sm * 1.4426950408889634f;
  k.out = a->out;
  k.lse = a->lse;
  k.n_split = p.n_split;
  k.heads_per_wg = p.heads_per_wg;
  k.keys_per_split = p.keys_per_split;
  k.part_o = p.n_split > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_o) : nullptr;
  k.part_ml = p.n_split > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_ml) : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(CSA2_SITE_ATTN, s, [&] { return csa2::launch_sparse_attn(k, s); });
  if (e != hipSuccess) return hip_fail(e, "sparse_attn launch");
  e = timed(CSA2_SITE_ATTN_COMBINE, s, [&] { return csa2::launch_attn_combine(k, s); });
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "attn combine launch");
}

int32_t csa2_mfma_dot_probe(const uint8_t* q, const uint8_t* k, int32_t n_q, int32_t n_k, float* out_f16,
                            float* out_f8, void* stream) {
  g_err.clear();
  if (n_q <= 0 || n_k <= 0 || n_q % 16 || n_k % 16 || n_q > (1 << 20) || n_k > (1 << 20))
    return fail(CSA2_EINVAL, "mfma probe: n_q %d, n_k %d not positive multiples of 16 up to 2^20", n_q, n_k);
  if (!q || !k || !out_f16 || !out_f8) return fail(CSA2_EINVAL, "mfma probe: null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(out_f16, 4) || !aligned(out_f8, 4))
    return fail(CSA2_EINVAL, "mfma probe: misaligned pointer");
  const hipError_t e = csa2::launch_mfma_dot_probe(q, k, n_q, n_k, out_f16, out_f8, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mfma probe");
  return CSA2_OK;
}

int32_t csa2_probe_scan_read(const uint8_t* keys, int32_t n_rows, int32_t n_keys, int32_t chunk, int32_t full_lines,
                             int32_t nontemporal, uint32_t* out, void* stream) {
  g_err.clear();
  if (n_rows < 1 || n_keys < 1 || chunk < 16 || n_keys > (1 << 24))
    return fail(CSA2_EINVAL, "scan probe: n_rows %d, n_keys %d, chunk %d out of range", n_rows, n_keys, chunk);
  const int64_t wgs = (int64_t)n_rows * ((n_keys + chunk - 1) / chunk);
  if (wgs > (1 << 20)) return fail(CSA2_EINVAL, "scan probe: %lld workgroups exceed 2^20", (long long)wgs);
  if (!keys || !out || !aligned(keys, 16) || !aligned(out, 4))
    return fail(CSA2_EINVAL, "scan probe: null or misaligned pointer");
  const hipError_t e = csa2::launch_scan_read_probe(keys, n_rows, n_keys, chunk, full_lines != 0, nontemporal != 0,
                                                    out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "scan probe");
}

int32_t csa2_probe_mfma_valu(int32_t n_valu, int32_t threads, int32_t iters, int32_t n_wg, float* out,
                             void* stream) {
  g_err.clear();
  if (n_valu != 0 && n_valu != 4 && n_valu != 8 && n_valu != 12 && n_valu != 16)
    return fail(CSA2_EINVAL, "mfma/valu probe: n_valu %d not one of 0, 4, 8, 12, 16", n_valu);
  if (threads != 256 && threads != 512) return fail(CSA2_EINVAL, "mfma/valu probe: threads %d not 256 or 512", threads);
  if (iters < 1 || iters > (1 << 20) || n_wg < 1 || n_wg > 65536)
    return fail(CSA2_EINVAL, "mfma/valu probe: iters %d or n_wg %d out of range", iters, n_wg);
  if (!out || !aligned(out, 4)) return fail(CSA2_EINVAL, "mfma/valu probe: null or misaligned out");
  const hipError_t e = csa2::launch_mfma_valu_probe(n_valu, threads, iters, n_wg, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "mfma/valu probe");
}

int32_t csa2_probe_gather(const uint8_t* codes, const uint8_t* scales, int64_t n_ent, const int32_t* ids,
                          int32_t n_rows, int32_t n_wg, int32_t whole_lines, uint32_t* out, void* stream) {
  g_err.clear();
  if (n_ent < 1 || n_ent > (1LL << 31) || n_rows < 1 || n_wg < 1 || n_wg > 65536)
    return fail(CSA2_EINVAL, "gather probe: n_ent %lld, n_rows %d or n_wg %d out of range", (long long)n_ent, n_rows,
                n_wg);
  if (!codes || !scales || !ids || !out || !aligned(codes, 16) || !aligned(scales, 16) || !aligned(ids, 4) ||
      !aligned(out, 4))
    return fail(CSA2_EINVAL, "gather probe: null or misaligned pointer");
  const hipError_t e = csa2::launch_gather_probe(codes, scales, n_ent, ids, n_rows, n_wg, whole_lines != 0, out,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "gather probe");
}

int32_t csa2_kernel_timer_start(int32_t site, int32_t max_launches) {
  g_err.clear();
  if (site < CSA2_SITE_KV_QUANT || site > CSA2_SITE_APPEND)
    return fail(CSA2_EINVAL, "kernel_timer_start: unknown site %d", site);
  if (max_launches < 1 || max_launches > 1000000)
    return fail(CSA2_EINVAL, "kernel_timer_start: max_launches %d outside [1, 1e6]", max_launches);
  const size_t need = 2 * (size_t)max_launches;
  while (g_timer.ev.size() < need) {
    // timing only: no system-scope fence around the kernel being measured
    // (callers synchronise through their own stream or device calls)
    hipEvent_t ev;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableSystemFence);
    if (e != hipSuccess) return hip_fail(e, "kernel_timer_start: hipEventCreate");
    g_timer.ev.push_back(ev);
  }
  g_timer.site = site;
  g_timer.used = 0;
  return CSA2_OK;
}

int32_t csa2_kernel_timer_stop(int32_t* n_launches, float* total_ms) {
  g_err.clear();
  if (!n_launches || !total_ms) return fail(CSA2_EINVAL, "kernel_timer_stop: NULL output");
  float tot = 0.0f;
  for (int32_t i = 0; i < g_timer.used; ++i) {
    hipError_t e = hipEventSynchronize(g_timer.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "kernel_timer_stop: hipEventSynchronize");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, g_timer.ev[2 * i], g_timer.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "kernel_timer_stop: hipEventElapsedTime");
    tot += ms;
  }
  *n_launches = g_timer.used;
  *total_ms = tot;
  g_timer.site = 0;
  g_timer.used = 0;
  return CSA2_OK;
}

}  // extern "C"
