// Exact top-k of the indexer scores [0539edu §3: top_k 512; hierarchical
// block: keep 2048 blocks; ties go to the lower position].
//
// Items are ranked by a composite key (order key of the score, ~position),
// so the k largest keys are the k highest scores with ties to the lower
// position.  The score kernel's per-row histogram of the top 12 bits gives
// the bin b* holding the k-th score; items in b* or above are candidates.
//   long rows:  a filter kernel (many workgroups per row) compacts each
//               chunk's candidates in item order; one 1024-thread workgroup
//               per row then settles the k-th composite key exactly with an
//               MSB-first radix select over the candidates of bin b* and
//               writes the kept ones in candidate order (ascending position).
//   short rows: one 1024-thread workgroup per row does both, with the
//               candidates in LDS (the workspace when they do not fit).
// The select leaves the row histogram zeroed for the next call.
#include "csa2_dev.h"
#include "csa2_launch.h"
#include "items.h"

namespace csa2 {

// ---------------------------------------------------------------------------
// filter (many workgroups per row) + select (one workgroup per row)
// ---------------------------------------------------------------------------

constexpr int kFiltThreads = 256;
constexpr int kFiltRound = kFiltThreads * 4;           // items per compaction round

// Composite order key: score order first, then lower position first.
__device__ __forceinline__ uint64_t comp_key(uint32_t okey, int64_t pos) {
  return ((uint64_t)okey << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
}
__device__ __forceinline__ int32_t comp_pos(uint64_t K) { return (int32_t)(0xFFFFFFFFu - (uint32_t)K); }
__device__ __forceinline__ float comp_score(uint64_t K) { return order_key_inv((uint32_t)(K >> 32)); }

// Exclusive prefix sum over a workgroup of NT threads (wave64); `total`
// receives the sum.  Uses wsum[NT/64] of shared scratch; ends synchronised.
// Branch-free: an in-bounds float4 load (the row's stride is a multiple of 4
// and i0 is too) with lanes past the row's items set to NaN.  A branch around
// a tail path would make the compiler wait for each load before the next.
__device__ __forceinline__ float4 load_items4(const float* srow, int64_t i0, int64_t n_row, int64_t stride) {
  const float4 t = *reinterpret_cast<const float4*>(srow + (i0 < stride ? i0 : 0));
  const float nan = __uint_as_float(0x7FC00000u);
  return make_float4(i0 + 0 < n_row ? t.x : nan, i0 + 1 < n_row ? t.y : nan,
                     i0 + 2 < n_row ? t.z : nan, i0 + 3 < n_row ? t.w : nan);
}

template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  lds_barrier();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = wsum[w];
    off += (w < wave) ? t : 0;
    tot += t;
  }
  total = tot;
  lds_barrier();
  return off + x - v;
}

constexpr int kStageCap = 4096;     // boundary-bin candidates staged in LDS

constexpr int kSelThreads = 1024;  // select workgroup
constexpr int kRegKeys = 8;        // candidates per thread held in registers by the select
constexpr int kMaxChunks = kMaxItems / kFiltChunk;

struct TopkShared {
  int wsum[kSelThreads / 64];
  int pair[3], n_stage;
  int digit, above, dcount;
  uint32_t hist[256];
  int coff[kMaxChunks + 1];          // first flattened candidate of each chunk
  union {
    uint64_t stage[kStageCap];                                 // radix select
    struct { int32_t pos[kMaxTopK]; float score[kMaxTopK]; } sel;  // candidate-mode sort
  } u;
};

// One radix step's decision, taken by wave 0 from sh.hist[0..256): the digit
// whose keys hold the need-th largest key (digits descending), the count of
// keys above it and its own count.
template <class SH>
__device__ __forceinline__ void pick_digit(SH& sh, int need) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    uint32_t h[4], l = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { h[i] = sh.hist[4 * tid + i]; l += h[i]; }
    uint32_t x = l;                                    // sum over lanes >= tid
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_down(x, d);
      if (tid + d < 64) x += y;
    }
    uint32_t cum = x - l;
    for (int i = 3; i >= 0; --i) {
      if (cum < (uint32_t)need && cum + h[i] >= (uint32_t)need) {
        sh.digit = 4 * tid + i; sh.above = (int)cum; sh.dcount = (int)h[i];
      }
      cum += h[i];
    }
  }
}

// Radix digits below the 12 histogram bits of a composite key: six 8-bit
// digits, then one 4-bit digit.
__device__ __forceinline__ int digit_shift(int step) { return step < 6 ? 44 - 8 * step : 0; }
__device__ __forceinline__ int digit_width(int step) { return step < 6 ? 8 : 4; }

// Threshold bin of a row from its score histogram: b*, the bin holding the
// kk-th largest score (kk = min(k, visible items)), the count of items in the
// bins above it and the count in b* or above; b* = -1 when every visible item
// is kept.
struct RowThreshold {
  int bstar, c_above, n_cand;
  uint32_t kk;
};

template <int NT>
__device__ __forceinline__ void hist_load(const uint32_t* gh, uint32_t (&hv)[kHistBins / NT]) {
#pragma unroll
  for (int i = 0; i < kHistBins / NT; ++i) hv[i] = gh[(kHistBins / NT) * threadIdx.x + i];
}

template <int NT>
__device__ __forceinline__ RowThreshold hist_threshold(const uint32_t (&hv)[kHistBins / NT], int k, int* wsum,
                                                       int* sh3) {
  const int tid = threadIdx.x;
  constexpr int kBpt = kHistBins / NT;                         // bins per thread
  uint32_t loc = 0;
#pragma unroll
  for (int i = 0; i < kBpt; ++i) loc += hv[i];
  int tot_i;
  const int below = block_excl_scan<NT>((int)loc, wsum, tot_i);   // bins of threads < tid
  const uint32_t total = (uint32_t)tot_i;
  if (tid == 0) { sh3[0] = -1; sh3[1] = 0; sh3[2] = (int)total; }
  lds_barrier();
  const uint32_t kk = min((uint32_t)k, total);
  if (kk < total) {
    const uint32_t above = total - (uint32_t)below - loc;      // bins of threads > tid
    if (above < kk && above + loc >= kk) {
      uint32_t cum = above;
      for (int b = kBpt - 1; b >= 0; --b) {
        if (cum + hv[b] >= kk) {
          sh3[0] = kBpt * tid + b; sh3[1] = (int)cum; sh3[2] = (int)(cum + hv[b]);
          break;
        }
        cum += hv[b];
      }
    }
  }
  lds_barrier();
  return RowThreshold{sh3[0], sh3[1], sh3[2], kk};
}

template <int NT>
__device__ __forceinline__ RowThreshold row_threshold(const uint32_t* gh, int k, int* wsum, int* sh3) {
  uint32_t hv[kHistBins / NT];
  hist_load<NT>(gh, hv);
  return hist_threshold<NT>(hv, k, wsum, sh3);
}

// Filter.  Workgroup (chunk c, row r) finds b* and writes every item of its
// chunk in b* or above -- a superset of the chunk's share of the top-k -- as
// composite keys, compacted in item order, plus their count.
__global__ __launch_bounds__(kFiltThreads) void topk_filter_kernel(SelectArgs a) {
  __shared__ int wsum[kFiltThreads / 64];
  __shared__ int pair[3];
  const int r = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int64_t nv = row_valid(a.im, r);
  const int64_t n_row = row_items(a.im, nv);
  const int64_t c0 = (int64_t)c * kFiltChunk;
  if (c0 >= n_row) return;                                     // uniform
  const int64_t c1 = min(c0 + (int64_t)kFiltChunk, n_row);

  // this thread's items, 4 consecutive per round, loaded before the scan
  const float* srow = a.scores + (int64_t)r * a.row_stride;
  constexpr int kRounds = kFiltChunk / kFiltRound;
  float v[kRounds][4];
#pragma unroll
  for (int rd = 0; rd < kRounds; ++rd) {
    const float4 q = load_items4(srow, c0 + (int64_t)rd * kFiltRound + 4 * tid, c1, a.row_stride);
    v[rd][0] = q.x; v[rd][1] = q.y; v[rd][2] = q.z; v[rd][3] = q.w;
  }
  const RowThreshold th = row_threshold<kFiltThreads>(a.hist + (int64_t)r * kHistBins, a.k, wsum, pair);

  // compaction in item order
  uint64_t* crow = a.cand + ((int64_t)r * a.n_chunks + c) * kFiltChunk;
  int written = 0;
#pragma unroll
  for (int rd = 0; rd < kRounds; ++rd) {
    const int64_t i0 = c0 + (int64_t)rd * kFiltRound + 4 * tid;
    uint32_t ok[4];
    int flag = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ok[j] = order_key(v[rd][j]);
      const bool keep = (v[rd][j] == v[rd][j]) && (int)(ok[j] >> (32 - kHistBits)) >= th.bstar;
      flag |= (int)keep << j;
    }
    int tot;
    int slot = block_excl_scan<kFiltThreads>(__popc(flag), wsum, tot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (flag & (1 << j)) crow[written + slot++] = comp_key(ok[j], item_pos(a.im, r, i0 + j, nv));
    }
    written += tot;
  }
  if (tid == 0) a.cand_count[(int64_t)r * a.n_chunks + c] = (uint32_t)written;
}

// Select.  One workgroup per row settles the k-th composite key T exactly:
// its top 12 bits are b*, the rest is found digit by digit (MSB first) among
// the candidates of bin b*.  The kept candidates (keys >= T) are written in
// candidate order, which is ascending position (candidate mode sorts).  The
// row's histogram is then cleared for the next call.
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelectArgs a) {
  __shared__ TopkShared sh;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t nv = row_valid(a.im, r);
  const int64_t n_row = row_items(a.im, nv);
  int32_t* oi = a.out_idx + (int64_t)r * a.k;
  float* os = a.out_score ? a.out_score + (int64_t)r * a.k : nullptr;
  if (n_row == 0) {                                            // uniform: nothing visible
    for (int j = tid; j < a.k; j += kSelThreads) {
      oi[j] = -1;
      if (os) os[j] = 0.0f;
    }
    return;
  }
  const int nch = (int)((n_row + kFiltChunk - 1) / kFiltChunk);
  uint32_t* gh = a.hist + (int64_t)r * kHistBins;
  const int64_t crow0 = (int64_t)r * a.n_chunks * kFiltChunk;
  const uint32_t* cnt = a.cand_count + (int64_t)r * a.n_chunks;
  // the chunks' candidate counts and the histogram are independent: both
  // loads fly together
  constexpr int kCpt = kMaxChunks / kSelThreads;
  int cc[kCpt];
#pragma unroll
  for (int i = 0; i < kCpt; ++i) {
    const int ch = kCpt * tid + i;
    cc[i] = (int)cnt[min(ch, nch - 1)];
  }
  uint32_t hv[kHistBins / kSelThreads];
  hist_load<kSelThreads>(gh, hv);
  const RowThreshold th = hist_threshold<kSelThreads>(hv, a.k, sh.wsum, sh.pair);
  const int bstar = th.bstar, c_above = th.c_above;
  const uint32_t kk = th.kk;

  // flattened candidate offsets: chunk ch holds [coff[ch], coff[ch + 1])
  int n_cand;
  {
    int loc = 0;
#pragma unroll
    for (int i = 0; i < kCpt; ++i) {
      const int ch = kCpt * tid + i;
      cc[i] = ch < nch ? cc[i] : 0;
      loc += cc[i];
    }
    int base = block_excl_scan<kSelThreads>(loc, sh.wsum, n_cand);
#pragma unroll
    for (int i = 0; i < kCpt; ++i) {
      const int ch = kCpt * tid + i;
      if (ch < nch) sh.coff[ch] = base;
      base += cc[i];
    }
    if (tid == 0) sh.coff[nch] = n_cand;
    __syncthreads();
  }

  // threshold T: the kk-th largest composite key (kept keys are >= T); its
  // top 12 bits are b*, the rest is found digit by digit among the
  // candidates of bin b*
  const bool sort = a.im.mode == kItemsCand;
  uint64_t T = 0;
  int nsel;
  if (n_cand <= kSelThreads * kRegKeys) {                   // uniform
    // each thread holds a run of kRegKeys consecutive candidates
    const int j0 = tid * kRegKeys;
    const int nm = max(0, min(kRegKeys, n_cand - j0));
    uint64_t K[kRegKeys];
    {
      int lo = 0, hi = nch;                                  // last chunk with coff <= j0
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sh.coff[mid] <= j0) lo = mid; else hi = mid;
      }
      int ch = lo;
#pragma unroll
      for (int i = 0; i < kRegKeys; ++i) {
        K[i] = 0;
        if (i < nm) {
          while (sh.coff[ch + 1] <= j0 + i) ++ch;
          K[i] = a.cand[crow0 + (int64_t)ch * kFiltChunk + (j0 + i - sh.coff[ch])];
        }
      }
    }
    if (bstar >= 0) {
      int need = (int)kk - c_above;
      uint64_t prefix = (uint64_t)bstar;
      for (int step = 0; step < 7; ++step) {
        const int dshift = digit_shift(step), w = digit_width(step);
        const uint32_t dmask = (1u << w) - 1u;
        if (tid < 256) sh.hist[tid] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kRegKeys; ++i)
          if (i < nm && (K[i] >> (dshift + w)) == prefix) atomicAdd(&sh.hist[(K[i] >> dshift) & dmask], 1u);
        __syncthreads();
        pick_digit(sh, need);
        __syncthreads();
        need -= sh.above;
        prefix = (prefix << w) | (uint64_t)sh.digit;
        const bool done = sh.dcount == need || dshift == 0;  // every key with this prefix is kept
        __syncthreads();
        if (done) {
          T = prefix << dshift;
          break;
        }
      }
    }
    // kept keys, written in candidate order
    int nk = 0;
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i) nk += (i < nm && kk > 0 && K[i] >= T) ? 1 : 0;
    int nout;
    int slot = block_excl_scan<kSelThreads>(nk, sh.wsum, nout);
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i) {
      if (i < nm && kk > 0 && K[i] >= T) {
        if (slot < a.k) {
          if (sort) {
            sh.u.sel.pos[slot] = comp_pos(K[i]);
            sh.u.sel.score[slot] = comp_score(K[i]);
          } else {
            oi[slot] = comp_pos(K[i]);
            if (os) os[slot] = comp_score(K[i]);
          }
        }
        ++slot;
      }
    }
    nsel = min(nout, a.k);
  } else {
    // many candidates (wide ties): walk them in global memory, staging the
    // candidates of bin b* in LDS when they fit
    if (bstar >= 0) {
      if (tid == 0) sh.n_stage = 0;
      __syncthreads();
      for (int ch = 0; ch < nch; ++ch) {
        const int cn = (int)cnt[ch];
        for (int j = tid; j < cn; j += kSelThreads) {
          const uint64_t K = a.cand[crow0 + (int64_t)ch * kFiltChunk + j];
          if ((int)(K >> 52) == bstar) {
            const int slot = atomicAdd(&sh.n_stage, 1);
            if (slot < kStageCap) sh.u.stage[slot] = K;
          }
        }
      }
      __syncthreads();
      const int n_st = sh.n_stage;
      const bool staged = n_st <= kStageCap;
      int need = (int)kk - c_above;
      uint64_t prefix = (uint64_t)bstar;
      for (int step = 0; step < 7; ++step) {
        const int dshift = digit_shift(step), w = digit_width(step);
        const uint32_t dmask = (1u << w) - 1u;
        if (tid < 256) sh.hist[tid] = 0u;
        __syncthreads();
        if (staged) {
          for (int j = tid; j < n_st; j += kSelThreads) {
            const uint64_t K = sh.u.stage[j];
            if ((K >> (dshift + w)) == prefix) atomicAdd(&sh.hist[(K >> dshift) & dmask], 1u);
          }
        } else {
          for (int ch = 0; ch < nch; ++ch) {
            const int cn = (int)cnt[ch];
            for (int j = tid; j < cn; j += kSelThreads) {
              const uint64_t K = a.cand[crow0 + (int64_t)ch * kFiltChunk + j];
              if ((K >> (dshift + w)) == prefix) atomicAdd(&sh.hist[(K >> dshift) & dmask], 1u);
            }
          }
        }
        __syncthreads();
        pick_digit(sh, need);
        __syncthreads();
        need -= sh.above;
        prefix = (prefix << w) | (uint64_t)sh.digit;
        const bool done = sh.dcount == need || dshift == 0;
        __syncthreads();
        if (done) {
          T = prefix << dshift;
          break;
        }
      }
    }
    int nout = 0;
    for (int base = 0; base < n_cand; base += kSelThreads) {
      const int j = base + tid;
      uint64_t K = 0;
      bool keep = false;
      if (j < n_cand && kk > 0) {
        int lo = 0, hi = nch;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (sh.coff[mid] <= j) lo = mid; else hi = mid;
        }
        K = a.cand[crow0 + (int64_t)lo * kFiltChunk + (j - sh.coff[lo])];
        keep = K >= T;
      }
      int t;
      const int slot = nout + block_excl_scan<kSelThreads>(keep ? 1 : 0, sh.wsum, t);
      if (keep && slot < a.k) {
        if (sort) {
          sh.u.sel.pos[slot] = comp_pos(K);
          sh.u.sel.score[slot] = comp_score(K);
        } else {
          oi[slot] = comp_pos(K);
          if (os) os[slot] = comp_score(K);
        }
      }
      nout += t;
    }
    nsel = min(nout, a.k);
  }

  // candidate mode: the caller's list has any order, sort by position
  if (sort) {
    int n2 = 1;
    while (n2 < nsel) n2 <<= 1;
    for (int i = nsel + tid; i < n2; i += kSelThreads) { sh.u.sel.pos[i] = 0x7FFFFFFF; sh.u.sel.score[i] = 0.f; }
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < n2; i += kSelThreads) {
          const int j = i ^ stride;
          if (j > i) {
            const bool up = (i & size) == 0;
            const int32_t pi = sh.u.sel.pos[i], pj = sh.u.sel.pos[j];
            if ((pi > pj) == up) {
              sh.u.sel.pos[i] = pj; sh.u.sel.pos[j] = pi;
              const float t2 = sh.u.sel.score[i]; sh.u.sel.score[i] = sh.u.sel.score[j]; sh.u.sel.score[j] = t2;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int j = tid; j < nsel; j += kSelThreads) {
      oi[j] = sh.u.sel.pos[j];
      if (os) os[j] = sh.u.sel.score[j];
    }
  }
  for (int j = nsel + tid; j < a.k; j += kSelThreads) {
    oi[j] = -1;
    if (os) os[j] = 0.0f;
  }

  // leave the row's histogram zeroed for the next call
  for (int b = tid; b < kHistBins; b += kSelThreads) gh[b] = 0u;
}

// ---------------------------------------------------------------------------
// Whole-row top-k: one workgroup of 1024 threads per row does filter and
// select together when the row is short enough to stream through one CU
// (used up to kRowMaxItems items, or with many rows).  The number of
// candidates -- items in bin b* or above -- is known from the histogram
// before any score is read, so they go to LDS when they fit, else to the
// row's candidate area in the workspace; the same code serves both.
// ---------------------------------------------------------------------------

constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kRowCap = 12288;                 // candidates held in LDS
constexpr int kRowU = 4;                        // float4 loads per thread per round
constexpr int kRowSub = kRowThreads * 4;        // items per sub-round (one float4 per thread)
constexpr int kRowRound = kRowSub * kRowU;      // items per round (one barrier)

struct RowShared {
  uint64_t cbuf[kRowCap];
  int32_t sel_pos[kMaxTopK];
  float sel_score[kMaxTopK];
  int wtot[2][kRowWaves][kRowU];
  int wsum[kRowWaves];
  uint32_t hist[256];
  int pair[3];
  int digit, above, dcount;
};

// One round's raw loads for one thread: items base + u*kRowSub + 4 tid + j
// (u, j < 4; the loads of a wave are contiguous) and, in pool mode, the id of
// the block each float4 belongs to.
struct RowRound {
  float4 v[kRowU];
  int32_t blk[kRowU];
};

// Raw loads of one round (addresses clamped into the row; masking happens in
// row_compact), unconditional so that nothing waits on them before use.
// Other modes than pool load a discarded word of the score row as block ids.
__device__ __forceinline__ void row_load(const SelectArgs& a, int r, const float* srow, int64_t base,
                                         RowRound& R) {
  const bool pool = a.im.mode == kItemsPool;
  const int32_t* lrow = pool ? a.im.list + (int64_t)r * a.im.list_len : reinterpret_cast<const int32_t*>(srow);
#pragma unroll
  for (int u = 0; u < kRowU; ++u) {
    const int64_t iu = base + (int64_t)u * kRowSub + 4 * threadIdx.x;
    R.v[u] = *reinterpret_cast<const float4*>(srow + (iu < a.row_stride ? iu : 0));
    R.blk[u] = lrow[pool && (iu >> 3) < a.im.list_len ? (iu >> 3) : 0];
  }
}

// Smallest score whose composite key lies in bin b* or above, as a float:
// for non-NaN x, x >= it exactly when order_key(x) >= b* << (32 - kHistBits)
// (the float order is the key order, and -0 and +0 share a key and compare
// equal).  NaN, the mark of items a row cannot see, compares false.  Bins
// below that of -inf hold only NaN patterns, so their threshold is -inf;
// bins above that of +inf hold none but NaN, whose threshold keeps nothing.
__device__ __forceinline__ float bin_floor(int bstar) {
  if (bstar < 0) return -INFINITY;                           // every visible item is kept
  const uint32_t k0 = (uint32_t)bstar << (32 - kHistBits);
  const float f = order_key_inv(k0);
  return (f != f && k0 < 0x80000000u) ? -INFINITY : f;
}

// Appends the round's items at or above the threshold to cbuf in item order.
// Within a sub-round u an item's slot counts the kept items of lower lanes
// (ballots of the bits of each lane's count) and of lower waves (per-wave
// totals in LDS, one lane per (u, wave) summed by a row scan).
__device__ __forceinline__ int row_compact(const SelectArgs& a, int r, int64_t nv, int64_t n_row, int64_t base,
                                           float thr, const RowRound& R, uint64_t* cbuf, int cap, int written,
                                           int parity, RowShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // items of the row from this thread's first one on (clamped to 32 bits)
  int rem = (int)max((int64_t)0, min(n_row - base - 4 * tid, (int64_t)kRowRound));
  asm volatile("" : "+v"(rem));                // 32-bit compares below, not 64-bit ones
  uint32_t fl[kRowU];
  int below[kRowU], wt[kRowU];
#pragma unroll
  for (int u = 0; u < kRowU; ++u) {
    const float x[4] = {R.v[u].x, R.v[u].y, R.v[u].z, R.v[u].w};
    fl[u] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) fl[u] |= (uint32_t)(x[j] >= thr && u * kRowSub + j < rem) << j;
    const int c = __popc(fl[u]);
    below[u] = 0;
    wt[u] = 0;
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const uint64_t m = __ballot((c >> b) & 1);
      below[u] += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
      wt[u] += __popcll(m) << b;
    }
  }
  if (lane == 0) *reinterpret_cast<int4*>(sh.wtot[parity][wave]) = make_int4(wt[0], wt[1], wt[2], wt[3]);
  lds_barrier();                               // the next round's loads stay in flight
  // lane (u = lane / 16, w = lane % 16) holds wave w's count of sub-round u;
  // an inclusive scan over each row of 16 lanes gives the waves' prefixes
  int sc = sh.wtot[parity][lane & 15][lane >> 4];
  sc += __builtin_amdgcn_update_dpp(0, sc, 0x111, 0xF, 0xF, true);   // row_shr:1
  sc += __builtin_amdgcn_update_dpp(0, sc, 0x112, 0xF, 0xF, true);   // row_shr:2
  sc += __builtin_amdgcn_update_dpp(0, sc, 0x114, 0xF, 0xF, true);   // row_shr:4
  sc += __builtin_amdgcn_update_dpp(0, sc, 0x118, 0xF, 0xF, true);   // row_shr:8
  const int64_t i0 = base + 4 * tid;
  int start = written;
#pragma unroll
  for (int u = 0; u < kRowU; ++u) {
    const int incl = __builtin_amdgcn_readlane(sc, 16 * u + wave);   // waves <= this one
    const int tot = __builtin_amdgcn_readlane(sc, 16 * u + 15);
    int slot = start + incl - wt[u] + below[u];
    const int64_t iu = i0 + (int64_t)u * kRowSub;
    if (a.im.mode == kItemsPool) {                             // uniform
      const int64_t pb = (int64_t)R.blk[u] * kBlockPos + (iu & 7);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((fl[u] >> j) & 1) {
          const float xj = j == 0 ? R.v[u].x : j == 1 ? R.v[u].y : j == 2 ? R.v[u].z : R.v[u].w;
          if (slot < cap) cbuf[slot] = comp_key(order_key(xj), pb + j);
          ++slot;
        }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((fl[u] >> j) & 1) {
          const float xj = j == 0 ? R.v[u].x : j == 1 ? R.v[u].y : j == 2 ? R.v[u].z : R.v[u].w;
          const int64_t pos = a.im.mode == kItemsCand ? item_pos(a.im, r, iu + j, nv) : iu + j;
          if (slot < cap) cbuf[slot] = comp_key(order_key(xj), pos);
          ++slot;
        }
    }
    start += tot;
  }
  return start;
}

// Collect, select and write one row with the candidates in cbuf (LDS or
// global).  Returns the number of ids written to the output (<= k).
__device__ __forceinline__ int row_select(const SelectArgs& a, int r, int64_t nv, int64_t n_row,
                                          const RowThreshold& th, RowRound& A, uint64_t* cbuf, int cap,
                                          RowShared& sh, int32_t* oi, float* os, bool sort) {
  const int tid = threadIdx.x;
  const float* srow = a.scores + (int64_t)r * a.row_stride;

  // 1. candidates in item order (A holds round 0, loaded before the threshold
  // search; a row longer than one round waits for each further round)
  const float thr = bin_floor(th.bstar);
  int written = 0, parity = 0;
  for (int64_t base = 0;; base += kRowRound) {
    written = row_compact(a, r, nv, n_row, base, thr, A, cbuf, cap, written, parity, sh);
    parity ^= 1;
    if (base + kRowRound >= n_row) break;
    row_load(a, r, srow, base + kRowRound, A);
  }
  __syncthreads();
  const int n_cand = min(written, cap);        // equal to th.n_cand: the histogram counted these items

  // 2. threshold key T among the candidates of bin b*
  uint64_t T = 0;
  if (th.bstar >= 0) {
    int need = (int)th.kk - th.c_above;
    uint64_t prefix = (uint64_t)th.bstar;
    for (int step = 0; step < 7; ++step) {
      const int dshift = digit_shift(step), w = digit_width(step);
      const uint32_t dmask = (1u << w) - 1u;
      if (tid < 256) sh.hist[tid] = 0u;
      __syncthreads();
      for (int j = tid; j < n_cand; j += kRowThreads) {
        const uint64_t K = cbuf[j];
        if ((K >> (dshift + w)) == prefix) atomicAdd(&sh.hist[(K >> dshift) & dmask], 1u);
      }
      __syncthreads();
      pick_digit(sh, need);
      __syncthreads();
      need -= sh.above;
      prefix = (prefix << w) | (uint64_t)sh.digit;
      const bool done = sh.dcount == need || dshift == 0;    // every key with this prefix is kept
      __syncthreads();
      if (done) {
        T = prefix << dshift;
        break;
      }
    }
  }

  // 3. kept keys (>= T) in candidate order: each thread a run of them
  const int per = (n_cand + kRowThreads - 1) / kRowThreads;
  const int j0 = tid * per, j1 = min(j0 + per, n_cand);
  int nk = 0;
  if (th.kk > 0)
    for (int j = j0; j < j1; ++j) nk += cbuf[j] >= T ? 1 : 0;
  int nout;
  int slot = block_excl_scan<kRowThreads>(nk, sh.wsum, nout);
  if (th.kk > 0) {
    for (int j = j0; j < j1; ++j) {
      const uint64_t K = cbuf[j];
      if (K >= T) {
        if (slot < a.k) {
          if (sort) {
            sh.sel_pos[slot] = comp_pos(K);
            sh.sel_score[slot] = comp_score(K);
          } else {
            oi[slot] = comp_pos(K);
            if (os) os[slot] = comp_score(K);
          }
        }
        ++slot;
      }
    }
  }
  return min(nout, a.k);
}

__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(SelectArgs a) {
  extern __shared__ __align__(16) unsigned char row_smem[];
  RowShared& sh = *reinterpret_cast<RowShared*>(row_smem);
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t nv = row_valid(a.im, r);
  const int64_t n_row = row_items(a.im, nv);
  int32_t* oi = a.out_idx + (int64_t)r * a.k;
  float* os = a.out_score ? a.out_score + (int64_t)r * a.k : nullptr;
  uint32_t* gh = a.hist + (int64_t)r * kHistBins;
  const bool sort = a.im.mode == kItemsCand;
  int nsel = 0;
  if (n_row > 0) {                                             // uniform
    uint32_t hv[kHistBins / kRowThreads];
    hist_load<kRowThreads>(gh, hv);
    RowRound A;                                                // the first round's scores fly
    row_load(a, r, a.scores + (int64_t)r * a.row_stride, 0, A);   // during the threshold search
    const RowThreshold th = hist_threshold<kRowThreads>(hv, a.k, sh.wsum, sh.pair);
    if (th.n_cand <= kRowCap)
      nsel = row_select(a, r, nv, n_row, th, A, sh.cbuf, kRowCap, sh, oi, os, sort);
    else
      nsel = row_select(a, r, nv, n_row, th, A, a.cand + (int64_t)r * a.n_chunks * kFiltChunk,
                        a.n_chunks * kFiltChunk, sh, oi, os, sort);
  }
  if (sort) {                                                  // candidate lists come in any order
    __syncthreads();
    int n2 = 1;
    while (n2 < nsel) n2 <<= 1;
    for (int i = nsel + tid; i < n2; i += kRowThreads) { sh.sel_pos[i] = 0x7FFFFFFF; sh.sel_score[i] = 0.f; }
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < n2; i += kRowThreads) {
          const int j = i ^ stride;
          if (j > i) {
            const bool up = (i & size) == 0;
            const int32_t pi = sh.sel_pos[i], pj = sh.sel_pos[j];
            if ((pi > pj) == up) {
              sh.sel_pos[i] = pj; sh.sel_pos[j] = pi;
              const float t2 = sh.sel_score[i]; sh.sel_score[i] = sh.sel_score[j]; sh.sel_score[j] = t2;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int j = tid; j < nsel; j += kRowThreads) {
      oi[j] = sh.sel_pos[j];
      if (os) os[j] = sh.sel_score[j];
    }
  }
  for (int j = nsel + tid; j < a.k; j += kRowThreads) {
    oi[j] = -1;
    if (os) os[j] = 0.0f;
  }
  // leave the row's histogram zeroed for the next call
  if (n_row > 0)
    for (int b = tid; b < kHistBins; b += kRowThreads) gh[b] = 0u;
}

hipError_t launch_topk_row(const SelectArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_row_kernel),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)sizeof(RowShared));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)a.n_rows), dim3(kRowThreads), sizeof(RowShared), stream, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(((int64_t)n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, (int64_t)n);
  return hipGetLastError();
}

hipError_t launch_topk_filter(const SelectArgs& a, hipStream_t stream) {
  if (a.n_rows == 0 || a.n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)a.n_chunks, (unsigned)a.n_rows),
                     dim3(kFiltThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_topk_select(const SelectArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)a.n_rows), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa2
