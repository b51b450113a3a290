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
//   rows of up to 16384 items: one 1024-thread workgroup per row holds the
//               row's keys in registers (16 per thread) and does both.
//   longer rows with many rows per call (a prefill chunk): one workgroup
//               per row streams the row, compacting candidates in LDS (the
//               workspace when they do not fit), and selects.
// The select leaves the row histogram zeroed for the next call.
#include "csa2_dev.h"
#include "csa2_launch.h"
#include "items.h"

namespace csa2 {

// ---------------------------------------------------------------------------
// filter (many workgroups per row) + select (one workgroup per row)
// ---------------------------------------------------------------------------

constexpr int kFiltThreads = 256;

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
__device__ __forceinline__ float4 load_items4_raw(const float* srow, int64_t i0, int64_t stride) {
  return *reinterpret_cast<const float4*>(srow + (i0 < stride ? i0 : 0));
}
__device__ __forceinline__ float4 mask_items4(float4 t, int64_t i0, int64_t n_row) {
  const float nan = __uint_as_float(0x7FC00000u);
  return make_float4(i0 + 0 < n_row ? t.x : nan, i0 + 1 < n_row ? t.y : nan,
                     i0 + 2 < n_row ? t.z : nan, i0 + 3 < n_row ? t.w : nan);
}

// On a path that discards loads issued above it (an early exit), mark them
// used there, so that the compiler cannot sink them below the branch into
// the path that uses them (where they would wait for the row's other loads
// before going out).
template <int N, int M>
__device__ __forceinline__ void keep_loads_above(const float4 (&v)[N], const uint32_t (&h)[M]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(v[i].x));
#pragma unroll
  for (int i = 0; i < M; ++i) asm volatile("" ::"v"(h[i]));
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

constexpr int kSelThreads = 1024;  // select workgroup

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


// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts and row
// broadcasts; lanes a shift does not reach add 0).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive prefix sum over the NT threads of a workgroup in thread order,
// and the total; one barrier.  wsum[NT/64] must not be reused by another scan
// before a further barrier.
template <int NT>
__device__ __forceinline__ int dpp_block_scan(int v, int* wsum, int& total) {
  constexpr int kW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int x = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = x;
  lds_barrier();
  const int ws = lane < kW ? wsum[lane] : 0;
  const int wi = wave_incl_scan(ws);
  total = __builtin_amdgcn_readlane(wi, kW - 1);
  const int before = wave > 0 ? __builtin_amdgcn_readlane(wi, wave - 1) : 0;
  return before + x - v;
}

// b* and the counts of a row's histogram, thread t holding the kB = 4096/NT
// bins 4095 - kB*t - i (i < kB, descending): the bin of the kk-th largest
// score, the items above it and in it; b* = -1 when every visible item is
// kept.  Two barriers; thr[0..2] is read back by every thread.  (Returned as
// RowThreshold{b*, above, in b*, kk}: its third field holds the count in b*.)
template <int NT>
__device__ __forceinline__ RowThreshold dpp_threshold(const uint32_t (&hv)[kHistBins / NT], int k, int* wsum,
                                                      int* thr) {
  constexpr int kB = kHistBins / NT;
  int loc = 0;
#pragma unroll
  for (int i = 0; i < kB; ++i) loc += (int)hv[i];
  int total;
  const int above = dpp_block_scan<NT>(loc, wsum, total);   // items in the bins above this thread's
  const uint32_t kk = min((uint32_t)k, (uint32_t)total);
  if (threadIdx.x == 0 && kk >= (uint32_t)total) { thr[0] = -1; thr[1] = 0; thr[2] = total; }
  if (kk < (uint32_t)total && (uint32_t)above < kk && (uint32_t)(above + loc) >= kk) {
    uint32_t cum = (uint32_t)above;
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      if (cum < kk && cum + hv[i] >= kk) {
        thr[0] = kHistBins - 1 - kB * (int)threadIdx.x - i; thr[1] = (int)cum; thr[2] = (int)hv[i];
      }
      cum += hv[i];
    }
  }
  lds_barrier();
  return RowThreshold{thr[0], thr[1], thr[2], kk};
}

// Loads the kB bins of thread t, descending (see dpp_threshold).
template <int NT>
__device__ __forceinline__ void hist_load_desc(const uint32_t* gh, uint32_t (&hv)[kHistBins / NT]) {
  constexpr int kB = kHistBins / NT;
#pragma unroll
  for (int q = 0; q < kB / 4; ++q) {
    const uint4 h = *reinterpret_cast<const uint4*>(gh + kHistBins - kB * (threadIdx.x + 1) + 4 * (kB / 4 - 1 - q));
    hv[4 * q] = h.w; hv[4 * q + 1] = h.z; hv[4 * q + 2] = h.y; hv[4 * q + 3] = h.x;
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

// Filter.  Workgroup (chunk c, row r) finds b* and writes every item of its
// chunk in b* or above -- a superset of the chunk's share of the top-k -- as
// composite keys, compacted in item order, plus their count.  Thread t owns
// the chunk's items 16t .. 16t+15, so one block scan places them all.
constexpr int kFiltPer = kFiltChunk / kFiltThreads;           // items per thread
static_assert(kFiltPer == 16, "16 items per filter thread");
__global__ __launch_bounds__(kFiltThreads) void topk_filter_kernel(SelectArgs a) {
  __shared__ int wsum[2][kFiltThreads / 64];
  __shared__ int thr[4];
  const int r = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int64_t c0 = (int64_t)c * kFiltChunk;

  // this thread's items and its bins, loaded first: their addresses do not
  // depend on the row's sequence and count, whose loads then overlap them
  const float* srow = a.scores + (int64_t)r * a.row_stride;
  const int64_t i0 = c0 + (int64_t)kFiltPer * tid;
  float4 raw[kFiltPer / 4];
#pragma unroll
  for (int u = 0; u < kFiltPer / 4; ++u) raw[u] = load_items4_raw(srow, i0 + 4 * u, a.row_stride);
  uint32_t hv[kHistBins / kFiltThreads];
  hist_load_desc<kFiltThreads>(a.hist + (int64_t)r * kHistBins, hv);

  const int64_t nv = row_valid(a.im, r);
  const int64_t n_row = row_items(a.im, nv);
  if (c0 >= n_row) {                                           // uniform
    keep_loads_above(raw, hv);
    return;
  }
  const int64_t c1 = min(c0 + (int64_t)kFiltChunk, n_row);
  float v[kFiltPer];
#pragma unroll
  for (int u = 0; u < kFiltPer / 4; ++u) {
    const float4 q = mask_items4(raw[u], i0 + 4 * u, c1);
    v[4 * u] = q.x; v[4 * u + 1] = q.y; v[4 * u + 2] = q.z; v[4 * u + 3] = q.w;
  }
  const RowThreshold th = dpp_threshold<kFiltThreads>(hv, a.k, wsum[0], thr);

  // compaction in item order
  const float thf = bin_floor(th.bstar);
  uint32_t flag = 0;
#pragma unroll
  for (int i = 0; i < kFiltPer; ++i) flag |= (uint32_t)(v[i] >= thf) << i;   // NaN (not visible) compares false
  int tot;
  int slot = dpp_block_scan<kFiltThreads>(__popc(flag), wsum[1], tot);
  uint64_t* crow = a.cand + ((int64_t)r * a.n_chunks + c) * kFiltChunk;
#pragma unroll
  for (int i = 0; i < kFiltPer; ++i) {
    if ((flag >> i) & 1u) crow[slot++] = comp_key(order_key(v[i]), item_pos(a.im, r, i0 + i, nv));
  }
  if (tid == 0) a.cand_count[(int64_t)r * a.n_chunks + c] = (uint32_t)tot;
}


// ---------------------------------------------------------------------------
// Register-resident selection.  Every thread of a 1024-thread workgroup holds
// NK composite keys of a run of consecutive items (0 = not a candidate), the
// runs in item order across threads.  The row's histogram gives b*; the k-th
// key T is settled by a radix select over the keys of bin b* with one barrier
// per digit (three LDS histograms in rotation: the one a step fills, the one
// the next step fills -- cleared two steps before -- and the one being
// cleared), every wave taking the same digit decision from the same counts;
// the kept keys (K >= T) are written in item order after one block scan.
// ---------------------------------------------------------------------------

constexpr int kRegThreads = 1024;
constexpr int kRegWaves = kRegThreads / 64;

struct __align__(16) RegShared {
  uint32_t h[3][256];               // radix digit counts, rotated per step
  int wsum[2][kRegWaves];           // wave totals of the two block scans
  int thr[4];                       // b*, items above b*, items in b*
  int flag;
};

// The k-th composite key among the candidates: b* fixes its top 12 bits,
// radix steps over the keys of bin b* the rest.  need = kk - items above b*,
// in_bin = items in b*.  sh.h[0] and sh.h[1] must be zero on entry (and
// their zeroing ordered before it by a barrier).  Uniform result.
template <int NK>
__device__ __forceinline__ uint64_t reg_radix(const uint64_t (&K)[NK], int bstar, int need, int in_bin,
                                              RegShared& sh) {
  if (bstar < 0) return 0;                                   // every candidate is kept
  uint64_t prefix = (uint64_t)bstar;
  if (need == in_bin) return prefix << 52;                   // the whole bin is kept
  const int lane = threadIdx.x & 63;
  for (int step = 0; step < 7; ++step) {
    const int dshift = digit_shift(step), w = digit_width(step);
    const uint32_t dmask = (1u << w) - 1u;
    uint32_t* H = sh.h[step % 3];
#pragma unroll
    for (int i = 0; i < NK; ++i)
      if (K[i] != 0 && (K[i] >> (dshift + w)) == prefix) atomicAdd(&H[(K[i] >> dshift) & dmask], 1u);
    lds_barrier();
    // every wave: lane l holds digits 255-4l .. 252-4l (descending); the
    // digit whose count crosses `need` from the top
    const uint4 hq = *reinterpret_cast<const uint4*>(&H[252 - 4 * lane]);
    const uint32_t hv[4] = {hq.w, hq.z, hq.y, hq.x};
    const int loc = (int)(hv[0] + hv[1] + hv[2] + hv[3]);
    const int incl = wave_incl_scan(loc);
    const int excl = incl - loc;
    int digit = 0, above = 0, dcount = 0;
    if (excl < need && incl >= need) {
      int cum = excl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (cum < need && cum + (int)hv[i] >= need) { digit = 255 - 4 * lane - i; above = cum; dcount = (int)hv[i]; }
        cum += (int)hv[i];
      }
    }
    const uint64_t hit = __ballot(excl < need && incl >= need);
    const int src = (int)__builtin_ctzll(hit);
    digit = __builtin_amdgcn_readlane(digit, src);
    above = __builtin_amdgcn_readlane(above, src);
    dcount = __builtin_amdgcn_readlane(dcount, src);
    if (threadIdx.x < 256) sh.h[(step + 2) % 3][threadIdx.x] = 0u;   // read by the previous step only
    need -= above;
    prefix = (prefix << w) | (uint64_t)digit;
    if (dcount == need || dshift == 0) return prefix << dshift;
  }
  return prefix;                                             // not reached
}

// Writes the kept keys (K != 0 and K >= T, none when kk == 0) of one set of
// per-thread runs at slots base + their rank in item order (those below k)
// to out_idx / out_score; returns how many the set keeps.  One barrier.
template <int NK>
__device__ __forceinline__ int reg_emit_at(const uint64_t (&K)[NK], uint64_t T, uint32_t kk, int k, int base,
                                           int32_t* oi, float* os, RegShared& sh) {
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < NK; ++i) cnt += (kk > 0 && K[i] != 0 && K[i] >= T) ? 1 : 0;
  int total;
  int slot = base + dpp_block_scan<kRegThreads>(cnt, sh.wsum[1], total);
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    if (kk > 0 && K[i] != 0 && K[i] >= T) {
      if (slot < k) {
        oi[slot] = comp_pos(K[i]);
        if (os) os[slot] = comp_score(K[i]);
      }
      ++slot;
    }
  }
  lds_barrier();                         // wsum[1] is free for the next set
  return total;
}

// As reg_emit_at from slot 0, then the -1 padding up to k; returns the count
// written (<= k).
template <int NK>
__device__ __forceinline__ int reg_emit(const uint64_t (&K)[NK], uint64_t T, uint32_t kk, int k, int32_t* oi,
                                        float* os, RegShared& sh) {
  const int n = min(reg_emit_at(K, T, kk, k, 0, oi, os, sh), k);
  for (int j = n + (int)threadIdx.x; j < k; j += kRegThreads) {
    oi[j] = -1;
    if (os) os[j] = 0.0f;
  }
  return n;
}

// The k-th composite key among n composite keys in LDS (the candidates of a
// row, bin b* or above), as reg_radix: thread t counts keys t, t + 1024, ...
// of bin b*'s prefix per digit.  sh.h[0] and sh.h[1] must be zero on entry.
__device__ __forceinline__ uint64_t lds_radix(const uint64_t* cand, int n, int bstar, int need, int in_bin,
                                              RegShared& sh) {
  if (bstar < 0) return 0;                                   // every candidate is kept
  uint64_t prefix = (uint64_t)bstar;
  if (need == in_bin) return prefix << 52;                   // the whole bin is kept
  const int lane = threadIdx.x & 63;
  for (int step = 0; step < 7; ++step) {
    const int dshift = digit_shift(step), w = digit_width(step);
    const uint32_t dmask = (1u << w) - 1u;
    uint32_t* H = sh.h[step % 3];
    for (int j = threadIdx.x; j < n; j += kRegThreads) {
      const uint64_t K = cand[j];
      if ((K >> (dshift + w)) == prefix) atomicAdd(&H[(K >> dshift) & dmask], 1u);
    }
    lds_barrier();
    const uint4 hq = *reinterpret_cast<const uint4*>(&H[252 - 4 * lane]);
    const uint32_t hv[4] = {hq.w, hq.z, hq.y, hq.x};
    const int loc = (int)(hv[0] + hv[1] + hv[2] + hv[3]);
    const int incl = wave_incl_scan(loc);
    const int excl = incl - loc;
    int digit = 0, above = 0, dcount = 0;
    if (excl < need && incl >= need) {
      int cum = excl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (cum < need && cum + (int)hv[i] >= need) { digit = 255 - 4 * lane - i; above = cum; dcount = (int)hv[i]; }
        cum += (int)hv[i];
      }
    }
    const int src = (int)__builtin_ctzll(__ballot(excl < need && incl >= need));
    digit = __builtin_amdgcn_readlane(digit, src);
    above = __builtin_amdgcn_readlane(above, src);
    dcount = __builtin_amdgcn_readlane(dcount, src);
    if (threadIdx.x < 256) sh.h[(step + 2) % 3][threadIdx.x] = 0u;
    need -= above;
    prefix = (prefix << w) | (uint64_t)digit;
    if (dcount == need || dshift == 0) return prefix << dshift;
  }
  return prefix;                                             // not reached
}

// Whole rows of at most kRegRowItems items (flat, block or pool mode): thread
// t loads items 16t .. 16t+15.  When the row's candidates (its items in b*
// or above, counted by the histogram) fit in LDS they are compacted there in
// item order first -- each thread writing only its candidates' (score,
// position) at the slots one block scan gives -- and the radix steps and the
// output walk the candidates alone, a few per thread; otherwise every thread
// keeps its 16 keys in registers (reg_radix, reg_emit).
constexpr int kRegRowNK = 16;
constexpr int kRowCompactCap = 12288;            // candidates compacted in LDS

struct __align__(16) RegRowShared {
  RegShared reg;
  uint64_t cand[kRowCompactCap];                 // (score bits, position), then their composite keys
};

__global__ __launch_bounds__(kRegThreads) void topk_reg_row_kernel(SelectArgs a) {
  extern __shared__ __align__(16) unsigned char reg_row_smem[];
  RegRowShared& shr = *reinterpret_cast<RegRowShared*>(reg_row_smem);
  RegShared& sh = shr.reg;
  const int r = blockIdx.x, tid = threadIdx.x;
  // the row's bins, scores and (pool) block ids first: their addresses do
  // not depend on the row's sequence and count, whose loads then overlap them
  uint32_t* gh = a.hist + (int64_t)r * kHistBins;
  uint32_t hv[kHistBins / kRegThreads];
  hist_load_desc<kRegThreads>(gh, hv);
  const float* srow = a.scores + (int64_t)r * a.row_stride;
  const int i0 = kRegRowNK * tid;
  float4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int iu = i0 + 4 * u;
    v[u] = *reinterpret_cast<const float4*>(srow + (iu < a.row_stride ? iu : 0));
  }
  int32_t blk[2] = {0, 0};
  if (a.im.mode == kItemsPool) {                               // uniform
    const int32_t* lrow = a.im.list + (int64_t)r * a.im.list_len;
    blk[0] = lrow[min(2 * tid, a.im.list_len - 1)];
    blk[1] = lrow[min(2 * tid + 1, a.im.list_len - 1)];
  }
  const int64_t nv = row_valid(a.im, r);
  const int n_row = (int)row_items(a.im, nv);
  int32_t* oi = a.out_idx + (int64_t)r * a.k;
  float* os = a.out_score ? a.out_score + (int64_t)r * a.k : nullptr;
  if (n_row == 0) {                                            // uniform: nothing visible
    keep_loads_above(v, hv);
    asm volatile("" ::"v"(blk[0]), "v"(blk[1]));
    for (int j = tid; j < a.k; j += kRegThreads) {
      oi[j] = -1;
      if (os) os[j] = 0.0f;
    }
    return;
  }
  if (tid < 256) { sh.h[0][tid] = 0u; sh.h[1][tid] = 0u; }
  const RowThreshold th = dpp_threshold<kRegThreads>(hv, a.k, sh.wsum[0], sh.thr);   // its barriers order the zeroing too
  const float thr = bin_floor(th.bstar);
  const int n_cand = th.c_above + th.n_cand;                   // items in b* or above (every visible one if b* < 0)
  const int need = (int)th.kk - th.c_above;
  if (n_cand <= kRowCompactCap) {                              // uniform
    // 1. the candidates' (score, position), compacted in item order
    uint32_t mask = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) mask |= (uint32_t)(i0 + 4 * u + j < n_row && x4[j] >= thr) << (4 * u + j);
    }
    int tot;
    int slot = dpp_block_scan<kRegThreads>(__popc(mask), sh.wsum[1], tot);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int item = i0 + 4 * u + j;
        const int32_t pos = a.im.mode == kItemsPool ? blk[(4 * u + j) >> 3] * kBlockPos + (item & 7) : item;
        if ((mask >> (4 * u + j)) & 1u) {
          shr.cand[slot] = ((uint64_t)(uint32_t)pos << 32) | __float_as_uint(x4[j]);
          ++slot;
        }
      }
    }
    lds_barrier();
    const int nc = min(tot, kRowCompactCap);                   // tot == n_cand: the histogram counted them
    for (int j = tid; j < nc; j += kRegThreads) {
      const uint64_t c = shr.cand[j];
      shr.cand[j] = comp_key(order_key(__uint_as_float((uint32_t)c)), (int32_t)(c >> 32));
    }
    lds_barrier();
    // 2. the k-th key among them
    const uint64_t T = lds_radix(shr.cand, nc, th.bstar, need, th.n_cand, sh);
    // 3. the kept ones (>= T), in candidate order: thread t a run of them
    const int per = (nc + kRegThreads - 1) / kRegThreads;
    const int j0 = tid * per, j1 = min(j0 + per, nc);
    int cnt = 0;
    if (th.kk > 0)
      for (int j = j0; j < j1; ++j) cnt += shr.cand[j] >= T ? 1 : 0;
    int nout;
    int o = dpp_block_scan<kRegThreads>(cnt, sh.wsum[1], nout);
    if (th.kk > 0) {
      for (int j = j0; j < j1; ++j) {
        const uint64_t K = shr.cand[j];
        if (K >= T) {
          if (o < a.k) {
            oi[o] = comp_pos(K);
            if (os) os[o] = comp_score(K);
          }
          ++o;
        }
      }
    }
    for (int j = min(nout, a.k) + tid; j < a.k; j += kRegThreads) {
      oi[j] = -1;
      if (os) os[j] = 0.0f;
    }
  } else {
    uint64_t K[kRegRowNK];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int item = i0 + 4 * u + j;
        const float x = x4[j];
        const bool cand = item < n_row && x >= thr;            // NaN (not visible) compares false
        const int32_t pos = a.im.mode == kItemsPool ? blk[(4 * u + j) >> 3] * kBlockPos + (item & 7) : item;
        K[4 * u + j] = cand ? comp_key(order_key(x), pos) : 0ull;
      }
    }
    const uint64_t T = reg_radix(K, th.bstar, need, th.n_cand, sh);
    reg_emit(K, T, th.kk, a.k, oi, os, sh);
  }
  // leave the row's histogram zeroed for the next call
  *reinterpret_cast<uint4*>(gh + kHistBins - 4 - 4 * tid) = make_uint4(0u, 0u, 0u, 0u);
}

// Select after the filter: one workgroup per row settles the k-th composite
// key T among the filter's candidates (compacted per chunk in item order, so
// candidate order is ascending position) and writes the kept ones in that
// order; candidate mode (caller lists in any order) sorts them by position
// in LDS first.  Thread t speculatively loads 8 candidate slots of chunk
// t / TPC (TPC threads per chunk, from the launch's chunk count) before the
// chunks' counts are known; when
// no chunk holds more candidates than its threads' slots, the keys are then
// in registers (slots past a chunk's count are masked).  Otherwise (wide
// ties) the same steps walk every chunk's candidates in global memory,
// 8192 per pass.
constexpr int kSelNK = 8;

struct __align__(16) SelShared {
  RegShared reg;
  int32_t pos[kMaxTopK];                  // candidate mode: kept ids and scores, sorted here
  float score[kMaxTopK];
};

// One pass of the global walk: the 8 candidate slots of global slot index
// (pass * kSelThreads + t) * 8 (chunk-major; past a chunk's count -> 0).
__device__ __forceinline__ void sel_pass_keys(const SelectArgs& a, int r, int nch, int pass, uint64_t (&K)[kSelNK]) {
  const int64_t g = ((int64_t)pass * kSelThreads + threadIdx.x) * kSelNK;
  const int c = (int)min(g / kFiltChunk, (int64_t)nch - 1);
  const int s0 = (int)(g - (int64_t)c * kFiltChunk);
  const bool in = g < (int64_t)nch * kFiltChunk;
  const int cnt = (int)a.cand_count[(int64_t)r * a.n_chunks + c];
  const uint64_t* crow = a.cand + ((int64_t)r * a.n_chunks + c) * kFiltChunk + (in ? s0 : 0);
#pragma unroll
  for (int i = 0; i < kSelNK; i += 2) {
    const uint4 q = *reinterpret_cast<const uint4*>(crow + i);
    K[i] = (in && s0 + i < cnt) ? (((uint64_t)q.y << 32) | q.x) : 0ull;
    K[i + 1] = (in && s0 + i + 1 < cnt) ? (((uint64_t)q.w << 32) | q.z) : 0ull;
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelectArgs a) {
  __shared__ SelShared shs;
  RegShared& sh = shs.reg;
  const int r = blockIdx.x, tid = threadIdx.x;
  // The row's bins, chunk counts and candidate slots go out first: their
  // addresses do not depend on the row's words, whose loads then overlap
  // them.  The slots are mapped for the launch's chunk count, TPC threads of
  // kSelNK slots per chunk (a row with fewer chunks leaves the threads past
  // its chunks idle; a chunk with more candidates than its slots takes the
  // walk over global memory below).
  uint32_t* gh = a.hist + (int64_t)r * kHistBins;
  uint32_t hv[kHistBins / kSelThreads];
  hist_load_desc<kSelThreads>(gh, hv);
  const int tpc = min(kFiltChunk / kSelNK, kSelThreads / a.n_chunks);  // 0 when there are more chunks than threads
  const int c = tpc > 0 ? min(tid / tpc, a.n_chunks - 1) : 0;
  const int s0 = tpc > 0 ? kSelNK * (tid % tpc) : 0;
  const int cnt = (int)a.cand_count[(int64_t)r * a.n_chunks + c];
  const uint64_t* crow = a.cand + ((int64_t)r * a.n_chunks + c) * kFiltChunk + s0;
  uint64_t K[kSelNK];
#pragma unroll
  for (int i = 0; i < kSelNK; i += 2) {
    const uint4 q = *reinterpret_cast<const uint4*>(crow + i);
    K[i] = ((uint64_t)q.y << 32) | q.x;
    K[i + 1] = ((uint64_t)q.w << 32) | q.z;
  }
  const int64_t nv = row_valid(a.im, r);
  const int64_t n_row = row_items(a.im, nv);
  int32_t* oi = a.out_idx + (int64_t)r * a.k;
  float* os = a.out_score ? a.out_score + (int64_t)r * a.k : nullptr;
  if (n_row == 0) {                                            // uniform: nothing visible
#pragma unroll
    for (int i = 0; i < kSelNK; ++i) asm volatile("" ::"v"(K[i]));   // the loads stay above the branch
#pragma unroll
    for (int i = 0; i < kHistBins / kSelThreads; ++i) asm volatile("" ::"v"(hv[i]));
    asm volatile("" ::"v"(cnt));
    for (int j = tid; j < a.k; j += kSelThreads) {
      oi[j] = -1;
      if (os) os[j] = 0.0f;
    }
    return;
  }
  const bool sort = a.im.mode == kItemsCand;
  const int nch = (int)((n_row + kFiltChunk - 1) / kFiltChunk);   // the row's chunks (<= a.n_chunks)
  if (tid < 256) { sh.h[0][tid] = 0u; sh.h[1][tid] = 0u; }
  if (tid == 0) sh.flag = tpc > 0 ? 0 : 1;
  lds_barrier();
  if (tpc > 0 && tid % tpc == 0 && tid < nch * tpc && cnt > kSelNK * tpc) sh.flag = 1;
  const RowThreshold th = dpp_threshold<kSelThreads>(hv, a.k, sh.wsum[0], sh.thr);   // its barriers publish the flag
  const bool spill = sh.flag != 0;                             // uniform: a chunk overflows its slots
  int32_t* sel_pos = sort ? shs.pos : oi;
  float* sel_score = sort ? shs.score : os;
  int nsel;
  if (!spill) {
    const bool mine = tid < nch * tpc;
#pragma unroll
    for (int i = 0; i < kSelNK; ++i) K[i] = (mine && s0 + i < cnt) ? K[i] : 0ull;
    const uint64_t T = reg_radix(K, th.bstar, (int)th.kk - th.c_above, th.n_cand, sh);
    nsel = reg_emit(K, T, th.kk, a.k, sel_pos, sel_score, sh);
  } else {
    const int passes = (int)(((int64_t)nch * kFiltChunk + kSelThreads * kSelNK - 1) / (kSelThreads * kSelNK));
    // T: the radix steps of reg_radix, each counting over every pass
    uint64_t T = 0;
    int need = (int)th.kk - th.c_above;
    if (th.bstar >= 0 && need != th.n_cand) {
      uint64_t prefix = (uint64_t)th.bstar;
      const int lane = tid & 63;
      for (int step = 0; step < 7; ++step) {
        const int dshift = digit_shift(step), w = digit_width(step);
        const uint32_t dmask = (1u << w) - 1u;
        uint32_t* H = sh.h[step % 3];
        for (int pass = 0; pass < passes; ++pass) {
          sel_pass_keys(a, r, nch, pass, K);
#pragma unroll
          for (int i = 0; i < kSelNK; ++i)
            if (K[i] != 0 && (K[i] >> (dshift + w)) == prefix) atomicAdd(&H[(K[i] >> dshift) & dmask], 1u);
        }
        lds_barrier();
        const uint4 q = *reinterpret_cast<const uint4*>(&H[252 - 4 * lane]);
        const uint32_t hv[4] = {q.w, q.z, q.y, q.x};
        const int loc = (int)(hv[0] + hv[1] + hv[2] + hv[3]);
        const int incl = wave_incl_scan(loc), excl = incl - loc;
        int digit = 0, above = 0, dcount = 0, cum = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (excl < need && incl >= need && cum < need && cum + (int)hv[i] >= need) {
            digit = 255 - 4 * lane - i; above = cum; dcount = (int)hv[i];
          }
          cum += (int)hv[i];
        }
        const int src = (int)__builtin_ctzll(__ballot(excl < need && incl >= need));
        digit = __builtin_amdgcn_readlane(digit, src);
        above = __builtin_amdgcn_readlane(above, src);
        dcount = __builtin_amdgcn_readlane(dcount, src);
        if (tid < 256) sh.h[(step + 2) % 3][tid] = 0u;
        need -= above;
        prefix = (prefix << w) | (uint64_t)digit;
        if (dcount == need || dshift == 0) { T = prefix << dshift; break; }
      }
    } else if (th.bstar >= 0) {
      T = (uint64_t)th.bstar << 52;
    }
    // the kept keys, pass by pass, in candidate order
    int base = 0;
    for (int pass = 0; pass < passes; ++pass) {
      sel_pass_keys(a, r, nch, pass, K);
      base += reg_emit_at(K, T, th.kk, a.k, base, sel_pos, sel_score, sh);
    }
    nsel = min(base, a.k);
    for (int j = nsel + tid; j < a.k; j += kSelThreads) {
      sel_pos[j] = -1;
      if (sel_score) sel_score[j] = 0.0f;
    }
  }
  if (sort) {                                                  // candidate lists come in any order
    __syncthreads();
    int n2 = 1;
    while (n2 < nsel) n2 <<= 1;
    for (int i = nsel + tid; i < n2; i += kSelThreads) { shs.pos[i] = 0x7FFFFFFF; shs.score[i] = 0.f; }
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < n2; i += kSelThreads) {
          const int j = i ^ stride;
          if (j > i) {
            const bool up = (i & size) == 0;
            const int32_t pi = shs.pos[i], pj = shs.pos[j];
            if ((pi > pj) == up) {
              shs.pos[i] = pj; shs.pos[j] = pi;
              const float t2 = shs.score[i]; shs.score[i] = shs.score[j]; shs.score[j] = t2;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int j = tid; j < a.k; j += kSelThreads) {
      oi[j] = j < nsel ? shs.pos[j] : -1;
      if (os) os[j] = j < nsel ? shs.score[j] : 0.0f;
    }
  }
  // leave the row's histogram zeroed for the next call
  *reinterpret_cast<uint4*>(gh + kHistBins - 4 - 4 * tid) = make_uint4(0u, 0u, 0u, 0u);
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
typedef float f4nt __attribute__((ext_vector_type(4)));

struct RowRound {
  float4 v[kRowU];
  int32_t blk[kRowU];
};

// Raw loads of one round (addresses clamped into the row; masking happens in
// row_compact), unconditional so that nothing waits on them before use.
// POOL: pool mode, whose block ids are loaded beside the scores (the other
// modes neither load nor hold them).
template <bool POOL>
__device__ __forceinline__ void row_load(const SelectArgs& a, int r, const float* srow, int64_t base,
                                         RowRound& R) {
#pragma unroll
  for (int u = 0; u < kRowU; ++u) {
    const int64_t iu = base + (int64_t)u * kRowSub + 4 * threadIdx.x;
    // non-temporal: each score is read once here
    const f4nt t = __builtin_nontemporal_load(reinterpret_cast<const f4nt*>(srow + (iu < a.row_stride ? iu : 0)));
    R.v[u] = make_float4(t[0], t[1], t[2], t[3]);
    if (POOL) R.blk[u] = a.im.list[(int64_t)r * a.im.list_len + ((iu >> 3) < a.im.list_len ? (iu >> 3) : 0)];
  }
}


// Appends the round's items at or above the threshold to cbuf in item order.
// Within a sub-round u an item's slot counts the kept items of lower lanes
// (ballots of the bits of each lane's count) and of lower waves (per-wave
// totals in LDS, one lane per (u, wave) summed by a row scan).
template <bool POOL>
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
    if (POOL) {
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
template <bool POOL>
__device__ __forceinline__ int row_select(const SelectArgs& a, int r, int64_t nv, int64_t n_row,
                                          const RowThreshold& th, RowRound& A, RowRound& B, uint64_t* cbuf,
                                          int cap, RowShared& sh, int32_t* oi, float* os, bool sort) {
  const int tid = threadIdx.x;
  const float* srow = a.scores + (int64_t)r * a.row_stride;

  // 1. candidates in item order.  A and B hold rounds 0 and 1, loaded before
  // the threshold search; while one round is compacted the next is in
  // flight, and its successor is loaded as soon as its registers are free.
  // The loads are unconditional (clamped addresses; rounds past the row are
  // read and ignored) so that each wait covers only its own round.
  const float thr = bin_floor(th.bstar);
  int written = 0, parity = 0;
  for (int64_t base = 0;; base += 2 * kRowRound) {
    written = row_compact<POOL>(a, r, nv, n_row, base, thr, A, cbuf, cap, written, parity, sh);
    parity ^= 1;
    if (base + kRowRound >= n_row) break;
    row_load<POOL>(a, r, srow, base + 2 * kRowRound, A);
    written = row_compact<POOL>(a, r, nv, n_row, base + kRowRound, thr, B, cbuf, cap, written, parity, sh);
    parity ^= 1;
    if (base + 2 * kRowRound >= n_row) break;
    row_load<POOL>(a, r, srow, base + 3 * kRowRound, B);
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

// A row whose threshold bin holds more candidates than LDS takes, with no
// candidate area in global memory (a one-stage call that does not filter):
// the exact threshold key by the same radix steps as row_select, each a pass
// over the row's stored scores, then the kept items in item order, straight
// to the output.  Only degenerate rows come here (a threshold bin of more
// than kRowCap scores: many equal scores, such as a row of zero queries).
// Returns the number of ids written (<= k).
__device__ __forceinline__ int row_select_stream(const SelectArgs& a, int r, int64_t nv, int64_t n_row,
                                                 const RowThreshold& th, RowShared& sh, int32_t* oi, float* os,
                                                 bool sort) {
  const int tid = threadIdx.x;
  const float* srow = a.scores + (int64_t)r * a.row_stride;
  const float thr = bin_floor(th.bstar);
  const int32_t* lrow = a.im.mode == kItemsPool ? a.im.list + (int64_t)r * a.im.list_len : nullptr;
  // candidate j of this thread's four items i0 .. i0 + 3 (as row_compact:
  // visible and at or above the threshold bin; NaN compares false)
  auto keys4 = [&](int64_t i0, uint64_t (&K)[4]) {
    uint32_t f = 0;
    const float4 v = i0 < n_row ? *reinterpret_cast<const float4*>(srow + i0) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = i0 + j;
      K[j] = 0;
      if (i < n_row && x[j] >= thr) {
        int64_t pos = i;
        if (a.im.mode == kItemsPool) pos = (int64_t)lrow[i >> 3] * kBlockPos + (i & 7);
        else if (a.im.mode == kItemsCand) pos = item_pos(a.im, r, i, nv);
        K[j] = comp_key(order_key(x[j]), pos);
        f |= 1u << j;
      }
    }
    return f;
  };
  constexpr int64_t kStep = 4 * kRowThreads;

  uint64_t T = 0;
  int need = (int)th.kk - th.c_above;
  uint64_t prefix = (uint64_t)th.bstar;
  for (int step = 0; step < 7; ++step) {
    const int dshift = digit_shift(step), w = digit_width(step);
    const uint32_t dmask = (1u << w) - 1u;
    if (tid < 256) sh.hist[tid] = 0u;
    if (tid == 0) { sh.digit = 0; sh.above = 0; sh.dcount = 0; }
    __syncthreads();
    for (int64_t base = 0; base < n_row; base += kStep) {
      uint64_t K[4];
      const uint32_t f = keys4(base + 4 * tid, K);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (((f >> j) & 1u) && (K[j] >> (dshift + w)) == prefix) atomicAdd(&sh.hist[(K[j] >> dshift) & dmask], 1u);
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

  // the kept keys (>= T) in item order
  int written = 0;
  for (int64_t base = 0; base < n_row; base += kStep) {
    uint64_t K[4];
    uint32_t f = keys4(base + 4 * tid, K);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (K[j] < T) f &= ~(1u << j);
    int tot;
    int slot = written + dpp_block_scan<kRowThreads>(__popc(f), sh.wsum, tot);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((f >> j) & 1u) {
        if (slot < a.k) {
          if (sort) {
            sh.sel_pos[slot] = comp_pos(K[j]);
            sh.sel_score[slot] = comp_score(K[j]);
          } else {
            oi[slot] = comp_pos(K[j]);
            if (os) os[slot] = comp_score(K[j]);
          }
        }
        ++slot;
      }
    written += tot;
    __syncthreads();                             // sh.wsum is reused by the next scan
  }
  return min(written, a.k);
}

template <bool POOL>
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
    RowRound A, B;                                             // the first two rounds' scores fly
    row_load<POOL>(a, r, a.scores + (int64_t)r * a.row_stride, 0, A);   // during the threshold search
    row_load<POOL>(a, r, a.scores + (int64_t)r * a.row_stride, kRowRound, B);
    const RowThreshold th = hist_threshold<kRowThreads>(hv, a.k, sh.wsum, sh.pair);
    if (th.n_cand <= kRowCap)
      nsel = row_select<POOL>(a, r, nv, n_row, th, A, B, sh.cbuf, kRowCap, sh, oi, os, sort);
    else if (a.cand)
      nsel = row_select<POOL>(a, r, nv, n_row, th, A, B, a.cand + (int64_t)r * a.n_chunks * kFiltChunk,
                        a.n_chunks * kFiltChunk, sh, oi, os, sort);
    else
      nsel = row_select_stream(a, r, nv, n_row, th, sh, oi, os, sort);
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
  if (a.im.n_items <= kRegThreads * kRegRowNK && a.im.mode != kItemsCand) {
    static const hipError_t rattr = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_reg_row_kernel),
                                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                                        (int)sizeof(RegRowShared));
    if (rattr != hipSuccess) return rattr;
    hipLaunchKernelGGL(topk_reg_row_kernel, dim3((unsigned)a.n_rows), dim3(kRegThreads), sizeof(RegRowShared),
                       stream, a);
    return hipGetLastError();
  }
  static const hipError_t attr_p = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_row_kernel<true>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)sizeof(RowShared));
  static const hipError_t attr_o = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_row_kernel<false>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)sizeof(RowShared));
  if (attr_p != hipSuccess) return attr_p;
  if (attr_o != hipSuccess) return attr_o;
  if (a.im.mode == kItemsPool)
    hipLaunchKernelGGL(topk_row_kernel<true>, dim3((unsigned)a.n_rows), dim3(kRowThreads), sizeof(RowShared), stream, a);
  else
    hipLaunchKernelGGL(topk_row_kernel<false>, dim3((unsigned)a.n_rows), dim3(kRowThreads), sizeof(RowShared), stream, a);
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
