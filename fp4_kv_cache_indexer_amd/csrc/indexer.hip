// Sparse indexer + exact top-k [0539edu §3: csa2.indexer (32 heads x 128,
// top_k 512) and its hierarchical block (2048 blocks x 8 positions)].
//
//   score:  I_t = sum_h w_h * max(0, q_h . k_t), q/k FP8 E4M3, float32
//           accumulation.  The 128-byte keys stream straight from HBM into
//           registers, are widened to fp16 there (exact: every E4M3 value is
//           an fp16 value) and meet the queries in v_mfma_f32_16x16x32_f16,
//           [32 heads x 128] x [128 x 16 entries] per 8 MFMAs; the head
//           reduction runs in the epilogue.  (gfx950's fp8 MFMAs were measured
//           to sum their products with less than float32 precision -- up to
//           ~1e-3 relative on heavy-tailed data -- which is as wide as the
//           top-k tie band; the fp16 MFMA matches a float32 FMA chain.)  Each
//           workgroup also histograms the top 12 bits of the order key of its
//           scores in LDS and folds that into a per-row histogram.
//   filter: many workgroups per row.  Each reads the row histogram, finds
//           the bin holding the k-th largest score and compacts the items of
//           its chunk in that bin or above, in item order, as composite keys
//           (order key of the score, ~position).
//   select: one workgroup per row over those candidates (a few thousand):
//           an MSB-first radix select finds the k-th largest composite key
//           exactly (ties -> lower position), and the kept candidates are
//           written in candidate order, which is ascending position.
#include "csa2_dev.h"
#include "csa2_launch.h"

namespace csa2 {

// ---------------------------------------------------------------------------
// item <-> position mapping
// ---------------------------------------------------------------------------

__device__ __forceinline__ int64_t row_seq_of(const ItemMap& im, int r) {
  return im.row_seq ? (int64_t)im.row_seq[r] : (int64_t)r;
}

// Entries visible to row r: n_valid clamped to [0, n_ent]; none if the row's
// sequence is not in the cache.
__device__ __forceinline__ int64_t row_valid(const ItemMap& im, int r) {
  const int64_t seq = row_seq_of(im, r);
  if (seq < 0 || seq >= im.n_seq) return 0;
  const int64_t nv = im.n_valid ? (int64_t)im.n_valid[r] : im.n_ent;
  return nv < 0 ? 0 : (nv > im.n_ent ? im.n_ent : nv);
}

__device__ __forceinline__ int64_t row_items(const ItemMap& im, int64_t nv) {
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

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = min((n + 255) / 256, (size_t)4096);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// score kernel
// ---------------------------------------------------------------------------

constexpr int kScoreThreads = 256;
constexpr int kScoreWaves = kScoreThreads / 64;
constexpr int kTilesPerIter = 4;   // 16-item tiles per group
// Chosen by measurement on the 8 x 131072-block coarse scan: double-buffered
// groups of 4 tiles, register budget for 2 waves per SIMD (28.7 us vs
// 29.8-37 us for the single-buffered, larger-group and tighter-budget forms).
constexpr bool kScoreDB = true;
constexpr int kScoreMinW = 2;

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  v8i v;
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  return v;
}

// 8 E4M3 bytes (two words, byte order = element order) widened to fp16.
__device__ __forceinline__ v8h fp8x8_to_f16(int w0, int w1) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w0, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w0, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w1, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w1, 1.0f, true);
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// DB: double-buffer the tile groups of a wave; MINW: waves per SIMD the
// register budget must allow.
template <int MODE, bool DB = false, int MINW = 4, int U = kTilesPerIter>
__global__ __launch_bounds__(kScoreThreads, MINW) void index_score_kernel(ScoreArgs a) {
  a.im.mode = MODE;                              // lets the item mapping fold away
  __shared__ uint32_t hist[kHistBins];
  const int r = blockIdx.y;
  const int64_t nv = row_valid(a.im, r);
  const int64_t n_row = row_items(a.im, nv);
  const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
  if (c0 >= n_row) return;                       // uniform for the workgroup
  const int64_t c1 = min(c0 + (int64_t)a.chunk, n_row);

  for (int b = threadIdx.x; b < kHistBins; b += kScoreThreads) hist[b] = 0u;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t seq = row_seq_of(a.im, r);
  const uint8_t* kbase = a.keys + seq * a.seq_rows * kIdxDim + g * 32;

  // MFMA A operands: indexer query rows n and 16+n, bytes [32g, 32g+32), as
  // four fp16 k-slices of 8.  The B operand (keys) uses the same byte split,
  // so each lane's query bytes meet the same key bytes and the four MFMAs
  // together form the full 128-term dot product.
  const uint8_t* qr = a.q + (int64_t)r * kIdxHeads * kIdxDim + g * 32;
  v8h qa0[4], qa1[4];
  {
    const v8i q0 = load32(qr + n * kIdxDim);
    const v8i q1 = load32(qr + (16 + n) * kIdxDim);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      qa0[u] = fp8x8_to_f16(q0[2 * u], q0[2 * u + 1]);
      qa1[u] = fp8x8_to_f16(q1[2 * u], q1[2 * u + 1]);
    }
  }
  float w0[4], w1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w0[i] = a.w ? a.w[r * kIdxHeads + 4 * g + i] : 1.0f;
    w1[i] = a.w ? a.w[r * kIdxHeads + 16 + 4 * g + i] : 1.0f;
  }
  float* srow = a.scores + (int64_t)r * a.row_stride;
  __syncthreads();

  // A wave works on groups of U tiles of 16 items (U a multiple of 4).
  // Loads are unconditional (an invisible item reads a visible row and its
  // score is masked when written).
  const int64_t ntiles = (c1 - c0 + 15) / 16;
  const int64_t gstride = (int64_t)kScoreWaves * U;
  const int32_t p0 = (int32_t)item_pos(a.im, r, c0, nv);
  const int32_t safe_pos = p0 >= 0 ? p0 : 0;
  auto load_group = [&](int64_t t0, v8i* kb, int32_t* pos) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t item = c0 + (t0 + u) * 16 + n;
      pos[u] = (item < c1) ? (int32_t)item_pos(a.im, r, item, nv) : -1;
      kb[u] = load32(kbase + (int64_t)(pos[u] >= 0 ? pos[u] : safe_pos) * kIdxDim);
    }
  };
  auto compute_group = [&](int64_t t0, const v8i* kb) {
#pragma unroll
    for (int u4 = 0; u4 < U; u4 += 4) {
      float p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // D[h][entry] = sum_k q[h][k] * key[entry][k]; lane: entry n, heads 4g+i
        v4f d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const v8h kh = fp8x8_to_f16(kb[u4 + u][2 * v], kb[u4 + u][2 * v + 1]);
          d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa0[v], kh, d0, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa1[v], kh, d1, 0, 0, 0);
        }
        float sp = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sp = fmaf(w0[i], fmaxf(d0[i], 0.0f), sp);
          sp = fmaf(w1[i], fmaxf(d1[i], 0.0f), sp);
        }
        p[u] = sp;
      }
      // transpose-reduce: lane (n, g) ends with the full score of tile
      // u4 + g, entry n (sum over the four head groups) after three lane
      // exchanges
      const bool b0 = g & 1, b1 = (g >> 1) & 1;
      float keep0 = b0 ? p[1] : p[0], send0 = b0 ? p[0] : p[1];
      float keep1 = b0 ? p[3] : p[2], send1 = b0 ? p[2] : p[3];
      keep0 += __shfl_xor(send0, 16);
      keep1 += __shfl_xor(send1, 16);
      float sc = b1 ? keep1 : keep0;
      sc += __shfl_xor(b1 ? keep0 : keep1, 32);
      const int64_t item = c0 + (t0 + u4 + g) * 16 + n;
      if (item < c1) {
        if (item_pos(a.im, r, item, nv) >= 0) {
          srow[item] = sc;
          atomicAdd(&hist[order_key(sc) >> (32 - kHistBits)], 1u);
        } else {
          srow[item] = __uint_as_float(0x7FC00000u);   // not visible
        }
      }
    }
  };
  v8i kA[U], kB[U];
  int32_t pA[U], pB[U];
  int64_t t0 = (int64_t)wave * U;
  if (DB) {
    if (t0 < ntiles) load_group(t0, kA, pA);
    for (; t0 < ntiles; t0 += 2 * gstride) {
      const int64_t t1 = t0 + gstride;
      if (t1 < ntiles) load_group(t1, kB, pB);
      compute_group(t0, kA);
      if (t1 >= ntiles) break;
      const int64_t t2 = t1 + gstride;
      if (t2 < ntiles) load_group(t2, kA, pA);
      compute_group(t1, kB);
    }
  } else {
    for (; t0 < ntiles; t0 += gstride) {
      load_group(t0, kA, pA);
      compute_group(t0, kA);
    }
  }
  __syncthreads();
  uint32_t* ghist = a.hist + (int64_t)r * kHistBins;
  for (int b = threadIdx.x; b < kHistBins; b += kScoreThreads) {
    const uint32_t c = hist[b];
    if (c) atomicAdd(&ghist[b], c);
  }
}

// Workgroups of one score kernel that fit on the device at once.
int score_resident_wgs() {
  static int cached = 0;
  if (cached) return cached;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, index_score_kernel<kItemsBlocks, kScoreDB, kScoreMinW>,
                                                   kScoreThreads, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();
    return 1024;
  }
  cached = cus * per_cu;
  return cached;
}

hipError_t launch_index_score(const ScoreArgs& a, hipStream_t stream) {
  if (a.n_rows == 0 || a.im.n_items == 0) return hipSuccess;
  const int64_t chunks = ((int64_t)a.im.n_items + a.chunk - 1) / a.chunk;
  const dim3 grid((unsigned)chunks, (unsigned)a.n_rows), block(kScoreThreads);
  switch (a.im.mode) {
    case kItemsFlat: hipLaunchKernelGGL((index_score_kernel<kItemsFlat, kScoreDB, kScoreMinW>), grid, block, 0, stream, a); break;
    case kItemsBlocks: hipLaunchKernelGGL((index_score_kernel<kItemsBlocks, kScoreDB, kScoreMinW>), grid, block, 0, stream, a); break;
    case kItemsPool: hipLaunchKernelGGL((index_score_kernel<kItemsPool, kScoreDB, kScoreMinW>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((index_score_kernel<kItemsCand, kScoreDB, kScoreMinW>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// top-k: filter (many workgroups per row) + select (one workgroup per row)
// ---------------------------------------------------------------------------

constexpr int kFiltThreads = 256;
constexpr int kFiltRound = kFiltThreads * 4;           // items per compaction round
constexpr int kSelThreads = 1024;
constexpr int kSelCap = 12288;                         // candidates held in LDS
constexpr int kMaxChunks = kMaxItems / kFiltChunk;

// Composite order key: score order first, then lower position first.
__device__ __forceinline__ uint64_t comp_key(uint32_t okey, int64_t pos) {
  return ((uint64_t)okey << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
}
__device__ __forceinline__ int32_t comp_pos(uint64_t K) { return (int32_t)(0xFFFFFFFFu - (uint32_t)K); }
__device__ __forceinline__ float comp_score(uint64_t K) { return order_key_inv((uint32_t)(K >> 32)); }

// Exclusive prefix sum over a workgroup of NT threads (wave64); `total`
// receives the sum.  Uses wsum[NT/64] of shared scratch; ends synchronised.
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
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = wsum[w];
    off += (w < wave) ? t : 0;
    tot += t;
  }
  total = tot;
  __syncthreads();
  return off + x - v;
}

// Filter: workgroup (chunk c, row r) finds the histogram bin holding the
// row's k-th largest score, then writes every item of its chunk in that bin
// or above -- a superset of the chunk's share of the top-k -- as composite
// keys, compacted in item order, plus their count.
__global__ __launch_bounds__(kFiltThreads) void topk_filter_kernel(SelectArgs a) {
  __shared__ uint32_t sc[kFiltThreads];
  __shared__ int wsum[kFiltThreads / 64];
  (void)sc;
  __shared__ int s_bstar;
  const int r = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int64_t nv = row_valid(a.im, r);
  const int64_t n_row = row_items(a.im, nv);
  const int64_t c0 = (int64_t)c * kFiltChunk;
  if (c0 >= n_row) return;                                   // uniform
  const int64_t c1 = min(c0 + (int64_t)kFiltChunk, n_row);

  // this thread's items, 4 consecutive per round, loaded before the scan
  const float* srow = a.scores + (int64_t)r * a.row_stride;
  constexpr int kRounds = kFiltChunk / kFiltRound;
  float v[kRounds][4];
#pragma unroll
  for (int rd = 0; rd < kRounds; ++rd) {
    const int64_t i0 = c0 + (int64_t)rd * kFiltRound + 4 * tid;
    if (i0 + 3 < c1) {
      const float4 q = *reinterpret_cast<const float4*>(srow + i0);   // rows are 16-byte aligned
      v[rd][0] = q.x; v[rd][1] = q.y; v[rd][2] = q.z; v[rd][3] = q.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[rd][j] = (i0 + j < c1) ? srow[i0 + j] : __uint_as_float(0x7FC00000u);
    }
  }

  // threshold bin from the row histogram (16 bins per thread)
  const uint32_t* gh = a.hist + (int64_t)r * kHistBins;
  uint32_t hv[kHistBins / kFiltThreads];
  uint32_t loc = 0;
#pragma unroll
  for (int i = 0; i < kHistBins / kFiltThreads; ++i) {
    hv[i] = gh[(kHistBins / kFiltThreads) * tid + i];
    loc += hv[i];
  }
  // suffix sums: scan the reversed thread order
  int tot_i;
  const int rev_ex = block_excl_scan<kFiltThreads>((int)loc, wsum, tot_i);   // sum over threads < tid
  (void)rev_ex;
  sc[tid] = loc;
  if (tid == 0) s_bstar = -1;
  __syncthreads();
  const uint32_t total = (uint32_t)tot_i;
  const uint32_t kk = min((uint32_t)a.k, total);
  if (kk < total) {
    // items in bins above this thread's 16 = total - (threads <= tid)
    const uint32_t above = total - (uint32_t)rev_ex - loc;
    if (above < kk && above + loc >= kk) {
      uint32_t cum = above;
      for (int b = kHistBins / kFiltThreads - 1; b >= 0; --b) {
        if (cum + hv[b] >= kk) { s_bstar = (kHistBins / kFiltThreads) * tid + b; break; }
        cum += hv[b];
      }
    }
  }
  __syncthreads();
  const int bstar = s_bstar;

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
      const bool keep = (v[rd][j] == v[rd][j]) && (int)(ok[j] >> (32 - kHistBits)) >= bstar;
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

hipError_t launch_topk_filter(const SelectArgs& a, hipStream_t stream) {
  if (a.n_rows == 0 || a.n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)a.n_chunks, (unsigned)a.n_rows),
                     dim3(kFiltThreads), 0, stream, a);
  return hipGetLastError();
}

struct SelShared {
  uint64_t key[kSelCap];
  int32_t sel_pos[kMaxTopK];     // candidate mode: kept ids before sorting
  float sel_score[kMaxTopK];
  uint32_t chunk_off[kMaxChunks + 1];
  uint32_t hist[256];
  uint32_t suf[257];
  int wsum[kSelThreads / 64];
  int digit, above, dcount;
};

// Select: exact top-k of the row's candidates (MSB-first radix on the
// composite keys), written in candidate order, which is ascending position.
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelectArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SelShared& sh = *reinterpret_cast<SelShared*>(smem_raw);
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t nv = row_valid(a.im, r);
  const int64_t n_row = row_items(a.im, nv);
  const int nch = (int)((n_row + kFiltChunk - 1) / kFiltChunk);
  const uint32_t* cnt = a.cand_count + (int64_t)r * a.n_chunks;
  const uint64_t* crow = a.cand + (int64_t)r * a.n_chunks * kFiltChunk;
  int32_t* oi = a.out_idx + (int64_t)r * a.k;
  float* os = a.out_score ? a.out_score + (int64_t)r * a.k : nullptr;

  // row histogram: valid items, the bin b* holding the k-th largest score and
  // the count of items above it (4 bins per thread)
  const uint32_t* gh = a.hist + (int64_t)r * kHistBins;
  uint32_t hv[kHistBins / kSelThreads];
  uint32_t loc = 0;
#pragma unroll
  for (int i = 0; i < kHistBins / kSelThreads; ++i) {
    hv[i] = gh[(kHistBins / kSelThreads) * tid + i];
    loc += hv[i];
  }
  int tot_valid;
  const int below = block_excl_scan<kSelThreads>((int)loc, sh.wsum, tot_valid);
  const int kk = min(a.k, tot_valid);
  if (tid == 0) { sh.digit = -1; sh.above = 0; }
  __syncthreads();
  if (kk < tot_valid) {
    const uint32_t above = (uint32_t)(tot_valid - below) - loc;
    if (above < (uint32_t)kk && above + loc >= (uint32_t)kk) {
      uint32_t cum = above;
      for (int b = kHistBins / kSelThreads - 1; b >= 0; --b) {
        if (cum + hv[b] >= (uint32_t)kk) { sh.digit = (kHistBins / kSelThreads) * tid + b; sh.above = (int)cum; break; }
        cum += hv[b];
      }
    }
  }
  __syncthreads();
  const int bstar = sh.digit;
  const int c_above = sh.above;

  // chunk offsets of the filtered candidates
  int C = 0;
  {
    int running = 0;
    for (int base = 0; base < nch; base += kSelThreads) {
      const int i = base + tid;
      const int v = i < nch ? (int)cnt[i] : 0;
      int t;
      const int ex = block_excl_scan<kSelThreads>(v, sh.wsum, t);
      if (i < nch) sh.chunk_off[i] = (uint32_t)(running + ex);
      running += t;
    }
    C = running;
    if (tid == 0) sh.chunk_off[nch] = (uint32_t)C;
  }
  __syncthreads();
  const bool in_lds = C <= kSelCap;

  // candidate j -> composite key (binary search over the chunk offsets)
  auto gkey = [&](int j) -> uint64_t {
    int lo = 0, hi = nch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int)sh.chunk_off[mid] <= j) lo = mid; else hi = mid - 1;
    }
    return crow[(int64_t)lo * kFiltChunk + (j - (int)sh.chunk_off[lo])];
  };
  if (in_lds) {
    for (int j = tid; j < C; j += kSelThreads) sh.key[j] = gkey(j);
  }
  __syncthreads();
  auto key_at = [&](int j) -> uint64_t { return in_lds ? sh.key[j] : gkey(j); };

  // threshold T: the kk-th largest composite key (all kept keys are >= T).
  // Its top 12 bits are b*; the rest is found digit by digit among the
  // candidates of bin b*.
  uint64_t T = 0;
  if (bstar >= 0) {
    int need = kk - c_above;
    uint64_t prefix = (uint64_t)bstar;
    // remaining 52 bits: six 8-bit digits, then one 4-bit digit
    for (int step = 0; step < 7; ++step) {
      const int dshift = step < 6 ? 44 - 8 * step : 0;     // digit = bits [dshift, dshift + w)
      const int w = step < 6 ? 8 : 4;
      const uint32_t dmask = (1u << w) - 1u;
      for (int b = tid; b < 256; b += kSelThreads) sh.hist[b] = 0u;
      __syncthreads();
      for (int j = tid; j < C; j += kSelThreads) {
        const uint64_t K = key_at(j);
        if ((K >> (dshift + w)) == prefix) atomicAdd(&sh.hist[(K >> dshift) & dmask], 1u);
      }
      __syncthreads();
      if (tid < 64) {                                      // one wave finds the digit
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

  // write the kept keys in candidate order -- ascending position, except in
  // candidate mode, where the caller's list has any order and a sort follows
  const bool sort = a.im.mode == kItemsCand;
  int written = 0;
  for (int base = 0; base < C; base += kSelThreads) {
    const int j = base + tid;
    uint64_t K = 0;
    const bool keep = j < C && kk > 0 && (K = key_at(j)) >= T;
    int t;
    const int slot = written + block_excl_scan<kSelThreads>(keep ? 1 : 0, sh.wsum, t);
    if (keep && slot < a.k) {
      if (sort) {
        sh.sel_pos[slot] = comp_pos(K);
        sh.sel_score[slot] = comp_score(K);
      } else {
        oi[slot] = comp_pos(K);
        if (os) os[slot] = comp_score(K);
      }
    }
    written += t;
  }
  const int nsel = min(written, a.k);
  if (sort) {
    int n2 = 1;
    while (n2 < nsel) n2 <<= 1;
    for (int i = nsel + tid; i < n2; i += kSelThreads) { sh.sel_pos[i] = 0x7FFFFFFF; sh.sel_score[i] = 0.f; }
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < n2; i += kSelThreads) {
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
    for (int j = tid; j < nsel; j += kSelThreads) {
      oi[j] = sh.sel_pos[j];
      if (os) os[j] = sh.sel_score[j];
    }
  }
  for (int j = nsel + tid; j < a.k; j += kSelThreads) {
    oi[j] = -1;
    if (os) os[j] = 0.0f;
  }
}

hipError_t launch_topk_select(const SelectArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_select_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sizeof(SelShared));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)a.n_rows), dim3(kSelThreads),
                     sizeof(SelShared), stream, a);
  return hipGetLastError();
}

}  // namespace csa2
