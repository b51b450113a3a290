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
//   select: one workgroup per row.  The row histogram gives the bin that
//           holds the k-th largest score; one pass over the row's scores
//           keeps everything above it and gathers that bin's members into
//           LDS; an MSB-first radix select on (score, ~position) settles the
//           boundary exactly (ties -> lower position); a bitonic sort puts
//           the kept positions in ascending order.
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
constexpr int kTilesPerIter = 4;   // 16-item tiles in flight per wave

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

template <int MODE>
__global__ __launch_bounds__(kScoreThreads) void index_score_kernel(ScoreArgs a) {
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
  float* srow = a.scores + (int64_t)r * a.im.n_items;
  __syncthreads();

  const int64_t ntiles = (c1 - c0 + 15) / 16;
  for (int64_t t0 = (int64_t)wave * kTilesPerIter; t0 < ntiles;
       t0 += (int64_t)kScoreWaves * kTilesPerIter) {
    v8i kb[kTilesPerIter];
    int64_t pos[kTilesPerIter];
#pragma unroll
    for (int u = 0; u < kTilesPerIter; ++u) {
      const int64_t item = c0 + (t0 + u) * 16 + n;
      pos[u] = (item < c1) ? item_pos(a.im, r, item, nv) : -1;
      if (pos[u] >= 0) {
        kb[u] = load32(kbase + pos[u] * kIdxDim);
      } else {
        kb[u] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < kTilesPerIter; ++u) {
      // D[h][entry] = sum_k q[h][k] * key[entry][k]; lane: entry n, heads 4g+i
      v4f d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const v8h kh = fp8x8_to_f16(kb[u][2 * v], kb[u][2 * v + 1]);
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa0[v], kh, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa1[v], kh, d1, 0, 0, 0);
      }
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s = fmaf(w0[i], fmaxf(d0[i], 0.0f), s);
        s = fmaf(w1[i], fmaxf(d1[i], 0.0f), s);
      }
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      const int64_t item = c0 + (t0 + u) * 16 + n;
      if (g == 0 && item < c1) {
        if (pos[u] >= 0) {
          srow[item] = s;
          atomicAdd(&hist[order_key(s) >> (32 - kHistBits)], 1u);
        } else {
          srow[item] = __uint_as_float(0x7FC00000u);   // not visible
        }
      }
    }
  }
  __syncthreads();
  uint32_t* ghist = a.hist + (int64_t)r * kHistBins;
  for (int b = threadIdx.x; b < kHistBins; b += kScoreThreads) {
    const uint32_t c = hist[b];
    if (c) atomicAdd(&ghist[b], c);
  }
}

hipError_t launch_index_score(const ScoreArgs& a, hipStream_t stream) {
  if (a.n_rows == 0 || a.im.n_items == 0) return hipSuccess;
  const int64_t chunks = ((int64_t)a.im.n_items + a.chunk - 1) / a.chunk;
  const dim3 grid((unsigned)chunks, (unsigned)a.n_rows), block(kScoreThreads);
  switch (a.im.mode) {
    case kItemsFlat: hipLaunchKernelGGL(index_score_kernel<kItemsFlat>, grid, block, 0, stream, a); break;
    case kItemsBlocks: hipLaunchKernelGGL(index_score_kernel<kItemsBlocks>, grid, block, 0, stream, a); break;
    case kItemsPool: hipLaunchKernelGGL(index_score_kernel<kItemsPool>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(index_score_kernel<kItemsCand>, grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// select kernel
// ---------------------------------------------------------------------------

constexpr int kSelThreads = 1024;
constexpr int kCandCap = 12288;

struct SelShared {
  uint32_t hist[kHistBins];
  uint32_t scan[kSelThreads];
  uint32_t cand_key[kCandCap];
  int32_t cand_pos[kCandCap];
  int32_t sel_pos[kMaxTopK];
  float sel_score[kMaxTopK];
  int32_t n_cand, n_sel, overflow, bstar, c_above, digit, dcount;
};

// Composite order key: score order first, then lower position first.
__device__ __forceinline__ uint64_t comp_key(uint32_t okey, int64_t pos) {
  return ((uint64_t)okey << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
}

__device__ __forceinline__ void sel_append(SelShared& sh, int kk, int32_t pos, float s) {
  const int slot = atomicAdd(&sh.n_sel, 1);
  if (slot < kk) {
    sh.sel_pos[slot] = pos;
    sh.sel_score[slot] = s;
  }
}

// Visit every candidate of the boundary bin with f(composite key, pos, score).
template <class F>
__device__ __forceinline__ void for_each_cand(SelShared& sh, const SelectArgs& a, int r,
                                              int64_t nv, int64_t n_row, const float* srow,
                                              bool from_lds, F f) {
  if (from_lds) {
    for (int j = threadIdx.x; j < sh.n_cand; j += kSelThreads) {
      const uint32_t ok = sh.cand_key[j];
      const int32_t p = sh.cand_pos[j];
      f(comp_key(ok, p), p, order_key_inv(ok));
    }
  } else {
    const uint32_t bstar = (uint32_t)sh.bstar;
    for (int64_t i = threadIdx.x; i < n_row; i += kSelThreads) {
      const float s = srow[i];
      if (s != s) continue;
      const uint32_t ok = order_key(s);
      if ((ok >> (32 - kHistBits)) != bstar) continue;
      const int64_t p = item_pos(a.im, r, i, nv);
      f(comp_key(ok, p), (int32_t)p, order_key_inv(ok));
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelectArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SelShared& sh = *reinterpret_cast<SelShared*>(smem_raw);
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nv = row_valid(a.im, r);
  const int64_t n_row = row_items(a.im, nv);
  const float* srow = a.scores + (int64_t)r * a.im.n_items;
  const uint32_t* ghist = a.hist + (int64_t)r * kHistBins;

  // 1. threshold bin: suffix sums over the row histogram (4 bins per thread)
  uint32_t loc = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t c = ghist[4 * tid + i];
    sh.hist[4 * tid + i] = c;
    loc += c;
  }
  sh.scan[tid] = loc;
  if (tid == 0) { sh.n_cand = 0; sh.n_sel = 0; sh.overflow = 0; sh.bstar = -1; sh.c_above = 0; }
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {      // inclusive suffix scan
    const uint32_t v = (tid + off < kSelThreads) ? sh.scan[tid + off] : 0u;
    __syncthreads();
    sh.scan[tid] += v;
    __syncthreads();
  }
  const uint32_t total = sh.scan[0];
  const int kk = (int)min((uint32_t)a.k, total);
  if (kk < (int)total) {
    const uint32_t above = (tid + 1 < kSelThreads) ? sh.scan[tid + 1] : 0u;
    if (above < (uint32_t)kk && sh.scan[tid] >= (uint32_t)kk) {
      uint32_t cum = above;
      for (int b = 4 * tid + 3; b >= 4 * tid; --b) {
        if (cum + sh.hist[b] >= (uint32_t)kk) { sh.bstar = b; sh.c_above = (int)cum; break; }
        cum += sh.hist[b];
      }
    }
  }
  __syncthreads();
  const int bstar = sh.bstar;

  // 2. one pass: keep everything above the bin, gather the bin's members
  for (int64_t i = tid; i < n_row; i += kSelThreads) {
    const float s = srow[i];
    if (s != s) continue;
    const uint32_t ok = order_key(s);
    const int bin = (int)(ok >> (32 - kHistBits));
    if (bin > bstar) {
      sel_append(sh, kk, (int32_t)item_pos(a.im, r, i, nv), s);
    } else if (bin == bstar) {
      const int slot = atomicAdd(&sh.n_cand, 1);
      if (slot < kCandCap) {
        sh.cand_key[slot] = ok;
        sh.cand_pos[slot] = (int32_t)item_pos(a.im, r, i, nv);
      } else {
        sh.overflow = 1;
      }
    }
  }
  __syncthreads();

  // 3. exact boundary: MSB-first radix select over (score, ~position)
  if (bstar >= 0) {
    const bool from_lds = sh.overflow == 0;
    int need = kk - sh.c_above;
    uint64_t prefix = (uint64_t)bstar >> 4;        // bits 63..56 shared by the bin
    bool done = false;
    for (int shift = 48; shift >= 0 && !done; shift -= 8) {
      for (int b = tid; b < 256; b += kSelThreads) sh.hist[b] = 0u;
      __syncthreads();
      for_each_cand(sh, a, r, nv, n_row, srow, from_lds, [&](uint64_t K, int32_t, float) {
        if ((K >> (shift + 8)) == prefix) atomicAdd(&sh.hist[(K >> shift) & 255u], 1u);
      });
      __syncthreads();
      if (tid == 0) {
        int cum = 0, d = 255;
        for (; d > 0; --d) {
          if (cum + (int)sh.hist[d] >= need) break;
          cum += (int)sh.hist[d];
        }
        sh.digit = d;
        sh.c_above = cum;
        sh.dcount = (int)sh.hist[d];
      }
      __syncthreads();
      const uint64_t D = (uint64_t)sh.digit;
      for_each_cand(sh, a, r, nv, n_row, srow, from_lds, [&](uint64_t K, int32_t p, float s) {
        if ((K >> (shift + 8)) == prefix && ((K >> shift) & 255u) > D) sel_append(sh, kk, p, s);
      });
      need -= sh.c_above;
      prefix = (prefix << 8) | D;
      if (sh.dcount == need || shift == 0) {
        for_each_cand(sh, a, r, nv, n_row, srow, from_lds, [&](uint64_t K, int32_t p, float s) {
          if ((K >> shift) == prefix) sel_append(sh, kk, p, s);
        });
        done = true;
      }
      __syncthreads();
    }
  }
  __syncthreads();

  // 4. ascending positions: bitonic sort of the kept (pos, score) pairs
  const int nsel = min(sh.n_sel, kk);
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
            const float t = sh.sel_score[i]; sh.sel_score[i] = sh.sel_score[j]; sh.sel_score[j] = t;
          }
        }
      }
      __syncthreads();
    }
  }

  // 5. write out, -1 padded
  int32_t* oi = a.out_idx + (int64_t)r * a.k;
  for (int j = tid; j < a.k; j += kSelThreads) {
    oi[j] = j < nsel ? sh.sel_pos[j] : -1;
    if (a.out_score) a.out_score[(int64_t)r * a.k + j] = j < nsel ? sh.sel_score[j] : 0.0f;
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
