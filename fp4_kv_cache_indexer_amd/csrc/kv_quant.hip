// Cache-write kernels: context-weighted pooling + FP4 E2M1 quantisation with
// per-16-channel E4M3 scales [0539edu §3; nxbn §4.2], and E4M3 block
// summaries of the index keys for the hierarchical indexer [0539edu §3].
//
// Both are HBM streaming kernels: one thread owns one 16-channel group (K1)
// or one 4-channel slice of a block (K2), so a wave reads contiguous runs of
// the token/key rows and writes contiguous code/summary runs.
#include "csa2_dev.h"
#include "csa2_launch.h"

namespace csa2 {

// E2M1 decision thresholds in units of the scale and whether a tie there
// rounds up (to the even code above): nearest-even on {0,.5,1,1.5,2,3,4,6}.
//   0.25 -> 0 (down), 0.75 -> 1.0 (up), 1.25 -> 1.0 (down), 1.75 -> 2 (up),
//   2.5 -> 2 (down), 3.5 -> 4 (up), 5 -> 4 (down).
__device__ __forceinline__ uint32_t e2m1_code(float y, float s) {
  const float a = fabsf(y);
  uint32_t mag = (a > 0.25f * s) + (a >= 0.75f * s) + (a > 1.25f * s) + (a >= 1.75f * s) +
                 (a > 2.5f * s) + (a >= 3.5f * s) + (a > 5.0f * s);
  if (s == 0.0f) mag = 0u;
  const uint32_t neg = (__float_as_uint(y) >> 31) & (mag != 0u);
  return mag | (neg << 3);
}

__device__ __forceinline__ void load_bf16x16(const uint16_t* p, float* v) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 8);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

// One thread = one (sequence, entry, 16-channel group).
template <int M, bool GATE>
__global__ __launch_bounds__(256) void kv_compress_quantize_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ z, int64_t n_seq, int64_t n_ent,
    int64_t x_seq_stride, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    int64_t out_seq_stride) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_seq * n_ent * 32) return;
  const int g = (int)(gid & 31);
  const int64_t ent = gid >> 5;
  const int64_t s = ent / n_ent, e = ent - s * n_ent;
  const int64_t tok0 = s * x_seq_stride + e * M;

  float y[16];
  if (M == 1) {
    load_bf16x16(x + tok0 * kD + g * 16, y);
  } else if (!GATE) {
    float acc[16], t[16];
    load_bf16x16(x + tok0 * kD + g * 16, acc);
#pragma unroll
    for (int j = 1; j < M; ++j) {
      load_bf16x16(x + (tok0 + j) * kD + g * 16, t);
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] += t[c];
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) y[c] = acc[c] * (1.0f / M);
  } else {
    float xv[M][16], zv[M][16];
#pragma unroll
    for (int j = 0; j < M; ++j) {
      load_bf16x16(x + (tok0 + j) * kD + g * 16, xv[j]);
      load_bf16x16(z + (tok0 + j) * kD + g * 16, zv[j]);
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      float mx = zv[0][c];
#pragma unroll
      for (int j = 1; j < M; ++j) mx = fmaxf(mx, zv[j][c]);
      float num = 0.0f, den = 0.0f;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const float w = expf(zv[j][c] - mx);
        num = fmaf(w, xv[j][c], num);
        den += w;
      }
      y[c] = __fdiv_rn(num, den);
    }
  }

  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fabsf(y[c]));
  const uint32_t sc = f32_to_e4m3(__fdiv_rn(amax, 6.0f));
  const float sv = e4m3_to_f32(sc);

  uint32_t lo = 0u, hi = 0u;
#pragma unroll
  for (int c = 0; c < 8; ++c) lo |= e2m1_code(y[c], sv) << (4 * c);
#pragma unroll
  for (int c = 0; c < 8; ++c) hi |= e2m1_code(y[8 + c], sv) << (4 * c);

  const int64_t oe = s * out_seq_stride + e;
  *reinterpret_cast<uint2*>(codes + oe * 256 + g * 8) = make_uint2(lo, hi);
  scales[oe * 32 + g] = (uint8_t)sc;
}

// One thread = one (sequence, block, 4 channels).
__global__ __launch_bounds__(256) void block_summary_kernel(const uint8_t* __restrict__ keys,
                                                            int64_t n_seq, int64_t n_ent,
                                                            int64_t blk_begin, int64_t n_blk_range,
                                                            uint8_t* __restrict__ summ) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_seq * n_blk_range * 32) return;
  const int c4 = (int)(gid & 31);
  const int64_t sb = gid >> 5;
  const int64_t s = sb / n_blk_range;
  const int64_t b = blk_begin + (sb - s * n_blk_range);
  const int64_t nb_total = (n_ent + kBlockPos - 1) / kBlockPos;
  const int64_t j0 = b * kBlockPos;
  const int cnt = (int)min((int64_t)kBlockPos, n_ent - j0);
  const uint8_t* base = keys + (s * n_ent + j0) * kIdxDim + c4 * 4;
  // all member loads at once (addresses clamped into the block), so the
  // block costs one memory latency rather than one per member
  uint32_t w[kBlockPos];
#pragma unroll
  for (int j = 0; j < kBlockPos; ++j)
    w[j] = *reinterpret_cast<const uint32_t*>(base + (int64_t)(j < cnt ? j : 0) * kIdxDim);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kBlockPos; ++j) {
    if (j < cnt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += e4m3_to_f32((w[j] >> (8 * i)) & 0xFFu);
    }
  }
  uint32_t out = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) out |= f32_to_e4m3(__fdiv_rn(acc[i], (float)cnt)) << (8 * i);
  *reinterpret_cast<uint32_t*>(summ + (s * nb_total + b) * kIdxDim + c4 * 4) = out;
}

// ---------------------------------------------------------------------------
// FP4 index keys: 128 E2M1 codes + one E4M3 scale per 32 channels (68 B per
// entry), quantised by the main-KV rule [daiw "four generations" table:
// 890 B/token = 2.5 entries x (288 + 68) B].
// ---------------------------------------------------------------------------

constexpr int kIdxFp4Group = 32;

// One thread = one (sequence, entry, 32-channel group) of bf16 keys.
__global__ __launch_bounds__(256) void index_key_quantize_kernel(
    const uint16_t* __restrict__ k, int64_t n_seq, int64_t n_ent, int64_t k_seq_stride,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t out_seq_stride) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_seq * n_ent * 4) return;
  const int g = (int)(gid & 3);
  const int64_t ent = gid >> 2;
  const int64_t s = ent / n_ent, e = ent - s * n_ent;
  const uint16_t* src = k + (s * k_seq_stride + e) * kIdxDim + g * kIdxFp4Group;
  float y[32];
  load_bf16x16(src, y);
  load_bf16x16(src + 16, y + 16);
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(y[c]));
  const uint32_t sc = f32_to_e4m3(__fdiv_rn(amax, 6.0f));
  const float sv = e4m3_to_f32(sc);
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q] = 0u;
#pragma unroll
    for (int c = 0; c < 8; ++c) w[q] |= e2m1_code(y[8 * q + c], sv) << (4 * c);
  }
  const int64_t oe = s * out_seq_stride + e;
  *reinterpret_cast<uint4*>(codes + oe * 64 + g * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[oe * 4 + g] = (uint8_t)sc;
}

// Block summaries of FP4 index keys: E4M3 of the float32 mean of the decoded
// members (their float32 partial sums are exact below 2^14; a block beyond
// that saturates E4M3).  One thread = one (sequence, block, 4 channels).
__global__ __launch_bounds__(256) void block_summary_fp4_kernel(const uint8_t* __restrict__ codes,
                                                                const uint8_t* __restrict__ scales,
                                                                int64_t n_seq, int64_t n_ent,
                                                                int64_t blk_begin, int64_t n_blk_range,
                                                                uint8_t* __restrict__ summ) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_seq * n_blk_range * 32) return;
  const int c4 = (int)(gid & 31);
  const int64_t sb = gid >> 5;
  const int64_t s = sb / n_blk_range;
  const int64_t b = blk_begin + (sb - s * n_blk_range);
  const int64_t nb_total = (n_ent + kBlockPos - 1) / kBlockPos;
  const int64_t j0 = b * kBlockPos;
  const int cnt = (int)min((int64_t)kBlockPos, n_ent - j0);
  // channels 4*c4 .. 4*c4+3: two code bytes and the scale of group c4 / 8
  const uint8_t* cb = codes + (s * n_ent + j0) * 64 + c4 * 2;
  const uint8_t* sb8 = scales + (s * n_ent + j0) * 4 + c4 / 8;
  uint32_t cw[kBlockPos], sw[kBlockPos];
#pragma unroll
  for (int j = 0; j < kBlockPos; ++j) {           // all member loads at once
    const int jj = j < cnt ? j : 0;
    cw[j] = *reinterpret_cast<const uint16_t*>(cb + (int64_t)jj * 64);
    sw[j] = sb8[(int64_t)jj * 4];
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kBlockPos; ++j) {
    if (j < cnt) {
      const float sv = e4m3_to_f32(sw[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += e2m1_to_f32((cw[j] >> (4 * i)) & 0xFu) * sv;
    }
  }
  uint32_t out = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) out |= f32_to_e4m3(__fdiv_rn(acc[i], (float)cnt)) << (8 * i);
  *reinterpret_cast<uint32_t*>(summ + (s * nb_total + b) * kIdxDim + c4 * 4) = out;
}

hipError_t launch_index_key_quantize(const void* k, int64_t n_seq, int64_t n_ent, int64_t k_seq_stride,
                                     uint8_t* codes, uint8_t* scales, int64_t out_seq_stride,
                                     hipStream_t stream) {
  const int64_t threads = n_seq * n_ent * 4;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(index_key_quantize_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(k), n_seq, n_ent, k_seq_stride, codes, scales,
                     out_seq_stride);
  return hipGetLastError();
}

hipError_t launch_block_summary_fp4(const uint8_t* codes, const uint8_t* scales, int64_t n_seq,
                                    int64_t n_ent, int64_t blk_begin, int64_t blk_end, uint8_t* summ,
                                    hipStream_t stream) {
  const int64_t nr = blk_end - blk_begin;
  const int64_t threads = n_seq * nr * 32;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(block_summary_fp4_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, codes, scales, n_seq, n_ent, blk_begin, nr, summ);
  return hipGetLastError();
}

hipError_t launch_kv_compress_quantize(const void* x, const void* z, int64_t n_seq, int64_t n_ent,
                                       int32_t m, int64_t x_seq_stride, uint8_t* codes,
                                       uint8_t* scales, int64_t out_seq_stride,
                                       hipStream_t stream) {
  const int64_t threads = n_seq * n_ent * 32;
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* zp = static_cast<const uint16_t*>(z);
#define CSA2_KQ(MM, GG)                                                                       \
  hipLaunchKernelGGL((kv_compress_quantize_kernel<MM, GG>), grid, block, 0, stream, xp, zp,   \
                     n_seq, n_ent, x_seq_stride, codes, scales, out_seq_stride)
  if (m == 1) CSA2_KQ(1, false);
  else if (m == 2 && z) CSA2_KQ(2, true);
  else if (m == 2) CSA2_KQ(2, false);
  else if (m == 4 && z) CSA2_KQ(4, true);
  else CSA2_KQ(4, false);
#undef CSA2_KQ
  return hipGetLastError();
}

hipError_t launch_block_summary(const uint8_t* keys, int64_t n_seq, int64_t n_ent,
                                int64_t blk_begin, int64_t blk_end, uint8_t* summ,
                                hipStream_t stream) {
  const int64_t nr = blk_end - blk_begin;
  const int64_t threads = n_seq * nr * 32;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(block_summary_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, keys, n_seq, n_ent, blk_begin, nr, summ);
  return hipGetLastError();
}

}  // namespace csa2
