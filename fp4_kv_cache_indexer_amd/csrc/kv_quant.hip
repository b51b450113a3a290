// Cache-write kernels: context-weighted pooling + FP4 E2M1 quantisation with
// per-16-channel E4M3 scales [0539edu §3; nxbn §4.2], and E4M3 block
// summaries of the index keys for the hierarchical indexer [0539edu §3].
//
// Both are HBM streaming kernels: one thread owns one 16-channel group (K1)
// or one 4-channel slice of a block (K2), so a wave reads contiguous runs of
// the token/key rows and writes contiguous code/summary runs.
#include "append_dev.h"
#include "attn_dev.h"
#include "csa2_dev.h"
#include "csa2_launch.h"

namespace csa2 {

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
  const uint16_t* xs[M];
  const uint16_t* zs[M];
#pragma unroll
  for (int j = 0; j < M; ++j) {
    xs[j] = x + (tok0 + j) * kD + g * 16;
    zs[j] = GATE ? z + (tok0 + j) * kD + g * 16 : nullptr;
  }
  uint32_t lo, hi;
  const uint32_t sc = pool_quantize16<M, GATE>(xs, zs, lo, hi);
  const int64_t oe = s * out_seq_stride + e;
  // non-temporal: the codes of a whole cache are streamed out once (a wave
  // writes two entries' 512 contiguous bytes) and read back much later
  typedef unsigned u2x __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(u2x{lo, hi}, reinterpret_cast<u2x*>(codes + oe * 256 + g * 8));
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

// One thread = one (sequence, block, 16 channels), for 16-byte aligned keys
// and summaries: each member is one 16-byte load (a wave's load covers 8
// whole key rows) decoded with the hardware E4M3 conversion (exact).  The
// members' sum is exact in float32 (multiples of 2^-9 below 2^12), so a full
// block's mean is that sum times 1/8 -- the same value the division gives --
// and the result equals block_summary_kernel's bit for bit.
__global__ __launch_bounds__(256) void block_summary16_kernel(const uint8_t* __restrict__ keys,
                                                              int64_t n_seq, int64_t n_ent,
                                                              int64_t blk_begin, int64_t n_blk_range,
                                                              uint8_t* __restrict__ summ) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_seq * n_blk_range * 8) return;
  const int c16 = (int)(gid & 7);
  const int64_t sb = gid >> 3;
  const int64_t s = sb / n_blk_range;
  const int64_t b = blk_begin + (sb - s * n_blk_range);
  const int64_t nb_total = (n_ent + kBlockPos - 1) / kBlockPos;
  const int64_t j0 = b * kBlockPos;
  const int cnt = (int)min((int64_t)kBlockPos, n_ent - j0);
  const uint8_t* base = keys + (s * n_ent + j0) * kIdxDim + c16 * 16;
  uint4 w[kBlockPos];
#pragma unroll
  for (int j = 0; j < kBlockPos; ++j)
    w[j] = *reinterpret_cast<const uint4*>(base + (int64_t)(j < cnt ? j : 0) * kIdxDim);
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < kBlockPos; ++j) {
    if (j < cnt) {
      const uint32_t ww[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)ww[q], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)ww[q], true);
        acc[4 * q] += lo[0];
        acc[4 * q + 1] += lo[1];
        acc[4 * q + 2] += hi[0];
        acc[4 * q + 3] += hi[1];
      }
    }
  }
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float m = cnt == kBlockPos ? acc[i] * (1.0f / kBlockPos) : __fdiv_rn(acc[i], (float)cnt);
    out[i >> 2] |= f32_to_e4m3(m) << (8 * (i & 3));
  }
  *reinterpret_cast<uint4*>(summ + (s * nb_total + b) * kIdxDim + c16 * 16) = make_uint4(out[0], out[1], out[2], out[3]);
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

// The same summaries with one thread per (sequence, block, 16 channels), for
// 8-byte aligned codes, 4-byte aligned scales and 16-byte aligned summaries:
// a member is one 8-byte code load and its 4-byte scale word, decoded by the
// hardware at unit scale (exact) and multiplied by the group scale (exact),
// so every member value, the order of the sums and the result are those of
// block_summary_fp4_kernel; a full block's mean is its sum times 1/8.
__global__ __launch_bounds__(256) void block_summary_fp4_16_kernel(const uint8_t* __restrict__ codes,
                                                                   const uint8_t* __restrict__ scales,
                                                                   int64_t n_seq, int64_t n_ent,
                                                                   int64_t blk_begin, int64_t n_blk_range,
                                                                   uint8_t* __restrict__ summ) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_seq * n_blk_range * 8) return;
  const int c16 = (int)(gid & 7);                 // channels 16*c16 .. 16*c16+15
  const int64_t sb = gid >> 3;
  const int64_t s = sb / n_blk_range;
  const int64_t b = blk_begin + (sb - s * n_blk_range);
  const int64_t nb_total = (n_ent + kBlockPos - 1) / kBlockPos;
  const int64_t j0 = b * kBlockPos;
  const int cnt = (int)min((int64_t)kBlockPos, n_ent - j0);
  const uint8_t* cb = codes + (s * n_ent + j0) * 64 + c16 * 8;
  const uint8_t* swp = scales + (s * n_ent + j0) * 4;
  uint2 cw[kBlockPos];
  uint32_t sw[kBlockPos];
#pragma unroll
  for (int j = 0; j < kBlockPos; ++j) {           // all member loads at once
    const int jj = j < cnt ? j : 0;
    cw[j] = *reinterpret_cast<const uint2*>(cb + (int64_t)jj * 64);
    sw[j] = *reinterpret_cast<const uint32_t*>(swp + (int64_t)jj * 4);
  }
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < kBlockPos; ++j) {
    if (j < cnt) {
      const float sv = e4m3_to_f32((sw[j] >> (8 * (c16 >> 1))) & 0xFFu);   // the 32-channel group
      float f[16];
      fp4x8_to_f32(cw[j].x, sv, f);
      fp4x8_to_f32(cw[j].y, sv, f + 8);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += f[i];
    }
  }
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float m = cnt == kBlockPos ? acc[i] * (1.0f / kBlockPos) : __fdiv_rn(acc[i], (float)cnt);
    out[i >> 2] |= f32_to_e4m3(m) << (8 * (i & 3));
  }
  *reinterpret_cast<uint4*>(summ + (s * nb_total + b) * kIdxDim + c16 * 16) = make_uint4(out[0], out[1], out[2], out[3]);
}

// ---------------------------------------------------------------------------
// Decode-time append (the row body is decode_append_row in append_dev.h,
// shared with the indexer's coarse scan, which can run it in extra
// workgroups of its own launch).
// ---------------------------------------------------------------------------

template <int M, bool GATE, int KF>
__global__ __launch_bounds__(128) void decode_append_kernel(AppendArgs a) {
  decode_append_row<M, GATE, KF>(a, blockIdx.x, threadIdx.x);
}

hipError_t launch_decode_append(const AppendArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_rows), block(128);
  const bool gate = a.gate != nullptr;
  const int kf = a.key_fp4 ? 1 : 0;
#define CSA2_AP(MM, GG, KK) hipLaunchKernelGGL((decode_append_kernel<MM, GG, KK>), grid, block, 0, stream, a)
#define CSA2_AP_K(MM, GG) do { if (kf) CSA2_AP(MM, GG, 1); else CSA2_AP(MM, GG, 0); } while (0)
  if (a.m == 1) CSA2_AP_K(1, false);
  else if (a.m == 2 && gate) CSA2_AP_K(2, true);
  else if (a.m == 2) CSA2_AP_K(2, false);
  else if (gate) CSA2_AP_K(4, true);
  else CSA2_AP_K(4, false);
#undef CSA2_AP_K
#undef CSA2_AP
  return hipGetLastError();
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
  if (reinterpret_cast<uintptr_t>(codes) % 8 == 0 && reinterpret_cast<uintptr_t>(scales) % 4 == 0 &&
      reinterpret_cast<uintptr_t>(summ) % 16 == 0) {
    hipLaunchKernelGGL(block_summary_fp4_16_kernel, dim3((unsigned)((threads / 4 + 255) / 256)), dim3(256), 0,
                       stream, codes, scales, n_seq, n_ent, blk_begin, nr, summ);
  } else {
    hipLaunchKernelGGL(block_summary_fp4_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, codes, scales, n_seq, n_ent, blk_begin, nr, summ);
  }
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
  if (n_seq * nr == 0) return hipSuccess;
  if (reinterpret_cast<uintptr_t>(keys) % 16 == 0 && reinterpret_cast<uintptr_t>(summ) % 16 == 0) {
    const int64_t threads = n_seq * nr * 8;
    hipLaunchKernelGGL(block_summary16_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, keys, n_seq, n_ent, blk_begin, nr, summ);
  } else {
    const int64_t threads = n_seq * nr * 32;
    hipLaunchKernelGGL(block_summary_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, keys, n_seq, n_ent, blk_begin, nr, summ);
  }
  return hipGetLastError();
}

}  // namespace csa2
