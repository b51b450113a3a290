// Cache-write kernels: context-weighted pooling + FP4 E2M1 quantisation with
// per-16-channel E4M3 scales [0539edu §3; nxbn §4.2], and E4M3 block
// summaries of the index keys for the hierarchical indexer [0539edu §3].
//
// Both are HBM streaming kernels: one thread owns one 16-channel group (K1)
// or one 4-channel slice of a block (K2), so a wave reads contiguous runs of
// the token/key rows and writes contiguous code/summary runs.
#include "attn_dev.h"
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

// Pool the m tokens of one group over 16 channels (xs[j], zs[j]: token j's
// channels) and quantise them: returns the E4M3 scale byte, the 16 E2M1
// codes in lo (channels 0-7) and hi (8-15).
template <int M, bool GATE>
__device__ __forceinline__ uint32_t pool_quantize16(const uint16_t* const* xs, const uint16_t* const* zs,
                                                   uint32_t& lo, uint32_t& hi) {
  float y[16];
  if (M == 1) {
    load_bf16x16(xs[0], y);
  } else if (!GATE) {
    float acc[16], t[16];
    load_bf16x16(xs[0], acc);
#pragma unroll
    for (int j = 1; j < M; ++j) {
      load_bf16x16(xs[j], t);
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] += t[c];
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) y[c] = acc[c] * (1.0f / M);
  } else {
    float xv[M][16], zv[M][16];
#pragma unroll
    for (int j = 0; j < M; ++j) {
      load_bf16x16(xs[j], xv[j]);
      load_bf16x16(zs[j], zv[j]);
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      float mx = zv[0][c];
#pragma unroll
      for (int j = 1; j < M; ++j) mx = fmaxf(mx, zv[j][c]);
      float wj[M];
      if (M == 2) {
        // one of the two max-subtracted logits is exactly 0 and expf(0) is
        // exactly 1: a single exponential gives the same two weights
        const float d0 = zv[0][c] - mx, d1 = zv[1][c] - mx;
        const float e = expf(fminf(d0, d1));
        wj[0] = d0 == 0.0f ? 1.0f : e;
        wj[M - 1] = d1 == 0.0f ? 1.0f : e;
      } else {
#pragma unroll
        for (int j = 0; j < M; ++j) wj[j] = expf(zv[j][c] - mx);
      }
      float num = 0.0f, den = 0.0f;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        num = fmaf(wj[j], xv[j][c], num);
        den += wj[j];
      }
      y[c] = __fdiv_rn(num, den);
    }
  }

  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fabsf(y[c]));
  const uint32_t sc = f32_to_e4m3(__fdiv_rn(amax, 6.0f));
  const float sv = e4m3_to_f32(sc);

  lo = 0u;
  hi = 0u;
#pragma unroll
  for (int c = 0; c < 8; ++c) lo |= e2m1_code(y[c], sv) << (4 * c);
#pragma unroll
  for (int c = 0; c < 8; ++c) hi |= e2m1_code(y[8 + c], sv) << (4 * c);
  return sc;
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
// Decode-time append: one launch per generated token and cache [0539edu §3:
// m = 2 in the encoder, 1 in the decoder; 128-token FP8 window].
// ---------------------------------------------------------------------------

// One workgroup of 128 threads per row (one new token of one sequence):
//   * every thread: 4 channels of the token into the E4M3 window ring;
//   * an open group (pos % m < m - 1): the token (and its gate logits) wait
//     in the pending buffer;
//   * a completed group: threads 0-31 pool + quantise one 16-channel group of
//     entry pos / m each, quantise 4 channels of its index key each (FP4:
//     the 32-channel group maximum over 8 neighbouring lanes) and refresh
//     4 channels of the block summary, taking the new member from their own
//     registers and the older members from the cache.
template <int M, bool GATE, int KF>
__global__ __launch_bounds__(128) void decode_append_kernel(AppendArgs a) {
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t s = a.row_seq ? a.row_seq[r] : r;
  const int64_t p = a.pos[r];
  if (s < 0 || s >= a.n_seq || p < 0 || (a.codes && p / M >= a.n_ent)) return;
  const uint16_t* x = a.x + (int64_t)r * kD;
  const uint16_t* z = GATE ? a.gate + (int64_t)r * kD : nullptr;

  // The block summary's older members [8*(e/8), e) are not written by this
  // launch: load them first, beside the token (clamped addresses, masked
  // later), so the row costs one memory latency rather than two.
  const int64_t e_ = p / M;
  const int64_t j0 = (e_ / kBlockPos) * kBlockPos;
  const int cnt = (int)(e_ - j0) + 1;            // members including the new entry
  uint32_t old_w[kBlockPos - 1], old_s[kBlockPos - 1];
  const bool summarise = a.codes && a.block_keys && (int)(p % M) == M - 1 && t < 32;
  if (summarise) {                                // uniform within each wave
#pragma unroll
    for (int i = 0; i < kBlockPos - 1; ++i) {
      const int64_t m = j0 + max(0, min(i, cnt - 2));
      if (KF == 0) {
        old_w[i] = *reinterpret_cast<const uint32_t*>(a.keys + (s * a.n_ent + m) * kIdxDim + 4 * t);
        old_s[i] = 0u;
      } else {
        old_w[i] = *reinterpret_cast<const uint16_t*>(a.keys + (s * a.n_ent + m) * 64 + 2 * t);
        old_s[i] = a.key_scales[(s * a.n_ent + m) * 4 + t / 8];
      }
    }
  }

  if (a.swa) {
    const uint2 w = *reinterpret_cast<const uint2*>(x + 4 * t);
    uint32_t b = 0u;
    b |= f32_to_e4m3(bf16_to_f32(w.x & 0xFFFFu));
    b |= f32_to_e4m3(bf16_to_f32(w.x >> 16)) << 8;
    b |= f32_to_e4m3(bf16_to_f32(w.y & 0xFFFFu)) << 16;
    b |= f32_to_e4m3(bf16_to_f32(w.y >> 16)) << 24;
    const int64_t slot = p % a.swa_cap;
    *reinterpret_cast<uint32_t*>(a.swa + (s * a.swa_cap + slot) * kD + 4 * t) = b;
  }
  if (!a.codes) return;          // a layer with a window only
  const int j = (int)(p % M);
  const int64_t e = p / M;     // the entry this token belongs to
  if (j < M - 1) {
    const int64_t pr = (s * (M - 1) + j) * kD + 4 * t;
    *reinterpret_cast<uint2*>(a.pend_x + pr) = *reinterpret_cast<const uint2*>(x + 4 * t);
    if (GATE) *reinterpret_cast<uint2*>(a.pend_gate + pr) = *reinterpret_cast<const uint2*>(z + 4 * t);
    return;
  }
  if (t >= 32) return;

  // ---- the entry: 16-channel group t
  {
    const uint16_t* xs[M];
    const uint16_t* zs[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const bool cur = i == M - 1;
      const int64_t pr = (s * (M - 1) + i) * kD + 16 * t;
      xs[i] = cur ? x + 16 * t : a.pend_x + pr;
      zs[i] = GATE ? (cur ? z + 16 * t : a.pend_gate + pr) : nullptr;
    }
    uint32_t lo, hi;
    const uint32_t sc = pool_quantize16<M, GATE>(xs, zs, lo, hi);
    const int64_t oe = s * a.n_ent + e;
    *reinterpret_cast<uint2*>(a.codes + oe * 256 + t * 8) = make_uint2(lo, hi);
    a.scales[oe * 32 + t] = (uint8_t)sc;
  }

  // ---- its index key: channels 4t .. 4t+3
  const uint16_t* kb = a.key + (int64_t)r * kIdxDim + 4 * t;
  const uint2 kw = *reinterpret_cast<const uint2*>(kb);
  float kv[4] = {bf16_to_f32(kw.x & 0xFFFFu), bf16_to_f32(kw.x >> 16), bf16_to_f32(kw.y & 0xFFFFu),
                 bf16_to_f32(kw.y >> 16)};
  const int64_t oe = s * a.n_ent + e;
  uint32_t new_key;      // E4M3: 4 bytes; FP4: 4 codes (16 bits) | scale << 16
  if (KF == 0) {
    new_key = f32_to_e4m3(kv[0]) | (f32_to_e4m3(kv[1]) << 8) | (f32_to_e4m3(kv[2]) << 16) |
              (f32_to_e4m3(kv[3]) << 24);
    *reinterpret_cast<uint32_t*>(a.keys + oe * kIdxDim + 4 * t) = new_key;
  } else {
    float amax = fmaxf(fmaxf(fabsf(kv[0]), fabsf(kv[1])), fmaxf(fabsf(kv[2]), fabsf(kv[3])));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));        // lanes 8g .. 8g+7: group g's 32 channels
    const uint32_t sc = f32_to_e4m3(__fdiv_rn(amax, 6.0f));
    const float sv = e4m3_to_f32(sc);
    uint32_t c = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) c |= e2m1_code(kv[i], sv) << (4 * i);
    *reinterpret_cast<uint16_t*>(a.keys + oe * 64 + 2 * t) = (uint16_t)c;
    if ((t & 7) == 0) a.key_scales[oe * 4 + t / 8] = (uint8_t)sc;
    new_key = c | (sc << 16);
  }

  // ---- the summary of the entry's block over the entries written so far:
  // the members loaded at the start, then the new one, in member order
  if (!summarise) return;
  const int64_t b = e / kBlockPos;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kBlockPos; ++i) {
    if (i < cnt) {
      const bool old = i < cnt - 1;
      const uint32_t w = old ? old_w[min(i, kBlockPos - 2)] : (KF == 0 ? new_key : (new_key & 0xFFFFu));
      if (KF == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += e4m3_to_f32((w >> (8 * c)) & 0xFFu);
      } else {
        const float sv = e4m3_to_f32(old ? old_s[min(i, kBlockPos - 2)] : (new_key >> 16));
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += e2m1_to_f32((w >> (4 * c)) & 0xFu) * sv;
      }
    }
  }
  uint32_t out = 0u;
#pragma unroll
  for (int c = 0; c < 4; ++c) out |= f32_to_e4m3(__fdiv_rn(acc[c], (float)cnt)) << (8 * c);
  const int64_t nb = (a.n_ent + kBlockPos - 1) / kBlockPos;
  *reinterpret_cast<uint32_t*>(a.block_keys + (s * nb + b) * kIdxDim + 4 * t) = out;
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
