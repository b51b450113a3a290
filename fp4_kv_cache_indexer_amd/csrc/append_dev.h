// Device code shared by the cache write, the decode-time append and the
// indexer's coarse scan (which can run the append of a decode step in its
// own launch): E2M1 quantisation of pooled groups [0539edu §3: fp4_e2m1 with
// e4m3_per_16_channel scales; nxbn §4.2: context-weighted pooling], the new
// entry's index key and the refreshed summary of its block [0539edu §3:
// positions_per_block 8].
#pragma once

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

// ---------------------------------------------------------------------------
// Decode-time append of one row (one generated token of one sequence)
// ---------------------------------------------------------------------------

// The entry a row's token completes, or -1: e = pos / m when the token is the
// last of its group (pos % m == m - 1), the row's sequence is in the cache
// and e < n_ent.
__device__ __forceinline__ int64_t append_entry(const AppendArgs& a, int r, int64_t& seq) {
  seq = a.row_seq ? a.row_seq[r] : r;
  const int64_t p = a.pos[r];
  if (seq < 0 || seq >= a.n_seq || p < 0 || !a.codes) return -1;
  if (p % a.m != a.m - 1 || p / a.m >= a.n_ent) return -1;
  return p / a.m;
}

// Older members [8*(e/8), e) of entry e's block, channels 4t..4t+3 (t < 32):
// E4M3 keys as one word each; FP4 keys as their 2 code bytes and the byte of
// their 32-channel group scale.  Addresses are clamped into the block, so
// members past cnt - 2 repeat a loaded one and are ignored by the summary.
template <int KF>
__device__ __forceinline__ void append_members4(const AppendArgs& a, int64_t s, int64_t e, int t,
                                                uint32_t (&old_w)[kBlockPos - 1], uint32_t (&old_s)[kBlockPos - 1]) {
  const int64_t j0 = (e / kBlockPos) * kBlockPos;
  const int cnt = (int)(e - j0) + 1;
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

// The new entry's index key, channels 4t..4t+3 of the bf16 key row (called
// by lanes t = 0..31 of one wave together: an FP4 group of 32 channels spans
// 8 neighbouring lanes).  E4M3: the 4 bytes; FP4: 4 codes (16 bits) | the
// group's scale byte << 16.
template <int KF>
__device__ __forceinline__ uint32_t append_key4(const uint16_t* key_row, int t) {
  const uint2 kw = *reinterpret_cast<const uint2*>(key_row + 4 * t);
  const float kv[4] = {bf16_to_f32(kw.x & 0xFFFFu), bf16_to_f32(kw.x >> 16), bf16_to_f32(kw.y & 0xFFFFu),
                       bf16_to_f32(kw.y >> 16)};
  if (KF == 0)
    return f32_to_e4m3(kv[0]) | (f32_to_e4m3(kv[1]) << 8) | (f32_to_e4m3(kv[2]) << 16) | (f32_to_e4m3(kv[3]) << 24);
  float amax = fmaxf(fmaxf(fabsf(kv[0]), fabsf(kv[1])), fmaxf(fabsf(kv[2]), fabsf(kv[3])));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));        // lanes 8g .. 8g+7: group g's 32 channels
  const uint32_t sc = f32_to_e4m3(__fdiv_rn(amax, 6.0f));
  const float sv = e4m3_to_f32(sc);
  uint32_t c = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) c |= e2m1_code(kv[i], sv) << (4 * i);
  return c | (sc << 16);
}

// Summary of entry e's block over its members [8*(e/8), e] written so far,
// channels 4t..4t+3 as 4 E4M3 bytes: the older members, then the new one, in
// member order, float32 sum divided by the member count (as the bulk
// summary with n_ent = e + 1).
template <int KF>
__device__ __forceinline__ uint32_t append_summary4(const uint32_t (&old_w)[kBlockPos - 1],
                                                    const uint32_t (&old_s)[kBlockPos - 1], int cnt,
                                                    uint32_t new_key) {
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
  return out;
}

// One row of the decode-time append, by threads t = 0..127 (t >= 128 do
// nothing) [0539edu §3: m = 2 in the encoder, 1 in the decoder; 128-token
// FP8 window]:
//   * every thread: 4 channels of the token into the E4M3 window ring;
//   * an open group (pos % m < m - 1): the token (and its gate logits) wait
//     in the pending buffer;
//   * a completed group: threads 0-31 pool + quantise one 16-channel group of
//     entry pos / m each, quantise 4 channels of its index key each (FP4:
//     the 32-channel group maximum over 8 neighbouring lanes) and refresh
//     4 channels of the block summary, taking the new member from their own
//     registers and the older members from the cache.
template <int M, bool GATE, int KF>
__device__ __forceinline__ void decode_append_row(const AppendArgs& a, int r, int t) {
  if (t >= 128) return;
  const int64_t s = a.row_seq ? a.row_seq[r] : r;
  const int64_t p = a.pos[r];
  if (s < 0 || s >= a.n_seq || p < 0 || (a.codes && p / M >= a.n_ent)) return;
  const uint16_t* x = a.x + (int64_t)r * kD;
  const uint16_t* z = GATE ? a.gate + (int64_t)r * kD : nullptr;

  // The block summary's older members [8*(e/8), e) are not written by this
  // row: load them first, beside the token, so the row costs one memory
  // latency rather than two.
  const int64_t e_ = p / M;
  const int cnt = (int)(e_ - (e_ / kBlockPos) * kBlockPos) + 1;   // members including the new entry
  uint32_t old_w[kBlockPos - 1], old_s[kBlockPos - 1];
  const bool summarise = a.codes && a.block_keys && (int)(p % M) == M - 1 && t < 32;
  if (summarise) append_members4<KF>(a, s, e_, t, old_w, old_s);   // uniform within each wave

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
  const int64_t oe = s * a.n_ent + e;
  const uint32_t new_key = append_key4<KF>(a.key + (int64_t)r * kIdxDim, t);
  if (KF == 0) {
    *reinterpret_cast<uint32_t*>(a.keys + oe * kIdxDim + 4 * t) = new_key;
  } else {
    *reinterpret_cast<uint16_t*>(a.keys + oe * 64 + 2 * t) = (uint16_t)(new_key & 0xFFFFu);
    if ((t & 7) == 0) a.key_scales[oe * 4 + t / 8] = (uint8_t)(new_key >> 16);
  }

  // ---- the summary of the entry's block over the entries written so far
  if (!summarise) return;
  const int64_t b = e / kBlockPos;
  const int64_t nb = (a.n_ent + kBlockPos - 1) / kBlockPos;
  *reinterpret_cast<uint32_t*>(a.block_keys + (s * nb + b) * kIdxDim + 4 * t) =
      append_summary4<KF>(old_w, old_s, cnt, new_key);
}

}  // namespace csa2
