// Device-side helpers shared by the CSA2 kernels (gfx950 only).
//
// Number formats of the cache [0539edu §3]: FP4 E2M1 main-KV elements, FP8
// E4M3 (OCP "FN": bias 7, max 448, no inf) scales / index keys / SWA tokens,
// bf16 queries.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kD = 512;          // latent channels
constexpr int kGroup = 16;       // channels per E4M3 scale
constexpr int kIdxHeads = 32;    // indexer heads
constexpr int kIdxDim = 128;     // indexer key/query dim
constexpr int kBlockPos = 8;     // positions per hierarchical block
constexpr int kMaxTopK = 2048;
constexpr int kHistBits = 12;    // top bits of the order key used by the score histograms
constexpr int kHistBins = 1 << kHistBits;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// E4M3FN
// ---------------------------------------------------------------------------

// Exact value of an E4M3FN byte (NaN code only for S.1111.111; never used as
// data by the kernels).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  float mag;
  if (e == 0) {
    mag = (float)m * 0.001953125f;  // m * 2^-9
  } else {
    // (8 + m) * 2^(e - 10): build the float32 directly
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return s ? -mag : mag;
}

// E2M1 code (sign bit 3, magnitude index 0..7) -> float32, exact.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t m = c & 7u;
  // magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
  const float mag = m < 4u ? 0.5f * (float)m : (float)(2u << ((m - 4u) >> 1)) * (1.0f + 0.5f * (float)(m & 1u));
  return (c & 8u) ? -mag : mag;
}

// Round a finite float32 to E4M3FN: nearest, ties to even, saturate at +-448,
// zero results encoded as +0.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const float a = fabsf(x);
  uint32_t mag;
  if (!(a < 448.0f)) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {              // below 2^-6: subnormal grid of 2^-9
    mag = (uint32_t)rintf(a * 512.0f);     // exact scaling, RNE; 8 -> 0x08 = 2^-6
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // -6..8
    float q = ldexpf(a, 3 - e);            // [8, 16), exact
    uint32_t n = (uint32_t)rintf(q);       // 8..16, RNE
    if (n == 16u) { n = 8u; ++e; }
    mag = ((uint32_t)(e + 7) << 3) | (n - 8u);
  }
  if (mag == 0u) return 0u;
  return mag | ((__float_as_uint(x) >> 31) << 7);
}

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Top half of a float32 whose low 16 bits are known to be zero (exact).
__device__ __forceinline__ uint32_t f32_hi16(float f) { return __float_as_uint(f) >> 16; }

// Round-to-nearest-even float32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------------------
// Order keys for top-k: larger float -> larger unsigned; -0 folded onto +0.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_key_inv(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load and store of the wave (vmcnt(0)), which
// drains prefetches issued before it; use this one where only LDS data is
// exchanged across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Row r's word of a per-row array, or the discarded stand-in word when the
// array is absent: the load is unconditional, so a row's words go out
// together instead of one after another behind branches.
__device__ __forceinline__ const int32_t* row_word_ptr(const int32_t* arr, int r, const void* any) {
  return arr ? arr + r : static_cast<const int32_t*>(any);
}

// Two (three) uniform words through the scalar cache, issued back to back
// and waited for once, in one asm block (the compiler would otherwise wait
// for the first before issuing the second).  The addresses must be uniform
// and readable.
__device__ __forceinline__ void scalar_words2(const int32_t* p0, const int32_t* p1, int32_t& v0, int32_t& v1) {
  asm volatile(
      "s_load_dword %0, %2, 0x0\n\t"
      "s_load_dword %1, %3, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(v0), "=&s"(v1)
      : "s"(p0), "s"(p1));
}
__device__ __forceinline__ void scalar_words3(const int32_t* p0, const int32_t* p1, const int32_t* p2, int32_t& v0,
                                              int32_t& v1, int32_t& v2) {
  asm volatile(
      "s_load_dword %0, %3, 0x0\n\t"
      "s_load_dword %1, %4, 0x0\n\t"
      "s_load_dword %2, %5, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(v0), "=&s"(v1), "=&s"(v2)
      : "s"(p0), "s"(p1), "s"(p2));
}

}  // namespace csa2
