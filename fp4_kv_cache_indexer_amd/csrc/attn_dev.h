// Device helpers shared by the attention kernels: exact dequantisation of
// FP4 entries and E4M3 window tokens, bf16 packing, and the swizzled row
// layout of the key-major tiles.
#pragma once
#include "csa2_dev.h"

namespace csa2 {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

// 8 FP4 channels (one word, channel 2j in the low nibble of byte j) times the
// group scale, as float32.  The hardware decode is exact for a unit scale;
// the product with an E4M3 scale has at most 6 significant bits, so it is
// exact in float32, bf16 and fp16 alike.
__device__ __forceinline__ void fp4x8_to_f32(uint32_t w, float sv, float* f) {
  v2f t;
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); f[0] = t[0] * sv; f[1] = t[1] * sv;
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); f[2] = t[0] * sv; f[3] = t[1] * sv;
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); f[4] = t[0] * sv; f[5] = t[1] * sv;
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); f[6] = t[0] * sv; f[7] = t[1] * sv;
}

// 8 E4M3 bytes (two words) as float32 (exact).
__device__ __forceinline__ void fp8x8_to_f32(uint32_t w0, uint32_t w1, float* f) {
  v2f t;
  t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false); f[0] = t[0]; f[1] = t[1];
  t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);  f[2] = t[0]; f[3] = t[1];
  t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false); f[4] = t[0]; f[5] = t[1];
  t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);  f[6] = t[0]; f[7] = t[1];
}

// Two exactly representable floats as a bf16 pair (their top halves).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// bf16 bits of a finite float, round to nearest even.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Swizzled rows of 64 segments of 16 bytes (8 bf16 channels): logical
// segment s of row t sits at s ^ tile_sw(t).  Reads of one segment of 16
// consecutive rows, and transpose reads of 2 segments of 4 rows per 16
// lanes, then hit distinct bank groups.
__device__ __forceinline__ int tile_sw(int t) { return ((t & 7) << 1) | ((t >> 3) & 1); }

}  // namespace csa2
