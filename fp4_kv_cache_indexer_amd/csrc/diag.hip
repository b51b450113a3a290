// Diagnostics: the 128-term dot products of the indexer's head scores
// [0539edu §3: q . k over the 128 index dims, E4M3 operands, float32
// accumulation] computed two ways on the matrix cores, so that a test can
// hold both against the exact sums:
//   * widened to fp16 and summed by v_mfma_f32_16x16x32_f16 in four 32-term
//     steps, as the indexer scans do (every E4M3 value is an fp16 value and
//     every product of two is exact in float32);
//   * fed as E4M3 to v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales,
//     one instruction for all 128 terms.
#include "csa2_dev.h"
#include "csa2_launch.h"

namespace csa2 {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8h e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

}  // namespace

// One wave per 16 x 16 block of (query, key) pairs.  Lane l holds bytes
// 32(l/16) .. +31 of query row l%16 and of key row l%16: the A and B
// operands take the same 32 dims per lane, so either instruction forms the
// full 128-term sum whatever order it adds them in.
__global__ __launch_bounds__(64) void mfma_dot_probe_kernel(const uint8_t* q, const uint8_t* k, int32_t n_k,
                                                            float* out16, float* out8) {
  const int lane = threadIdx.x;
  const int row = lane & 15, quarter = lane >> 4;
  const int qi = blockIdx.y * 16 + row, ki = blockIdx.x * 16 + row;
  const uint4* qp = reinterpret_cast<const uint4*>(q + (int64_t)qi * kIdxDim + 32 * quarter);
  const uint4* kp = reinterpret_cast<const uint4*>(k + (int64_t)ki * kIdxDim + 32 * quarter);
  const uint4 q0 = qp[0], q1 = qp[1], k0 = kp[0], k1 = kp[1];
  const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};

  v4f d16 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int v = 0; v < 4; ++v)
    d16 = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16(qw[2 * v], qw[2 * v + 1]),
                                                 e4m3x8_to_f16(kw[2 * v], kw[2 * v + 1]), d16, 0, 0, 0);
  const v8i qa = {(int)qw[0], (int)qw[1], (int)qw[2], (int)qw[3], (int)qw[4], (int)qw[5], (int)qw[6], (int)qw[7]};
  const v8i kb = {(int)kw[0], (int)kw[1], (int)kw[2], (int)kw[3], (int)kw[4], (int)kw[5], (int)kw[6], (int)kw[7]};
  // format codes 0 (E4M3) for both operands; scale exponents 127 (x1)
  const v4f d8 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, kb, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127,
                                                                  0, 127);
  // D[i][j] = sum_k A[i][k] B[k][j]: lane l holds column l%16 (key), rows
  // 4(l/16) + r (queries) in register r
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t o = (int64_t)(blockIdx.y * 16 + 4 * quarter + r) * n_k + blockIdx.x * 16 + row;
    out16[o] = d16[r];
    out8[o] = d8[r];
  }
}

hipError_t launch_mfma_dot_probe(const uint8_t* q, const uint8_t* k, int32_t n_q, int32_t n_k, float* out16,
                                 float* out8, hipStream_t stream) {
  if (n_q <= 0 || n_k <= 0) return hipSuccess;
  hipLaunchKernelGGL(mfma_dot_probe_kernel, dim3((unsigned)(n_k / 16), (unsigned)(n_q / 16)), dim3(64), 0, stream,
                     q, k, n_k, out16, out8);
  return hipGetLastError();
}

}  // namespace csa2
