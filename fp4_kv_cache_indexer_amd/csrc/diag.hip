// Diagnostics.  The 128-term dot products of the indexer's head scores
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
typedef float v16f __attribute__((ext_vector_type(16)));

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

// ---------------------------------------------------------------------------
// Timing probes: the read shapes and the issue mix behind the kernels' designs
// ---------------------------------------------------------------------------

typedef unsigned int u4v __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 probe_load16(const uint8_t* p) {
  return NT ? __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p)))
            : *reinterpret_cast<const uint4*>(p);
}

// Reads n_rows x n_keys keys of 128 bytes the way a block-summary scan does:
// a workgroup takes `chunk` keys of one row, its four waves take groups of
// four 16-key tiles, two groups in flight.  FULL = false: lane (n, g) reads
// bytes 32g .. +31 of key n of a tile (two instructions, each touching half
// of 16 lines); FULL = true: each instruction reads 8 whole keys.  The data
// are XOR-folded and one word per thread is written.
template <bool FULL, bool NT>
__global__ __launch_bounds__(256) void scan_read_probe_kernel(const uint8_t* keys, int32_t n_keys, int32_t chunk,
                                                             int32_t chunks_per_row, uint32_t* out) {
  const int r = blockIdx.x / chunks_per_row, c = blockIdx.x % chunks_per_row;
  const int c0 = c * chunk, c1 = min(c0 + chunk, n_keys);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t acc = 0;
  if (c0 < c1) {
    const uint8_t* base = keys + (size_t)r * n_keys * kIdxDim;
    const int ngroups = (c1 - c0 + 63) / 64;
    auto load = [&](int grp, uint4 (&v)[8]) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = c0 + grp * 64 + u * 16;
        if (FULL) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int key = min(t + 8 * j + (lane >> 3), c1 - 1);
            v[2 * u + j] = probe_load16<NT>(base + (size_t)key * kIdxDim + 16 * (lane & 7));
          }
        } else {
          const int key = min(t + (lane & 15), c1 - 1);
          v[2 * u] = probe_load16<NT>(base + (size_t)key * kIdxDim + 32 * (lane >> 4));
          v[2 * u + 1] = probe_load16<NT>(base + (size_t)key * kIdxDim + 32 * (lane >> 4) + 16);
        }
      }
    };
    uint4 A[8], B[8];
    int g = wave;
    load(g, A);
    for (; g < ngroups; g += 8) {
      load(g + 4, B);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc ^= A[i].x ^ A[i].y ^ A[i].z ^ A[i].w;
      load(g + 8, A);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc ^= B[i].x ^ B[i].y ^ B[i].z ^ B[i].w;
    }
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_scan_read_probe(const uint8_t* keys, int32_t n_rows, int32_t n_keys, int32_t chunk, bool full,
                                  bool nt, uint32_t* out, hipStream_t stream) {
  const int32_t cpr = (n_keys + chunk - 1) / chunk;
  const dim3 grid((unsigned)(n_rows * cpr)), block(256);
  if (full && nt) hipLaunchKernelGGL((scan_read_probe_kernel<true, true>), grid, block, 0, stream, keys, n_keys, chunk, cpr, out);
  else if (full) hipLaunchKernelGGL((scan_read_probe_kernel<true, false>), grid, block, 0, stream, keys, n_keys, chunk, cpr, out);
  else if (nt) hipLaunchKernelGGL((scan_read_probe_kernel<false, true>), grid, block, 0, stream, keys, n_keys, chunk, cpr, out);
  else hipLaunchKernelGGL((scan_read_probe_kernel<false, false>), grid, block, 0, stream, keys, n_keys, chunk, cpr, out);
  return hipGetLastError();
}

// One dependent chain of v_mfma_f32_32x32x16_f16 per wave with NV independent
// float FMAs after each MFMA (fenced so the compiler keeps the mix).  With one
// workgroup per CU, a workgroup of 256 threads puts one wave on each SIMD, 512
// threads two.
template <int NV>
__global__ __launch_bounds__(512) void mfma_valu_probe_kernel(int32_t iters, float* out) {
  const int l = threadIdx.x;
  v8h qa, kb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    qa[i] = (_Float16)((l + i) * 0.001f);
    kb[i] = (_Float16)((l - i) * 0.001f);
  }
  v16f d = v16f{};
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = l * 0.01f + j;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      d = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa, kb, d, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NV; ++j) x[j] = fmaf(x[j], 1.0001f, 0.5f);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += d[i] + x[i];
  out[(size_t)blockIdx.x * blockDim.x + l] = s;
}

hipError_t launch_mfma_valu_probe(int32_t n_valu, int32_t threads, int32_t iters, int32_t n_wg, float* out,
                                  hipStream_t stream) {
  const dim3 grid((unsigned)n_wg), block((unsigned)threads);
  switch (n_valu) {
    case 0: hipLaunchKernelGGL(mfma_valu_probe_kernel<0>, grid, block, 0, stream, iters, out); break;
    case 4: hipLaunchKernelGGL(mfma_valu_probe_kernel<4>, grid, block, 0, stream, iters, out); break;
    case 8: hipLaunchKernelGGL(mfma_valu_probe_kernel<8>, grid, block, 0, stream, iters, out); break;
    case 12: hipLaunchKernelGGL(mfma_valu_probe_kernel<12>, grid, block, 0, stream, iters, out); break;
    default: hipLaunchKernelGGL(mfma_valu_probe_kernel<16>, grid, block, 0, stream, iters, out); break;
  }
  return hipGetLastError();
}

// The attention gather's reads without its dequantisation: rows of 512 entry
// ids over FP4 entries (256 code bytes, 32 scale bytes), one 128-thread
// workgroup per row group (rows blockIdx.x + k * gridDim.x), 32-key chunks,
// four chunks of loads in flight; ids are clamped into [0, n_ent).  WHOLE = false: lane (key n = 16 (t / 64) +
// t % 16, quarter q = (t / 16) % 4) reads 4 x 16 code bytes at 64q + 16i and
// 8 scale bytes at 8q (the attention kernels' mapping); WHOLE = true: lane
// group g of wave w takes entries 16w + 4g + i, load i reading 16 code bytes
// at 16 (t % 16) (whole lines) and 4 scale bytes.
template <bool WHOLE>
__global__ __launch_bounds__(128) void gather_probe_kernel(const uint8_t* codes, const uint8_t* scales, int64_t n_ent,
                                                          const int32_t* ids, int32_t n_rows, uint32_t* out) {
  __shared__ __align__(16) int32_t sid[512];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t acc = 0;
  for (int r = blockIdx.x; r < n_rows; r += gridDim.x) {
    __syncthreads();
    for (int i = t; i < 512; i += 128) sid[i] = (int32_t)min(max((int64_t)ids[(size_t)r * 512 + i], (int64_t)0), n_ent - 1);
    __syncthreads();
    for (int c0 = 0; c0 < 16; c0 += 4) {
      uint4 v[4][4];
      uint32_t s[4][4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int base = (c0 + cc) * 32;
        if (!WHOLE) {
          const int key = 16 * w + (lane & 15), q = (lane >> 4) & 3;
          const int64_t p = sid[base + key];
          const uint8_t* la = codes + p * 256 + 64 * q;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[cc][i] = *reinterpret_cast<const uint4*>(la + 16 * i);
          const uint2 sc = *reinterpret_cast<const uint2*>(scales + p * 32 + 8 * q);
          s[cc][0] = sc.x; s[cc][1] = sc.y; s[cc][2] = 0u; s[cc][3] = 0u;
        } else {
          const int4 pp = *reinterpret_cast<const int4*>(&sid[base + 16 * w + 4 * (lane >> 4)]);
          const int64_t p4[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[cc][i] = *reinterpret_cast<const uint4*>(codes + p4[i] * 256 + 16 * (lane & 15));
            s[cc][i] = *reinterpret_cast<const uint32_t*>(scales + p4[i] * 32 + 4 * ((lane & 15) >> 1));
          }
        }
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc ^= v[cc][i].x ^ v[cc][i].y ^ v[cc][i].z ^ v[cc][i].w ^ s[cc][i];
    }
  }
  out[(size_t)blockIdx.x * 128 + t] = acc;
}

hipError_t launch_gather_probe(const uint8_t* codes, const uint8_t* scales, int64_t n_ent, const int32_t* ids,
                               int32_t n_rows, int32_t n_wg, bool whole, uint32_t* out, hipStream_t stream) {
  if (whole)
    hipLaunchKernelGGL(gather_probe_kernel<true>, dim3((unsigned)n_wg), dim3(128), 0, stream, codes, scales, n_ent, ids,
                       n_rows, out);
  else
    hipLaunchKernelGGL(gather_probe_kernel<false>, dim3((unsigned)n_wg), dim3(128), 0, stream, codes, scales, n_ent, ids,
                       n_rows, out);
  return hipGetLastError();
}

}  // namespace csa2
