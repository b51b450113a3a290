// Joint sparse + sliding-window attention over the FP4 latent cache
// [daiw "four factors" table: one 512-dim latent shared by all query heads;
//  0539edu §3: top_k 512, 128-token FP8 window].
//
// Keys = values = the latent.  A workgroup owns (row, 64 heads, a range of
// keys).  Per chunk of 32 keys it gathers the selected FP4 entries (288 B
// each) and the FP8 window tokens, dequantises them exactly to bf16 into LDS
// in two layouts -- key-major bf16 for QK^T and channel-major fp16 for PV
// (every dequantised value is exact in both) -- and runs
//   S^T[t][h] = sum_c K[t][c] Q[h][c]           (v_mfma_f32_16x16x32_bf16)
//   O^T[c][h] += sum_t K[t][c] P[h][t]          (v_mfma_f32_16x16x32_f16)
// P is rounded to fp16 (11 significant bits) for the PV product.
// with an online softmax in float32.  Computing the transposed products puts
// one head per lane (lane % 16) in both the score tile and the output tile,
// so the softmax statistics never leave the lane group and P feeds the PV
// MFMA straight from registers.  Rows with few keys per workgroup are split
// over several workgroups whose (O, max, sum) partials are merged by
// attn_combine_kernel.
#include "csa2_dev.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int kKeyChunk = 32;
constexpr int kKrStride = kD * 2 + 16;          // bytes per key row in LDS (bf16 + pad)
constexpr int kKtStride = kKeyChunk * 2 + 16;   // bytes per channel row in LDS

// Channel-major rows hold 4 slots of 16 bytes (8 keys each).  Slot s of row
// c is stored at slot s ^ ((c >> 3) & 3): the transposing writes (lanes 8
// rows apart) then spread over the banks, and the PV operand reads (16
// consecutive rows) stay conflict-free.
__device__ __forceinline__ int kt_off(int c, int byte) {
  return c * kKtStride + ((((byte >> 4) ^ (c >> 3)) & 3) << 4) + (byte & 15);
}

constexpr int kMaxKeysPerSplit = 1024;          // selected ids staged in LDS per workgroup

struct AttnShared {
  uint8_t kr[kKeyChunk * kKrStride];
  uint8_t kt[kD * kKtStride];
  int32_t kvalid[kKeyChunk];
  int32_t sidx[kMaxKeysPerSplit];
};

typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

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

// Two floats as an fp16 pair; exact inputs pass unchanged.
__device__ __forceinline__ uint32_t pack_f16_exact(float lo, float hi) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(lo, hi);
  return __builtin_bit_cast(uint32_t, h);
}

// Two floats as an fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16_rne(float lo, float hi) {
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// The raw bytes one thread gathers for its 8 keys x 8 channels of a chunk.
struct Gather {
  uint32_t code[8];   // FP4: 8 channels (one word)
  uint32_t scale[8];  // FP4: the group's E4M3 scale byte
  uint2 swa[8];       // window token: 8 E4M3 bytes
  int kind[8];        // 0 none, 1 selected entry, 2 window token
};

// One wave per SIMD: the 128 output accumulators live in AGPRs next to the
// 64 query registers, so nothing spills.  Always 4 waves: every wave gathers
// and dequantises; waves past the row's head count skip the MFMA work.
__global__ __launch_bounds__(256, 1) void sparse_attn_kernel(AttnArgs a) {
  __shared__ AttnShared sh;
  const int split = blockIdx.x, r = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int H = a.n_heads;
  const bool computes = hg * 64 + wave * 16 < H;
  const int h = computes ? hg * 64 + wave * 16 + n : 0;
  const int64_t seq = a.row_seq ? a.row_seq[r] : r;
  const bool seq_ok = seq >= 0 && seq < a.n_seq;
  const int nsel = seq_ok ? a.top_k : 0;
  int swl = (a.swa_len && seq_ok) ? a.swa_len[r] : 0;
  swl = max(0, min(swl, a.swa_cap));
  int swst = a.swa_start ? a.swa_start[r] : 0;
  if (a.swa_cap > 0) { swst %= a.swa_cap; if (swst < 0) swst += a.swa_cap; }
  const int nk = nsel + swl;
  const int k0 = split * a.keys_per_split;
  const int k1 = min(nk, k0 + a.keys_per_split);

  const int32_t* idxr = a.idx ? a.idx + (int64_t)r * a.top_k : nullptr;
  const uint8_t* codes_s = a.codes + (seq_ok ? seq : 0) * a.n_ent * (kD / 2);
  const uint8_t* scales_s = a.scales + (seq_ok ? seq : 0) * a.n_ent * (kD / kGroup);
  const uint8_t* swa_s = a.swa ? a.swa + (seq_ok ? seq : 0) * (int64_t)a.swa_cap * kD : nullptr;
  const uint16_t* qrow = a.q + ((int64_t)r * H + h) * kD + 8 * g;
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.q + (int64_t)r * H * kD);   // readable, discarded

  // stage this split's selected ids
  const int nsel_here = max(0, min(k1, nsel) - k0);
  for (int i = tid; i < nsel_here; i += 256) sh.sidx[i] = idxr[k0 + i];

  // Q as the B operand of S^T = K Q^T: head n, channels ks*32 + 8g .. +8.
  v8bf qreg[kD / 32];
#pragma unroll
  for (int ks = 0; ks < kD / 32; ++ks)
    qreg[ks] = computes ? *reinterpret_cast<const v8bf*>(qrow + ks * 32) : v8bf{};

  v4f acc[kD / 16];
#pragma unroll
  for (int ct = 0; ct < kD / 16; ++ct) acc[ct] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  // this thread's unit of every chunk: keys t0..t0+7, channels c0..c0+7
  const int cb = tid & 63, kg = tid >> 6;
  const int c0 = cb * 8, t0 = kg * 8;
  lds_barrier();                                     // sidx ready (q loads stay in flight)

  // issue every load of a chunk at once (no data-dependent branches)
  auto issue = [&](int kc, Gather& G) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = kc + t0 + j;
      const bool in_range = key < k1;
      const bool is_sel = in_range && key < nsel;
      const int32_t p = is_sel ? sh.sidx[key - k0] : -1;
      const bool ok = is_sel && p >= 0 && (int64_t)p < a.n_ent;
      const bool is_swa = in_range && !is_sel;
      int slot = swst + (key - nsel);
      if (slot >= a.swa_cap) slot -= a.swa_cap;
      const uint8_t* ca = ok ? codes_s + (int64_t)p * (kD / 2) + c0 / 2 : dummy;
      const uint8_t* sa = ok ? scales_s + (int64_t)p * (kD / kGroup) + c0 / kGroup : dummy;
      const uint8_t* wa = is_swa ? swa_s + (int64_t)slot * kD + c0 : dummy;
      G.code[j] = *reinterpret_cast<const uint32_t*>(ca);
      G.scale[j] = *sa;
      G.swa[j] = *reinterpret_cast<const uint2*>(wa);
      G.kind[j] = ok ? 1 : (is_swa ? 2 : 0);
    }
  };

  Gather G;
  if (k0 < k1) issue(k0, G);
  for (int kc = k0; kc < k1; kc += kKeyChunk) {
    lds_barrier();     // the previous chunk's LDS reads are done
    // ---- dequantise the gathered bytes into LDS (bf16 key-major, fp16 channel-major)
    {
      uint32_t rows[8][4];     // fp16 pairs of the 8 keys, transposed below
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float f[8];
        if (G.kind[j] == 1) {
          fp4x8_to_f32(G.code[j], e4m3_to_f32(G.scale[j]), f);
        } else if (G.kind[j] == 2) {
          fp8x8_to_f32(G.swa[j].x, G.swa[j].y, f);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) f[i] = 0.0f;
        }
        *reinterpret_cast<uint4*>(sh.kr + (t0 + j) * kKrStride + c0 * 2) =
            make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
#pragma unroll
        for (int q = 0; q < 4; ++q) rows[j][q] = pack_f16_exact(f[2 * q], f[2 * q + 1]);
        if (cb == 0) sh.kvalid[t0 + j] = G.kind[j] != 0;
      }
      // transpose the 8x8 fp16 block: channel c0+cc gets keys t0..t0+7
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int d = cc >> 1;
        const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
        uint32_t t[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) t[q] = __builtin_amdgcn_perm(rows[2 * q + 1][d], rows[2 * q][d], sel);
        *reinterpret_cast<uint4*>(sh.kt + kt_off(c0 + cc, t0 * 2)) = make_uint4(t[0], t[1], t[2], t[3]);
      }
    }
    lds_barrier();
    // the gather registers are free again: the next chunk's loads fly during
    // this chunk's MFMAs and are consumed by the next dequantisation
    if (kc + kKeyChunk < k1) issue(kc + kKeyChunk, G);
    if (!computes) continue;

    // ---- S^T = K Q^T for the wave's 16 heads: lane holds head n, keys 4g+i and 16+4g+i
    float s[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      v4f st = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = sh.kr + (mt * 16 + n) * kKrStride + 16 * g;
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) {
        const v8bf ka = *reinterpret_cast<const v8bf*>(krow + ks * 64);
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qreg[ks], st, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s[mt * 4 + i] = st[i];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = (j < 4) ? (4 * g + j) : (16 + 4 * g + j - 4);
      s[j] = sh.kvalid[t] ? s[j] * a.sm_scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
    uint32_t pw[4];
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float p0 = (s[j] == -INFINITY) ? 0.0f : exp2f(s[j] - m_new);
      const float p1 = (s[j + 1] == -INFINITY) ? 0.0f : exp2f(s[j + 1] - m_new);
      pw[j >> 1] = pack_f16_rne(p0, p1);
      // the normaliser sums the weights exactly as the PV product sees them
      psum += (float)__builtin_bit_cast(_Float16, (uint16_t)(pw[j >> 1] & 0xFFFFu)) +
              (float)__builtin_bit_cast(_Float16, (uint16_t)(pw[j >> 1] >> 16));
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    v8h pb;
    {
      uint32_t* pbw = reinterpret_cast<uint32_t*>(&pb);
      pbw[0] = pw[0]; pbw[1] = pw[1]; pbw[2] = pw[2]; pbw[3] = pw[3];
    }

    // ---- O^T[c][h] += K^T P^T (fp16): A rows = channels, k-slot j <-> key 4g+j / 16+4g+j-4
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct) {
      const int c = ct * 16 + n;
      const uint2 lo = *reinterpret_cast<const uint2*>(sh.kt + kt_off(c, 8 * g));
      const uint2 hi = *reinterpret_cast<const uint2*>(sh.kt + kt_off(c, 32 + 8 * g));
      v8h ka;
      uint32_t* kaw = reinterpret_cast<uint32_t*>(&ka);
      kaw[0] = lo.x; kaw[1] = lo.y; kaw[2] = hi.x; kaw[3] = hi.y;
      v4f o = acc[ct];
      o[0] *= alpha; o[1] *= alpha; o[2] *= alpha; o[3] *= alpha;
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, pb, o, 0, 0, 0);
    }
  }

  if (!computes) return;
  // ---- finish: the full sum for head n lives across the 4 lane groups
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const int64_t rh = (int64_t)r * H + h;
  if (a.n_split == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float* orow = a.out + rh * kD + 4 * g;
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct) {
      const v4f o = acc[ct];
      *reinterpret_cast<float4*>(orow + ct * 16) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    }
    if (a.lse && g == 0)
      a.lse[rh] = l_run > 0.0f ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
  } else {
    const int64_t base = ((int64_t)split * a.n_rows * H + rh);
    float* orow = a.part_o + base * kD + 4 * g;
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct) {
      const v4f o = acc[ct];
      *reinterpret_cast<float4*>(orow + ct * 16) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (g == 0) {
      a.part_ml[base * 2] = m_run;
      a.part_ml[base * 2 + 1] = l_run;
    }
  }
}

// Merge the key-split partials of one (row, head): 128 threads x 4 channels.
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int64_t rh = blockIdx.x;
  const int64_t RH = (int64_t)a.n_rows * a.n_heads;
  float M = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, a.part_ml[(s * RH + rh) * 2]);
  float L = 0.0f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < a.n_split; ++s) {
    const float ms = a.part_ml[(s * RH + rh) * 2];
    const float ls = a.part_ml[(s * RH + rh) * 2 + 1];
    if (ms == -INFINITY || ls == 0.0f) continue;
    const float f = exp2f(ms - M);
    L += ls * f;
    const float4 p = *reinterpret_cast<const float4*>(a.part_o + (s * RH + rh) * kD + 4 * threadIdx.x);
    o.x += p.x * f; o.y += p.y * f; o.z += p.z * f; o.w += p.w * f;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  *reinterpret_cast<float4*>(a.out + rh * kD + 4 * threadIdx.x) =
      make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  if (a.lse && threadIdx.x == 0)
    a.lse[rh] = L > 0.0f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  const int hgroups = (a.n_heads + 63) / 64;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3((unsigned)a.n_split, (unsigned)a.n_rows, (unsigned)hgroups),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t stream) {
  if (a.n_rows == 0 || a.n_split == 1) return hipSuccess;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(a.n_rows * a.n_heads)), dim3(128), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace csa2
