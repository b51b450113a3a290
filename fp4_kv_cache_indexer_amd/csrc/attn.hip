// Joint sparse + sliding-window attention over the FP4 latent cache
// [daiw "four factors" table: one 512-dim latent shared by all query heads;
//  0539edu §3: top_k 512, 128-token FP8 window].
//
// Keys = values = the latent.  A workgroup of 512 threads owns (row, up to
// 64 heads, a range of keys).  Per chunk of 32 keys it gathers the selected
// FP4 entries (288 B each) and the FP8 window tokens, dequantises them
// exactly into LDS in two layouts -- key-major bf16 for QK^T and
// channel-major fp16 for PV (every dequantised value is exact in both) --
// and runs
//   S^T[t][h] = sum_c K[t][c] Q[h][c]           (v_mfma_f32_16x16x32_bf16)
//   O^T[c][h] += sum_t K[t][c] P[h][t]          (v_mfma_f32_16x16x32_f16)
// with an online softmax in float32; P enters the PV product as the sum of
// two fp16 terms (about 22 significant bits, two MFMAs on the same K
// operand) and the normaliser sums the weights as that product sees them.  The
// transposed products put one head per lane (lane % 16) in both the score
// and the output tiles.  Rows with few keys per workgroup are split over
// several workgroups whose (O, max, sum) partials are merged by
// attn_combine_kernel.
#include "attn_dev.h"
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

constexpr int kAttnThreads = 512;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kPsLo = kKeyChunk * 2;            // offset of P's low fp16 terms in a head row
constexpr int kPsStride = kKeyChunk * 4 + 16;   // bytes per head row of P (hi + lo fp16 + pad)

constexpr int kHeadsPerWG = 64;                 // up to 4 head groups of 16 per workgroup
constexpr int kMaxKeysPerSplit = 1024;          // selected ids staged in LDS per workgroup

struct AttnShared {
  uint8_t kr[kKeyChunk * kKrStride];
  uint8_t kt[kD * kKtStride];
  uint8_t ps[kHeadsPerWG * kPsStride];
  float alpha[kHeadsPerWG];     // rescale factor of the current chunk per head
  float lsum[kHeadsPerWG];      // final softmax sum per head
  int32_t kvalid[kKeyChunk];
  int32_t sidx[kMaxKeysPerSplit];
};
static_assert(offsetof(AttnShared, sidx) % 16 == 0, "staged ids are read 4 at a time");

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

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

// The raw bytes one thread gathers for its 4 keys x 8 channels of a chunk.
struct Gather {
  uint32_t code[4];   // FP4: 8 channels (one word)
  uint32_t scale[4];  // FP4: the aligned word holding the group's E4M3 scale byte
  uint2 swa[4];       // window token: 8 E4M3 bytes
  int kind[4];        // 0 none, 1 selected entry, 2 window token
};

// Per chunk, waves hg < HG (one per 16-head group) compute that group's
// scores for all 32 keys, so the online softmax stays inside the wave: each
// keeps the running max and sum of its heads in registers and hands the
// fp16 weights P and the rescale factor of its heads to the other waves
// through LDS.  All 8 waves then share the PV product: wave w owns one head
// group and a block of channel tiles, so every lane rescales its
// accumulators by a single factor.  HG, the 16-head groups of a workgroup
// (1, 2 or 4), is a compile-time constant so that the PV tile loop has no
// branches: its LDS operand reads then overlap the MFMAs instead of each
// tile waiting for its own read.
template <int HG>
__global__ __launch_bounds__(kAttnThreads, 1) void sparse_attn_kernel(AttnArgs a) {
  static_assert(HG == 1 || HG == 2 || HG == 4, "16-head groups per workgroup");
  extern __shared__ __align__(16) unsigned char attn_smem[];
  AttnShared& sh = *reinterpret_cast<AttnShared*>(attn_smem);
  const int split = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int H = a.n_heads;
  const int hbase = blockIdx.z * kHeadsPerWG;
  const bool qk_wave = wave < HG;
  // PV: waves per head group, head group and first channel tile of this wave
  constexpr int wph = kAttnWaves / HG;
  constexpr int pv_tiles = (kD / 16) / wph;
  const int pv_hg = wave / wph;
  const int pv_ct0 = (wave % wph) * pv_tiles;

  int32_t w_seq, w_len, w_st;
  scalar_words3(row_word_ptr(a.row_seq, r, a.q), row_word_ptr(a.swa_len, r, a.q), row_word_ptr(a.swa_start, r, a.q),
                w_seq, w_len, w_st);
  const int64_t seq = a.row_seq ? (int64_t)w_seq : (int64_t)r;
  const bool seq_ok = seq >= 0 && seq < a.n_seq;
  const int nsel = seq_ok ? a.top_k : 0;
  int swl = (a.swa_len && seq_ok) ? w_len : 0;
  swl = max(0, min(swl, a.swa_max));
  int swst = a.swa_start ? w_st : 0;
  if (a.swa_cap > 0) { swst %= a.swa_cap; if (swst < 0) swst += a.swa_cap; }
  const int nk = nsel + swl;
  const int k0 = split * a.keys_per_split;
  const int k1 = min(nk, k0 + a.keys_per_split);

  const int32_t* idxr = a.idx ? a.idx + (int64_t)r * a.top_k : nullptr;
  const uint8_t* codes_s = a.codes + (seq_ok ? seq : 0) * a.n_ent * (kD / 2);
  const uint8_t* scales_s = a.scales + (seq_ok ? seq : 0) * a.n_ent * (kD / kGroup);
  const uint8_t* swa_s = a.swa ? a.swa + (seq_ok ? seq : 0) * (int64_t)a.swa_cap * kD : nullptr;
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.q + (int64_t)r * H * kD);   // readable, discarded

  // stage the selected ids this split may use; the count depends on top_k
  // only, so these loads start at once, beside the row parameters
  const int nst = max(0, min(k0 + a.keys_per_split, a.top_k) - k0);
  for (int i = tid; i < nst; i += kAttnThreads) sh.sidx[i] = idxr[k0 + i];

  // QK waves: Q as the B operand of S^T = K Q^T, head n of the group,
  // channels ks*32 + 8g .. +8
  v8bf qreg[kD / 32];
  {
    const int hq = hbase + (qk_wave ? wave : 0) * 16 + n;
    const uint16_t* qrow = a.q + ((int64_t)r * H + hq) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks)
      qreg[ks] = qk_wave ? *reinterpret_cast<const v8bf*>(qrow + ks * 32) : v8bf{};
  }
  float m_run = -INFINITY, l_run = 0.0f;                     // QK waves: head n of group `wave`

  v4f acc[pv_tiles];
#pragma unroll
  for (int t = 0; t < pv_tiles; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // this thread's unit of every chunk: keys t0..t0+3, channels c0..c0+7
  const int cb = tid & 63, kq = tid >> 6;
  const int c0 = cb * 8, t0 = kq * 4;
  // sidx ready.  Also retire the Q loads here (issued with the id loads):
  // left pending into the loop, every wait for them would drain the next
  // chunk's prefetched gathers as well.
  lds_barrier();
  __builtin_amdgcn_s_waitcnt(0);

  // issue every load of a chunk at once (no data-dependent branches)
  auto issue = [&](int kc, Gather& G) {
    // the staged ids of keys kc+t0 .. kc+t0+3 in one aligned 16-byte read;
    // a read clamped to the end of the stage only feeds keys past the
    // staged (selected) ones, which do not use it
    const int sb = min(kc - k0 + t0, kMaxKeysPerSplit - 4);
    const int4 ids4 = *reinterpret_cast<const int4*>(&sh.sidx[sb]);
    const int32_t ids[4] = {ids4.x, ids4.y, ids4.z, ids4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = kc + t0 + j;
      const bool in_range = key < k1;
      const bool is_sel = in_range && key < nsel;
      const int32_t p = is_sel ? ids[j] : -1;
      const bool ok = is_sel && p >= 0 && (int64_t)p < a.n_ent;
      const bool is_swa = in_range && !is_sel;
      int slot = swst + (key - nsel);
      if (slot >= a.swa_cap) slot -= a.swa_cap;
      const uint8_t* ca = ok ? codes_s + (int64_t)p * (kD / 2) + c0 / 2 : dummy;
      const uint8_t* sa = ok ? scales_s + (int64_t)p * (kD / kGroup) + ((c0 / kGroup) & ~3) : dummy;
      const uint8_t* wa = is_swa ? swa_s + (int64_t)slot * kD + c0 : dummy;
      G.code[j] = *reinterpret_cast<const uint32_t*>(ca);
      G.scale[j] = *reinterpret_cast<const uint32_t*>(sa);   // byte extracted when used
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
      uint32_t rows[4][4];     // fp16 pairs of the 4 keys, transposed below
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float f[8];
        if (G.kind[j] == 1) {
          fp4x8_to_f32(G.code[j], e4m3_to_f32((G.scale[j] >> (8 * ((c0 / kGroup) & 3))) & 0xFFu), f);
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
      // transpose the 4x8 fp16 block: channel c0+cc gets keys t0..t0+3
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int d = cc >> 1;
        const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t w0 = __builtin_amdgcn_perm(rows[1][d], rows[0][d], sel);
        const uint32_t w1 = __builtin_amdgcn_perm(rows[3][d], rows[2][d], sel);
        *reinterpret_cast<uint2*>(sh.kt + kt_off(c0 + cc, t0 * 2)) = make_uint2(w0, w1);
      }
    }
    lds_barrier();
    // the gather registers are free again: the next chunk's loads fly during
    // this chunk's MFMAs and are consumed by the next dequantisation
    if (kc + kKeyChunk < k1) issue(kc + kKeyChunk, G);

    // ---- QK waves: S^T = K Q^T for the group's 16 heads; lane holds head n,
    // keys 4g+i (tile 0) and 16+4g+i (tile 1)
    if (qk_wave) {
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
      // P as the sum of two fp16 terms, hi = fp16(p) and lo = fp16(p - hi),
      // which carries about 22 significant bits into the PV product
      uint32_t ph[4], pl[4];
      float psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float p0 = (s[j] == -INFINITY) ? 0.0f : exp2f(s[j] - m_new);
        const float p1 = (s[j + 1] == -INFINITY) ? 0.0f : exp2f(s[j + 1] - m_new);
        const uint32_t h = pack_f16_rne(p0, p1);
        const float h0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
        const float h1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(h >> 16));
        const uint32_t l = pack_f16_rne(p0 - h0, p1 - h1);
        const float l0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(l & 0xFFFFu));
        const float l1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(l >> 16));
        ph[j >> 1] = h;
        pl[j >> 1] = l;
        // the normaliser sums the weights exactly as the PV product sees them
        psum += (h0 + l0) + (h1 + l1);
      }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      uint8_t* prow = sh.ps + (wave * 16 + n) * kPsStride;
      *reinterpret_cast<uint2*>(prow + 8 * g) = make_uint2(ph[0], ph[1]);                 // keys 4g..4g+3
      *reinterpret_cast<uint2*>(prow + 32 + 8 * g) = make_uint2(ph[2], ph[3]);            // keys 16+4g..
      *reinterpret_cast<uint2*>(prow + kPsLo + 8 * g) = make_uint2(pl[0], pl[1]);
      *reinterpret_cast<uint2*>(prow + kPsLo + 32 + 8 * g) = make_uint2(pl[2], pl[3]);
      if (g == 0) sh.alpha[wave * 16 + n] = alpha;
    }
    lds_barrier();

    // ---- all waves: O^T[c][h] += K^T P^T (fp16) over the wave's channel
    // tiles; k-slot j of lane group g is key 8g+j in both operands
    {
      const float alpha = sh.alpha[pv_hg * 16 + n];
      const uint8_t* prow = sh.ps + (pv_hg * 16 + n) * kPsStride + 16 * g;
      const v8h pb = *reinterpret_cast<const v8h*>(prow);
      const v8h pbl = *reinterpret_cast<const v8h*>(prow + kPsLo);
#pragma unroll
      for (int t = 0; t < pv_tiles; ++t) {
        const int c = (pv_ct0 + t) * 16 + n;
        const v8h ka = *reinterpret_cast<const v8h*>(sh.kt + kt_off(c, 16 * g));
        v4f o = acc[t];
        o[0] *= alpha; o[1] *= alpha; o[2] *= alpha; o[3] *= alpha;
        o = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, pbl, o, 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, pb, o, 0, 0, 0);
      }
    }
  }

  // ---- finish: QK waves hand the sums of their heads to the PV waves
  if (qk_wave && g == 0) {
    sh.lsum[wave * 16 + n] = l_run;
    const int64_t rh = (int64_t)r * H + hbase + wave * 16 + n;
    if (a.n_split == 1) {
      if (a.lse) a.lse[rh] = l_run > 0.0f ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
    } else {
      const int64_t base = (int64_t)split * a.n_rows * H + rh;
      a.part_ml[base * 2] = m_run;
      a.part_ml[base * 2 + 1] = l_run;
    }
  }
  lds_barrier();
  const int64_t rh = (int64_t)r * H + hbase + pv_hg * 16 + n;
  if (a.n_split == 1) {
    const float l = sh.lsum[pv_hg * 16 + n];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* orow = a.out + rh * kD + 4 * g;
#pragma unroll
    for (int t = 0; t < pv_tiles; ++t) {
      const v4f o = acc[t];
      *reinterpret_cast<float4*>(orow + (pv_ct0 + t) * 16) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    }
  } else {
    const int64_t base = (int64_t)split * a.n_rows * H + rh;
    float* orow = a.part_o + base * kD + 4 * g;
#pragma unroll
    for (int t = 0; t < pv_tiles; ++t) {
      const v4f o = acc[t];
      *reinterpret_cast<float4*>(orow + (pv_ct0 + t) * 16) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
}

// Merge the key-split partials of one (row, head): 128 threads x 4 channels.
// Up to 16 splits are read in one batch of unconditional (clamped) loads --
// maxima, sums and outputs together -- so the merge costs one memory
// latency; more splits take further batches against a first pass for the
// overall maximum.
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int64_t rh = blockIdx.x;
  const int64_t RH = (int64_t)a.n_rows * a.n_heads;
  const int ns = a.n_split;
  constexpr int kB = 16;
  float M = -INFINITY;
  if (ns > kB)
    for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_ml[(s * RH + rh) * 2]);
  float L = 0.0f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < ns; s0 += kB) {
    float4 p[kB];
    float ms[kB], ls[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int64_t sj = min(s0 + j, ns - 1);
      p[j] = *reinterpret_cast<const float4*>(a.part_o + (sj * RH + rh) * kD + 4 * threadIdx.x);
      ms[j] = a.part_ml[(sj * RH + rh) * 2];
      ls[j] = a.part_ml[(sj * RH + rh) * 2 + 1];
    }
    if (ns <= kB) {
#pragma unroll
      for (int j = 0; j < kB; ++j) M = fmaxf(M, ms[j]);   // clamped slots repeat a real split
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      // splits past the end, and splits that saw no key, weigh nothing
      const bool use = s0 + j < ns && ms[j] != -INFINITY && ls[j] != 0.0f;
      const float f = use ? exp2f(ms[j] - M) : 0.0f;
      L += use ? ls[j] * f : 0.0f;
      o.x += use ? p[j].x * f : 0.0f;
      o.y += use ? p[j].y * f : 0.0f;
      o.z += use ? p[j].z * f : 0.0f;
      o.w += use ? p[j].w * f : 0.0f;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  *reinterpret_cast<float4*>(a.out + rh * kD + 4 * threadIdx.x) =
      make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  if (a.lse && threadIdx.x == 0)
    a.lse[rh] = L > 0.0f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  if (a.heads_per_wg == 16) return launch_sparse_attn_narrow(a, stream);
  if (a.n_heads >= 32) return launch_sparse_attn_tile(a, stream);
  // every workgroup holds min(64, H) heads (H is 16, 32, 64 or 128)
  const int hg = min(kHeadsPerWG, a.n_heads) / 16;
  auto kern = hg == 4 ? &sparse_attn_kernel<4> : hg == 2 ? &sparse_attn_kernel<2> : &sparse_attn_kernel<1>;
  static const hipError_t attr = [] {
    hipError_t e = hipSuccess;
    for (auto k : {&sparse_attn_kernel<1>, &sparse_attn_kernel<2>, &sparse_attn_kernel<4>}) {
      const hipError_t ek = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(AttnShared));
      if (ek != hipSuccess) e = ek;
    }
    return e;
  }();
  if (attr != hipSuccess) return attr;
  const int hblocks = (a.n_heads + kHeadsPerWG - 1) / kHeadsPerWG;
  hipLaunchKernelGGL(kern, dim3((unsigned)a.n_split, (unsigned)a.n_rows, (unsigned)hblocks),
                     dim3(kAttnThreads), sizeof(AttnShared), stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t stream) {
  if (a.n_rows == 0 || a.n_split == 1) return hipSuccess;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(a.n_rows * a.n_heads)), dim3(128), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace csa2
