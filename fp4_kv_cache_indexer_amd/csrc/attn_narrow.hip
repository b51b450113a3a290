// Joint sparse + sliding-window attention for few rows: one 16-head group per
// workgroup [daiw "four factors" table: one 512-dim latent shared by all
// query heads; 0539edu §3: top_k 512, 128-token FP8 window].
//
// Same mathematics as sparse_attn_kernel (attn.hip), shaped for latency when
// the rows alone cannot fill the GPU: a row's heads are spread over 16-head
// workgroups and its keys over splits, and each workgroup needs only ~53 KB
// of LDS and 128 registers per lane, so two share a CU.  Per chunk of
// 32 keys:
//   * all 512 threads gather the selected FP4 entries (256 code + 32 E4M3
//     scale bytes each) or FP8 window tokens and dequantise them exactly into
//     one key-major bf16 tile (swizzled rows);
//   * waves 0 and 1 compute S^T[t][h] = sum_c K[t][c] Q[h][c] for keys
//     16w..16w+15 (Q staged in LDS, v_mfma_f32_16x16x32_bf16), exchange
//     their chunk maxima through LDS so both keep the same reference max,
//     run the online softmax in float32 and hand P to the other waves as
//     hi + lo bf16 terms (about 16 significant bits) with the rescale factor;
//     each sums the weights of its own keys;
//   * all 8 waves accumulate O^T[c][h] += sum_t K[t][c] P[h][t] for 4 channel
//     tiles each, reading K^T from the tile with the LDS transpose read.
// The score tiles leave head n and keys {4g..4g+3} (wave 0) and
// {16+4g..16+4g+3} (wave 1) in lane (n, g), exactly the k-slot order of the
// PV operand the transpose read builds, so lane (n, g) of every wave reads
// the 32 bytes lanes (n, g) of waves 0 and 1 wrote.  Split partials are
// merged by attn_combine_kernel.
#include <algorithm>

#include "attn_dev.h"
#include "csa2_launch.h"

namespace csa2 {

namespace {

constexpr int kChunk = 32;
constexpr int kRow = kD * 2;                   // bytes of one bf16 row of 512 channels
constexpr int kHeads = 16;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kTilesPerWave = (kD / 16) / kWaves;   // 4 output channel tiles per wave
constexpr int kMaxSplitKeys = 512;             // selected ids of one workgroup at most
constexpr float kSlack = 8.0f;                 // log2 growth of the max tolerated before rescaling

struct NarrowShared {
  uint8_t tile[kChunk * kRow];                 // dequantised keys, swizzled rows
  uint8_t q[kHeads * kRow];                    // Q of the group, swizzled rows
  uint4 p[kHeads * 4][2];                      // per (head, lane group): P hi, P lo
  float alpha[kHeads];
  float mx[2][kHeads];                         // the two key halves' chunk maxima
  float lsum[2][kHeads];                       // the two key halves' weight sums
  int32_t kvalid[kChunk];
  int32_t sidx[kMaxSplitKeys + 1];             // + a slot for threads that stage no id
};

// The raw bytes one thread gathers for its key and 32 channels of a chunk:
// a selected entry's 16 code bytes and the 16-byte half of its scale row
// holding its two group scales, or a window token's 32 bytes.
struct Gather32 {
  uint4 lo, hi;
  int kind;           // 0 none, 1 selected entry, 2 window token
};

}  // namespace

__global__ __launch_bounds__(kThreads, 4) void sparse_attn_narrow_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char narrow_smem[];
  NarrowShared& sh = *reinterpret_cast<NarrowShared*>(narrow_smem);
  // Workgroups go to the 8 XCDs in turn by linear id; work item t is taken
  // by workgroup (t mod B) * 8 + t / B, so that XCD x holds the contiguous
  // items [xB, xB + B), head group fastest: the head groups of one (row,
  // split), which gather the same keys, share one L2.
  const int H = a.n_heads;
  const int nhg = H / kHeads;
  const int t = (int)(blockIdx.x & 7u) * a.xcd_block + (int)(blockIdx.x >> 3);
  if (t >= a.n_split * a.n_rows * nhg) return;   // padding of the last blocks
  const int hg = t % nhg, sr = t / nhg;
  const int split = sr % a.n_split, r = sr / a.n_split;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int hbase = hg * kHeads;

  int32_t w_seq, w_len, w_st;                    // loaded together
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

  // stage the split's selected ids (one per thread; a split without any
  // reads Q's first word) and the group's Q: all loads go out before the
  // first LDS write waits for them
  static_assert(kMaxSplitKeys <= kThreads, "one staged id per thread");
  constexpr int kQPer = kHeads * kRow / 16 / kThreads;  // 16-byte Q units per thread
  const int nst = max(0, min(k0 + a.keys_per_split, a.top_k) - k0);
  const int32_t id_v = *(nst > 0 ? idxr + k0 + min(tid, nst - 1) : reinterpret_cast<const int32_t*>(a.q));
  uint4 qv[kQPer];
#pragma unroll
  for (int i = 0; i < kQPer; ++i) {
    const int u = i * kThreads + tid;              // 16-byte unit: head u/64, segment u%64
    qv[i] = *reinterpret_cast<const uint4*>(a.q + ((int64_t)r * H + hbase + (u >> 6)) * kD + (u & 63) * 8);
  }
  sh.sidx[tid < nst ? tid : kMaxSplitKeys] = id_v;   // no branch for the Q loads to sink below
#pragma unroll
  for (int i = 0; i < kQPer; ++i) {
    const int u = i * kThreads + tid;
    const int h = u >> 6, seg = u & 63;
    *reinterpret_cast<uint4*>(sh.q + h * kRow + ((seg ^ tile_sw(h)) << 4)) = qv[i];
  }
  float m_run = -INFINITY, l_run = 0.0f;            // waves 0, 1: head n, own key half
  v4f acc[kTilesPerWave];
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // dequantisation unit: key tq, channels 32cq .. 32cq+31
  const int tq = tid >> 4, cq = tid & 15;
  // operand offsets: row n of a 16-row block at segment 4ks + g (physical
  // 4(ks ^ (sw >> 2)) + (g ^ (sw & 3))); transpose reads of rows 4g + n/4,
  // channels 16ct + 4(n%4) (physical segment 2(ct ^ (sw >> 1)) + (e ^ (sw & 1))):
  // the varying parts are XORed into bits the bases leave for them
  const int swn = tile_sw(n);
  const int qk_base = n * kRow + ((g ^ (swn & 3)) << 4) + ((swn >> 2) << 6);
  const int tr_row = 4 * g + (n >> 2);
  const int tr_sw = tile_sw(tr_row);
  const int pv_base = tr_row * kRow + ((((n & 3) >> 1) ^ (tr_sw & 1)) << 4) + (n & 1) * 8 + ((tr_sw >> 1) << 5);
  const int ct0 = wave * kTilesPerWave;

  lds_barrier();                 // sidx and Q staged
  __builtin_amdgcn_s_waitcnt(0); // and their loads retired (the gathers are counted from here)

  auto issue = [&](int kc, Gather32& G) __attribute__((always_inline)) {
    const int key = kc + tq;
    const bool in_range = key < k1;
    const bool is_sel = in_range && key < nsel;
    const int32_t p = is_sel ? sh.sidx[min(max(key - k0, 0), kMaxSplitKeys - 1)] : -1;
    const bool ok = is_sel && p >= 0 && (int64_t)p < a.n_ent;
    const bool is_swa = in_range && !is_sel;
    int slot = swst + (key - nsel);
    if (slot >= a.swa_cap) slot -= a.swa_cap;
    const uint8_t* wa = is_swa ? swa_s + (int64_t)slot * kD + 32 * cq : dummy;
    const uint8_t* la = ok ? codes_s + (int64_t)p * (kD / 2) + 16 * cq : wa;
    const uint8_t* ha = ok ? scales_s + (int64_t)p * (kD / kGroup) + ((2 * cq) & ~15) : wa + 16;
    G.lo = *reinterpret_cast<const uint4*>(la);
    G.hi = *reinterpret_cast<const uint4*>(ha);
    G.kind = ok ? 1 : (is_swa ? 2 : 0);
  };

  Gather32 G;
  issue(k0, G);
  for (int kc = k0; kc < k1; kc += kChunk) {
    // ---- dequantise the gathered bytes into the tile
    {
      float f[32];
      if (G.kind == 1) {
        const int b0 = (2 * cq) & 15;                 // scale bytes of groups 2cq, 2cq+1
        const uint32_t w01 = (b0 & 4) ? G.hi.y : G.hi.x;
        const uint32_t w23 = (b0 & 4) ? G.hi.w : G.hi.z;
        const uint32_t w = (b0 & 8) ? w23 : w01;
        const float s0 = e4m3_to_f32((w >> (8 * (b0 & 3))) & 0xFFu);
        const float s1 = e4m3_to_f32((w >> (8 * ((b0 & 3) + 1))) & 0xFFu);
        fp4x8_to_f32(G.lo.x, s0, f);
        fp4x8_to_f32(G.lo.y, s0, f + 8);
        fp4x8_to_f32(G.lo.z, s1, f + 16);
        fp4x8_to_f32(G.lo.w, s1, f + 24);
      } else if (G.kind == 2) {
        fp8x8_to_f32(G.lo.x, G.lo.y, f);
        fp8x8_to_f32(G.lo.z, G.lo.w, f + 8);
        fp8x8_to_f32(G.hi.x, G.hi.y, f + 16);
        fp8x8_to_f32(G.hi.z, G.hi.w, f + 24);
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) f[i] = 0.0f;
      }
      const int sw = tile_sw(tq);
      uint8_t* row = sh.tile + tq * kRow;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<uint4*>(row + (((4 * cq + q4) ^ sw) << 4)) =
            make_uint4(pack_bf16(f[8 * q4], f[8 * q4 + 1]), pack_bf16(f[8 * q4 + 2], f[8 * q4 + 3]),
                       pack_bf16(f[8 * q4 + 4], f[8 * q4 + 5]), pack_bf16(f[8 * q4 + 6], f[8 * q4 + 7]));
      sh.kvalid[tq] = G.kind != 0;              // the key's 16 threads store the same value
    }
    // the gather registers are free: the next chunk's loads fly during this one
    if (kc + kChunk < k1) issue(kc + kChunk, G);
    lds_barrier();

    // ---- waves 0 and 1: scores of keys 16w..16w+15, softmax, P.  Both keep
    // the same reference max (from both halves' maxima, exchanged in LDS)
    // and each sums the weights of its own keys.
    float s[4];
    if (wave < 2) {
      int qk_b = qk_base;
      asm volatile("" : "+v"(qk_b));
      const int toff = wave * 16 * kRow;
      // two accumulators (even and odd channel steps) halve the dependent
      // MFMA chain
      v4f sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kD / 32; ks += 2) {
        const int off0 = (qk_b ^ ((ks & 3) << 6)) + (ks >> 2) * 256;
        const int off1 = (qk_b ^ (((ks + 1) & 3) << 6)) + ((ks + 1) >> 2) * 256;
        const v8bf qa = *reinterpret_cast<const v8bf*>(sh.q + off0);
        const v8bf ka = *reinterpret_cast<const v8bf*>(sh.tile + off0 + toff);
        const v8bf qb = *reinterpret_cast<const v8bf*>(sh.q + off1);
        const v8bf kb = *reinterpret_cast<const v8bf*>(sh.tile + off1 + toff);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qa, sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb, sb, 0, 0, 0);
        if ((ks & 7) == 6) __builtin_amdgcn_sched_barrier(0);   // bounded read-ahead
      }
      const v4f st = sa + sb;
      const int4 vv = *reinterpret_cast<const int4*>(&sh.kvalid[16 * wave + 4 * g]);
      s[0] = vv.x ? st[0] * a.sm_scale_log2 : -INFINITY;
      s[1] = vv.y ? st[1] * a.sm_scale_log2 : -INFINITY;
      s[2] = vv.z ? st[2] * a.sm_scale_log2 : -INFINITY;
      s[3] = vv.w ? st[3] * a.sm_scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (g == 0) sh.mx[wave][n] = mx;
    }
    lds_barrier();
    if (wave < 2) {
      const float mx = fmaxf(sh.mx[0][n], sh.mx[1][n]);
      // the reference max moves only when the chunk's max exceeds it by more
      // than the slack (weights stay below 2^slack); only then are the
      // accumulators rescaled
      const bool move = mx > m_run + kSlack;
      const float m_new = move ? mx : m_run;
      const float alpha = (move && m_run != -INFINITY) ? exp2f(m_run - m_new) : 1.0f;
      m_run = m_new;
      uint32_t ph[2], pl[2];
      float psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        // the hardware exp2 (weights below 2^-126 may flush to zero)
        const float p0 = (s[j] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s[j] - m_new);
        const float p1 = (s[j + 1] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s[j + 1] - m_new);
        const uint32_t h0 = bf16_rne(p0), h1 = bf16_rne(p1);
        const float hf0 = __uint_as_float(h0 << 16), hf1 = __uint_as_float(h1 << 16);
        const uint32_t l0 = bf16_rne(p0 - hf0), l1 = bf16_rne(p1 - hf1);
        ph[j >> 1] = h0 | (h1 << 16);
        pl[j >> 1] = l0 | (l1 << 16);
        // the normaliser sums the weights exactly as the PV product sees them
        psum += (hf0 + __uint_as_float(l0 << 16)) + (hf1 + __uint_as_float(l1 << 16));
      }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      l_run = l_run * alpha + psum;
      // k-slots 0-3 (keys 4g..4g+3) from wave 0, 4-7 (16+4g..) from wave 1
      reinterpret_cast<uint2*>(&sh.p[n * 4 + g][0])[wave] = make_uint2(ph[0], ph[1]);
      reinterpret_cast<uint2*>(&sh.p[n * 4 + g][1])[wave] = make_uint2(pl[0], pl[1]);
      if (wave == 0 && g == 0) sh.alpha[n] = alpha;
    }
    lds_barrier();

    // ---- all waves: O^T += K^T P^T over 4 channel tiles; k-slots 0-3 of
    // lane group g are keys 4g..4g+3, slots 4-7 keys 16+4g..16+4g+3
    {
      int pv_b = pv_base;
      asm volatile("" : "+v"(pv_b));
      const float alpha = sh.alpha[n];
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int t = 0; t < kTilesPerWave; ++t) {
          acc[t][0] *= alpha; acc[t][1] *= alpha; acc[t][2] *= alpha; acc[t][3] *= alpha;
        }
      }
      const v8bf pb = __builtin_bit_cast(v8bf, sh.p[n * 4 + g][0]);
      const v8bf pbl = __builtin_bit_cast(v8bf, sh.p[n * 4 + g][1]);
#pragma unroll
      for (int t = 0; t < kTilesPerWave; ++t) {
        const int ct = ct0 + t;
        const uint8_t* base = sh.tile + (pv_b ^ ((ct & 7) << 5)) + (ct >> 3) * 256;
        const v4s k_lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base));
        const v4s k_hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + 16 * kRow));
        const v8bf ka = __builtin_bit_cast(v8bf, make_uint4(
            __builtin_bit_cast(uint2, k_lo).x, __builtin_bit_cast(uint2, k_lo).y,
            __builtin_bit_cast(uint2, k_hi).x, __builtin_bit_cast(uint2, k_hi).y));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, pbl, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, pb, acc[t], 0, 0, 0);
      }
    }
    lds_barrier();                 // the tile is free for the next chunk
  }

  // ---- finish: waves 0 and 1 hand their sums to the others
  const int64_t rh = (int64_t)r * H + hbase + n;
  if (wave < 2 && g == 0) sh.lsum[wave][n] = l_run;
  lds_barrier();
  const float l = sh.lsum[0][n] + sh.lsum[1][n];
  if (wave == 0 && g == 0) {
    if (a.n_split == 1) {
      if (a.lse) a.lse[rh] = l > 0.0f ? (m_run + log2f(l)) * 0.69314718055994531f : -INFINITY;
    } else {
      const int64_t base = (int64_t)split * a.n_rows * H + rh;
      a.part_ml[base * 2] = m_run;
      a.part_ml[base * 2 + 1] = l;
    }
  }
  if (a.n_split == 1) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* orow = a.out + rh * kD + 4 * g;
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const v4f o = acc[t];
      *reinterpret_cast<float4*>(orow + (ct0 + t) * 16) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    }
  } else {
    const int64_t base = (int64_t)split * a.n_rows * H + rh;
    float* orow = a.part_o + base * kD + 4 * g;
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const v4f o = acc[t];
      *reinterpret_cast<float4*>(orow + (ct0 + t) * 16) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_sparse_attn_narrow(const AttnArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  // a split stages at most kMaxSplitKeys selected ids (window keys need none)
  if (std::min(a.keys_per_split, a.top_k) > kMaxSplitKeys || a.n_heads % kHeads) return hipErrorInvalidValue;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&sparse_attn_narrow_kernel),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)sizeof(NarrowShared));
  if (attr != hipSuccess) return attr;
  // the XCD-major order of the work items (see the kernel): blocks of B
  // items, B a multiple of the head groups
  const int nhg = a.n_heads / kHeads;
  const int64_t total = (int64_t)a.n_split * a.n_rows * nhg;
  if (total > (int64_t)1 << 30) return hipErrorInvalidValue;
  AttnArgs k = a;
  k.xcd_block = (int32_t)(((total + 7) / 8 + nhg - 1) / nhg * nhg);
  hipLaunchKernelGGL(sparse_attn_narrow_kernel, dim3((unsigned)(8 * k.xcd_block)), dim3(kThreads),
                     sizeof(NarrowShared), stream, k);
  return hipGetLastError();
}

}  // namespace csa2
