// Joint sparse + sliding-window attention for many rows: 64 heads per
// workgroup, MFMA 32x32x16 tiles [daiw "four factors" table: one 512-dim
// latent shared by all query heads (K = V); 0539edu §3: top_k 512,
// 128-token FP8 window].
//
// Same mathematics as the other attention kernels.  A workgroup of 8 waves
// owns (row, 64 heads, a range of keys) and walks it in chunks of 32 keys
// through a four-stage pipeline, one barrier per step; chunk c is
//   * written at step c by 2 dequantising waves, which gather the selected
//     FP4 entries (256 code + 32 E4M3 scale bytes each) or FP8 window tokens
//     four chunks ahead and write them exactly, as fp16, into one key-major
//     tile (4 tiles in rotation);
//   * multiplied at step c + 1 by 2 score waves, one per 32-head tile:
//     S^T[key][head] = K Q^T (v_mfma_f32_32x32x16_f16, Q held in registers);
//   * turned into probabilities at step c + 2 by the same waves (the online
//     softmax runs between the MFMAs of the next chunk), which hand P (one
//     fp16 term) and the per-head rescale factor over through LDS;
//   * accumulated at step c + 3 by 4 output waves: O^T[channel][head] +=
//     K^T P^T (128 channels and both head tiles each), reading K^T with the
//     LDS transpose read.
// Exactness: every E2M1 x E4M3 product and every E4M3 value is an fp16 value.
// The bf16 queries are scaled per head by a power of two that puts their
// largest magnitude in [2^14, 2^15) and converted to fp16: exact except for
// elements more than 2^29 times smaller than the head's largest, whose
// rounding changes a score by less than float32 rounding of the sum; the
// power of two is folded into the softmax scale.  P enters the PV product as
// one fp16 term (11 significant bits) and the normaliser sums exactly the
// weights the product sees.  The score tile's lane layout (head = lane % 32,
// keys 16s + 8(i/4) + 4(lane/32) + i%4 for register 8s + i) is taken as the
// k-slot order of the PV product, so a score lane's P registers are the PV
// operand of the same lane: P goes through LDS lane-major, and the K^T
// operand is read with the same key order.
#include "attn_dev.h"
#include "csa2_launch.h"

namespace csa2 {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTChunk = 32;                    // keys per chunk
constexpr int kTRow = kD * 2;                  // bytes of one fp16 key row
constexpr int kTThreads = 512;
constexpr int kTHeads = 64;                    // heads per workgroup (2 tiles of 32)
constexpr int kTMaxKeys = 1024;                // selected ids staged per workgroup
constexpr int kTTiles = 4;                     // key tiles in rotation
constexpr float kTSlack = 8.0f;                // log2 growth of the max tolerated before rescaling

struct __align__(16) TileShared {
  uint8_t k[kTTiles][kTChunk * kTRow];         // fp16 key tiles, rows swizzled in 16-byte segments
  uint8_t p[2][2][2 * 64 * 16];                // P per (buffer, head tile): [k-step][lane], 8 fp16 each
  float bias[kTTiles][kTChunk];                // per key of a tile: 0 if it takes part, -inf if not
  float alpha[2][kTHeads];                     // per-head rescale factor of a chunk
  float lsum[kTHeads];
  int32_t sidx[kTMaxKeys];
};

// The swizzle of a key row: 16-byte segment s of row r sits at s ^ tsw(r).
// tsw is a bijection of the row's low four bits (bit 0 of r -> 4, bit 1 -> 10,
// bit 2 -> 1, bit 3 -> 2 under XOR) chosen so that every LDS access of the
// kernel touches distinct banks in each group of lanes served together, for
// 32 or 64 banks of 4 bytes: the score waves' 16-byte reads (16 consecutive
// rows, one segment), the dequantising waves' 16-byte writes (the same) and
// the output waves' transpose reads (4 consecutive rows x 2 or 4 consecutive
// segments).
__device__ __forceinline__ int tsw(int row) {
  return ((row >> 2) & 1) | ((((row >> 1) ^ (row >> 3)) & 1) << 1) | ((row & 1) << 2) | (((row >> 1) & 1) << 3);
}

// The raw bytes one dequantising thread gathers for its key and 128 channels
// of a chunk: a selected entry's 64 code bytes (lo) and 8 scale bytes, or a
// window token's 128 bytes (lo, hi).
struct TGather {
  uint4 lo[4], hi[4];
  uint2 sc;
  int kind;                                    // 0 none, 1 selected entry, 2 window token
};

// The lane halves' values of x combined: both halves get op(x[l mod 32],
// x[l mod 32 + 32]) (v_permlane32_swap hands each half the other's value).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);   // lower half's value first in both halves
}

}  // namespace

__global__ __launch_bounds__(kTThreads, 2) void sparse_attn_tile_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char tile_smem[];
  TileShared& sh = *reinterpret_cast<TileShared*>(tile_smem);
  const int split = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.n_heads;
  const int hbase = blockIdx.z * kTHeads;
  const int h32 = lane >> 5;                   // lane half
  const int l32 = lane & 31;

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
  const int nch = k1 > k0 ? (k1 - k0 + kTChunk - 1) / kTChunk : 0;
  const int nsteps = nch > 0 ? nch + 3 : 0;     // the last chunk is accumulated at step nch + 2

  const int32_t* idxr = a.idx ? a.idx + (int64_t)r * a.top_k : nullptr;
  const uint8_t* codes_s = a.codes + (seq_ok ? seq : 0) * a.n_ent * (kD / 2);
  const uint8_t* scales_s = a.scales + (seq_ok ? seq : 0) * a.n_ent * (kD / kGroup);
  const uint8_t* swa_s = a.swa ? a.swa + (seq_ok ? seq : 0) * (int64_t)a.swa_cap * kD : nullptr;
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.q + (int64_t)r * H * kD);   // readable, discarded

  const int nst = max(0, min(k0 + a.keys_per_split, a.top_k) - k0);
  for (int i = tid; i < nst; i += kTThreads) sh.sidx[i] = idxr[k0 + i];

  const bool qk_wave = wave < 2, pv_wave = wave == 2 || wave == 3 || wave == 6 || wave == 7;
  const int pw = wave == 2 ? 0 : wave == 3 ? 1 : wave == 6 ? 2 : 3;   // output wave index: channels 128pw..
  const int dq = tid - 256;                    // dequantising thread 0..127 (waves 4, 5)
  // its key of the chunk and channel quarter: 16 consecutive keys per group
  // of 16 lanes (distinct LDS banks for the tile writes)
  const int dq_key = 16 * (dq >> 6) + (dq & 15), dq_q = (dq >> 4) & 3;

  // per-role state (each role touches only its own)
  uint4 qreg[kD / 16];                         // score waves: Q of the lane's head, fp16 pairs
  float qscale = 0.0f;                         // sm_scale * log2(e) * 2^e of the lane's head
  float m_run = -INFINITY, l_run = 0.0f;       // in log2 units of the scaled scores
  v16f acc[4][2];                              // output waves: O^T tiles

  lds_barrier();                               // sidx staged
  __builtin_amdgcn_s_waitcnt(0);               // and the id loads retired

  // ---- dequantising waves: gather (issue) and write one chunk.  The scale
  // word is loaded first and every gather issues the same nine loads (out of
  // range: a readable dummy), so the wait before a chunk's use leaves the
  // younger chunks' loads in flight.
  auto gather = [&](int c, TGather& G) __attribute__((always_inline)) {
    const int key = k0 + c * kTChunk + dq_key;
    const bool in_range = key < k1;
    const bool is_sel = in_range && key < nsel;
    const int32_t p = is_sel ? sh.sidx[min(max(key - k0, 0), kTMaxKeys - 1)] : -1;
    const bool ok = is_sel && p >= 0 && (int64_t)p < a.n_ent;
    const bool is_swa = in_range && !is_sel;
    int slot = swst + (key - nsel);
    if (slot >= a.swa_cap) slot -= a.swa_cap;
    const uint8_t* wa = is_swa ? swa_s + (int64_t)slot * kD + 128 * dq_q : dummy;
    const uint8_t* la = ok ? codes_s + (int64_t)p * (kD / 2) + 64 * dq_q : wa;
    const uint8_t* ha = is_swa ? wa + 64 : dummy;
    const uint8_t* sa = ok ? scales_s + (int64_t)p * (kD / kGroup) + 8 * dq_q : dummy;
    G.sc = *reinterpret_cast<const uint2*>(sa);
#pragma unroll
    for (int i = 0; i < 4; ++i) G.lo[i] = *reinterpret_cast<const uint4*>(la + 16 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) G.hi[i] = *reinterpret_cast<const uint4*>(ha + 16 * i);
    G.kind = ok ? 1 : (is_swa ? 2 : 0);
  };
  // 16-byte segment 16*dq_q + j of the thread's key row holds channels
  // 128*dq_q + 8j .. +7; one branch per key (a chunk is all selected entries
  // or all window tokens but at one boundary)
  auto dequant = [&](const TGather& G, int buf) __attribute__((always_inline)) {
    uint8_t* trow = sh.k[buf] + dq_key * kTRow + 256 * dq_q;
    const int x = tsw(dq_key);                 // segment 16*dq_q + j sits at 16*dq_q + (j ^ x)
    if (G.kind == 1) {
      // the eight group scales as fp16 (every E4M3 value is one), two per word
      const v2h sp[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(G.sc.x, 1.0f, false),
                         __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(G.sc.x, 1.0f, true),
                         __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(G.sc.y, 1.0f, false),
                         __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(G.sc.y, 1.0f, true)};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint4 q = G.lo[j >> 2];
        const uint32_t w = (j & 2) ? ((j & 1) ? q.w : q.z) : ((j & 1) ? q.y : q.x);
        const _Float16 sv = sp[j >> 2][(j >> 1) & 1];      // group j / 2
        const v2h s2 = v2h{sv, sv};
        const v2h c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
        const v2h c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
        const v2h c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
        const v2h c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
        *reinterpret_cast<uint4*>(trow + 16 * (j ^ x)) =
            make_uint4(__builtin_bit_cast(uint32_t, c0), __builtin_bit_cast(uint32_t, c1),
                       __builtin_bit_cast(uint32_t, c2), __builtin_bit_cast(uint32_t, c3));
      }
    } else if (G.kind == 2) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint4 s8 = (j < 8) ? G.lo[j >> 1] : G.hi[(j - 8) >> 1];
        const uint32_t w0 = (j & 1) ? s8.z : s8.x, w1 = (j & 1) ? s8.w : s8.y;
        const v2h c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
        const v2h c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
        const v2h c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
        const v2h c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
        *reinterpret_cast<uint4*>(trow + 16 * (j ^ x)) =
            make_uint4(__builtin_bit_cast(uint32_t, c0), __builtin_bit_cast(uint32_t, c1),
                       __builtin_bit_cast(uint32_t, c2), __builtin_bit_cast(uint32_t, c3));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) *reinterpret_cast<uint4*>(trow + 16 * j) = make_uint4(0u, 0u, 0u, 0u);
    }
    if (dq_q == 0) sh.bias[buf][dq_key] = G.kind != 0 ? 0.0f : -INFINITY;
  };

  // ---- score waves.  qk: S^T of the chunk in tile `tile` (raw dot products;
  // lane: head l32, keys 8(v/4) + 4*h32 + v%4 of register v).
  // The A operand of k-step ks = 4a + b is segment 8a + 2b + h32 of key row
  // l32, at 8(a ^ x3) + ((2b + h32) ^ xl) with x = tsw(l32), x3 = x >> 3,
  // xl = x & 7; 8(a ^ x3) = 8a + 8x3 for even a and 8a - 8x3 for odd a, so the
  // byte offset is qk_off[b][a & 1] + 128a: eight lane bases and immediates.
  int qk_off[4][2];
  {
    const int x = tsw(l32);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int base = l32 * kTRow + 16 * ((2 * b + h32) ^ (x & 7));
      qk_off[b][0] = base + 128 * (x >> 3);
      qk_off[b][1] = base - 128 * (x >> 3);
    }
  }
  auto qk = [&](int tile, v16f& S) __attribute__((always_inline)) {
    const uint8_t* t = sh.k[tile];
    S = v16f{};
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      const v8h ka = *reinterpret_cast<const v8h*>(t + qk_off[ks & 3][(ks >> 2) & 1] + 128 * (ks >> 2));
      S = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, __builtin_bit_cast(v8h, qreg[ks]), S, 0, 0, 0);
    }
  };
  // softmax: the online softmax step of chunk c from its S; P into P buffer
  // c & 1, the rescale factor of the chunk into alpha[c & 1]
  auto softmax = [&](int c, const v16f& S) __attribute__((always_inline)) {
    const float* bb = sh.bias[c & (kTTiles - 1)] + 4 * h32;
    float t[16];
    float cmax = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 b4 = *reinterpret_cast<const float4*>(bb + 8 * g);   // keys 8g + 4*h32 .. +3
      const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        t[4 * g + i] = fmaf(S[4 * g + i], qscale, bv[i]);
        cmax = fmaxf(cmax, t[4 * g + i]);
      }
    }
    cmax = halves_max(cmax);
    // the reference max moves only when the chunk's max exceeds it by more
    // than the slack (weights stay below 2^slack, well inside fp16)
    // (branch-free: alpha = 2^(m_run - m_new), 0 from -inf, 1 while no key
    // has come)
    const bool move = cmax > m_run + kTSlack;
    const float m_new = move ? cmax : m_run;
    const bool none = m_new == -INFINITY;
    const float alpha = __builtin_amdgcn_exp2f(none ? 0.0f : m_run - m_new);
    m_run = m_new;
    const float msub = none ? 0.0f : m_new;    // no key yet: every t is -inf, every weight 0
    uint32_t ph[8];
    float psum = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const v2h h = v2h{(_Float16)__builtin_amdgcn_exp2f(t[v] - msub), (_Float16)__builtin_amdgcn_exp2f(t[v + 1] - msub)};
      psum = __builtin_amdgcn_fdot2(h, v2h{(_Float16)1.0f, (_Float16)1.0f}, psum, false);   // the weights as the product sees them
      ph[v >> 1] = __builtin_bit_cast(uint32_t, h);
    }
    l_run = l_run * alpha + halves_sum(psum);
    uint8_t* pr = sh.p[c & 1][wave] + lane * 16;
    *reinterpret_cast<uint4*>(pr) = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    *reinterpret_cast<uint4*>(pr + 1024) = make_uint4(ph[4], ph[5], ph[6], ph[7]);
    sh.alpha[c & 1][32 * wave + l32] = alpha;  // both halves store the same value
  };
  // One step of the steady state: S of chunk c into Snew while the softmax of
  // chunk c - 1 (the same arithmetic as softmax()) runs from Sold.  The MFMAs
  // form one dependent chain and a wave waits at each for the one before, so
  // the softmax is cut into small pieces placed one after each MFMA (fenced
  // against reordering), where they issue while it runs; the K operand is
  // read four MFMAs ahead.
  auto qk_softmax = [&](int c, v16f& Snew, const v16f& Sold) __attribute__((always_inline)) {
    const uint8_t* tk = sh.k[c & (kTTiles - 1)];
    const float* bb = sh.bias[(c - 1) & (kTTiles - 1)] + 4 * h32;
    v8h kb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kb[i] = *reinterpret_cast<const v8h*>(tk + qk_off[i][0]);
    float4 b4[4];
    float t[16], e0 = 0.0f;
    float cmax = -INFINITY, alpha = 1.0f, msub = 0.0f, psum = 0.0f;
    uint32_t ph[8];
    Snew = v16f{};
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      Snew = __builtin_amdgcn_mfma_f32_32x32x16_f16(kb[ks & 3], __builtin_bit_cast(v8h, qreg[ks]), Snew, 0, 0, 0);
      if (ks + 4 < kD / 16) {
        const int kn = ks + 4;
        kb[ks & 3] = *reinterpret_cast<const v8h*>(tk + qk_off[kn & 3][(kn >> 2) & 1] + 128 * (kn >> 2));
      }
      if (ks == 0) {
#pragma unroll
        for (int g = 0; g < 4; ++g) b4[g] = *reinterpret_cast<const float4*>(bb + 8 * g);   // keys 8g + 4*h32 ..
      } else if (ks >= 4 && ks < 12) {
        const int v = 2 * (ks - 4);
        const float4 bg = b4[v >> 2];
        t[v] = fmaf(Sold[v], qscale, (v & 2) ? bg.z : bg.x);
        t[v + 1] = fmaf(Sold[v + 1], qscale, (v & 2) ? bg.w : bg.y);
        cmax = fmaxf(cmax, fmaxf(t[v], t[v + 1]));
      } else if (ks == 12) {
        cmax = halves_max(cmax);
      } else if (ks == 13) {
        const bool move = cmax > m_run + kTSlack;
        const float m_new = move ? cmax : m_run;
        const bool none = m_new == -INFINITY;
        alpha = __builtin_amdgcn_exp2f(none ? 0.0f : m_run - m_new);
        m_run = m_new;
        msub = none ? 0.0f : m_new;
      } else if (ks >= 14 && ks < 30) {
        const int v = ks - 14;
        const float e = __builtin_amdgcn_exp2f(t[v] - msub);
        if ((v & 1) == 0) {
          e0 = e;
        } else {
          const v2h h = v2h{(_Float16)e0, (_Float16)e};
          psum = __builtin_amdgcn_fdot2(h, v2h{(_Float16)1.0f, (_Float16)1.0f}, psum, false);
          ph[v >> 1] = __builtin_bit_cast(uint32_t, h);
        }
      } else if (ks == 30) {
        l_run = l_run * alpha + halves_sum(psum);
        uint8_t* pr = sh.p[(c - 1) & 1][wave] + lane * 16;
        *reinterpret_cast<uint4*>(pr) = make_uint4(ph[0], ph[1], ph[2], ph[3]);
        *reinterpret_cast<uint4*>(pr + 1024) = make_uint4(ph[4], ph[5], ph[6], ph[7]);
        sh.alpha[(c - 1) & 1][32 * wave + l32] = alpha;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- output waves: O^T += K^T P^T for chunk (tile buf, P pbuf).
  // Transpose reads: the 16-lane group G = lane/16 reads keys
  // 16s + 8j + 4*(G/2) .. +3 at channels 32*(4pw + ct) + 16*(G%2) .. +15;
  // lane n of the group addresses key row 16s + 8j + row0 (row0 = 4(G/2) +
  // n/4) and the 8 bytes of channels 4*(n%4) .. +3.  The row's swizzle is
  // x = tsw(row0) ^ 2j (tsw is linear over XOR and tsw(8) = 2; 16s does not
  // enter), and the segment 4(4pw + ct) + c' (c' = 2(G%2) + (n%4)/2)
  // swizzles to 16pw + 4(ct ^ (x >> 2)) + (c' ^ (x & 3)): a lane base per
  // (j, ct), plus kTRow * 16s as an immediate.
  int pv_off[2][4];
  {
    const int G = lane >> 4, n = lane & 15;
    const int row0 = 4 * (G >> 1) + (n >> 2);
    const int cq = 2 * (G & 1) + ((n & 3) >> 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int x = tsw(row0) ^ (2 * j);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        pv_off[j][ct] = (row0 + 8 * j) * kTRow + 256 * pw + 64 * (ct ^ (x >> 2)) + 16 * (cq ^ (x & 3)) + 8 * (n & 1);
    }
  }
  auto accumulate = [&](int c) __attribute__((always_inline)) {
    const uint8_t* tile = sh.k[c & (kTTiles - 1)];
    const int pbuf = c & 1;
    // every LDS read of the chunk first, then the rescale check
    const float al0 = sh.alpha[pbuf][l32], al1 = sh.alpha[pbuf][32 + l32];
    v8h pb[2][2];                              // [head tile][k-step]
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const uint8_t* pr = sh.p[pbuf][ht] + lane * 16;
      pb[ht][0] = *reinterpret_cast<const v8h*>(pr);
      pb[ht][1] = *reinterpret_cast<const v8h*>(pr + 1024);
    }
    v8h ka[4][2];                              // [channel tile][k-step]
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v4s part[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          part[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(tile + pv_off[j][ct] + kTRow * 16 * s));
        const uint2 lo = __builtin_bit_cast(uint2, part[0]), hi = __builtin_bit_cast(uint2, part[1]);
        ka[ct][s] = __builtin_bit_cast(v8h, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
    }
    if (__builtin_amdgcn_ballot_w64(al0 != 1.0f || al1 != 1.0f)) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        acc[ct][0] *= al0;
        acc[ct][1] *= al1;
      }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        acc[ct][ht] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ct][0], pb[ht][0], acc[ct][ht], 0, 0, 0);
        acc[ct][ht] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ct][1], pb[ht][1], acc[ct][ht], 0, 0, 0);
      }
  };

  // ---- the pipeline, one barrier per step.  Each role runs its own loop
  // (the roles are whole waves, and every wave passes the same nsteps + 1
  // barriers), so the registers of one role's state are free for the
  // others'.
  const int64_t rh0 = (int64_t)r * H + hbase;
  if (qk_wave) {
    // the score wave shares its SIMD with a dequantising wave: issuing at a
    // raised priority keeps its dependent MFMA chain from waiting behind
    // the other wave's vector instructions
    __builtin_amdgcn_s_setprio(3);
    // score waves: Q of head tile `wave` (head 32*wave + l32), channels
    // 16ks + 8*h32 .. +8 for ks < 32, scaled by a power of two into fp16.
    // The tile's 32 rows (32 KB, contiguous) come in with one 1 KB row per
    // load and pass through key tile 2 + wave (first written at step 2):
    // row t's 16-byte block l at block l ^ tsw(t).
    {
      const int hq = hbase + 32 * wave + l32;
      const bool hok = hq < H;
      const int nrow = min(32, H - (hbase + 32 * wave));
      const uint16_t* qsrc = a.q + ((int64_t)r * H + hbase + 32 * wave) * kD + 8 * lane;
      uint8_t* qs = sh.k[2 + wave];
#pragma unroll
      for (int t = 0; t < 32; ++t)
        qreg[t] = t < nrow ? *reinterpret_cast<const uint4*>(qsrc + t * kD) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int t = 0; t < 32; ++t) *reinterpret_cast<uint4*>(qs + t * kTRow + 16 * (lane ^ tsw(t))) = qreg[t];
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks)
        qreg[ks] = *reinterpret_cast<const uint4*>(qs + l32 * kTRow + 16 * ((2 * ks + h32) ^ tsw(l32)));
      // the largest magnitude from the bits (finite bf16: the order of the
      // magnitude bits is the order of the magnitudes)
      uint32_t mbits = 0u;
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const uint32_t w4[4] = {qreg[ks].x, qreg[ks].y, qreg[ks].z, qreg[ks].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) mbits = max(mbits, max(w4[i] & 0x7FFFu, (w4[i] >> 16) & 0x7FFFu));
      }
      float amax = bf16_to_f32(mbits);
      amax = fmaxf(amax, __shfl_xor(amax, 32));  // the head's other half
      int ex = 0;
      if (amax > 0.0f) { (void)frexpf(amax, &ex); ex -= 15; }   // amax * 2^-ex in [2^14, 2^15)
      const float sc = ldexpf(1.0f, -ex);
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {     // converted in place: bf16 pairs -> fp16 pairs
        const uint32_t w4[4] = {qreg[ks].x, qreg[ks].y, qreg[ks].z, qreg[ks].w};
        uint32_t o4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const _Float16 lo = (_Float16)(bf16_to_f32(w4[i] & 0xFFFFu) * sc);
          const _Float16 hi = (_Float16)(bf16_to_f32(w4[i] >> 16) * sc);
          o4[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        qreg[ks] = hok ? make_uint4(o4[0], o4[1], o4[2], o4[3]) : make_uint4(0u, 0u, 0u, 0u);
      }
      qscale = a.sm_scale_log2 * ldexpf(1.0f, ex);
    }



    // step 0: chunk 0 written; step 1: its S; step c + 1 (1 <= c < nch): S of
    // chunk c between the softmax of chunk c - 1; then the last softmax and
    // one idle step
    if (nsteps > 0) {
      v16f Sa, Sb;
      lds_barrier();
      qk(0, Sa);
      lds_barrier();
      int c = 1;
#pragma unroll 1
      for (;;) {
        if (c >= nch) { softmax(c - 1, Sa); lds_barrier(); lds_barrier(); break; }
        qk_softmax(c, Sb, Sa);
        lds_barrier();
        ++c;
        if (c >= nch) { softmax(c - 1, Sb); lds_barrier(); lds_barrier(); break; }
        qk_softmax(c, Sa, Sb);
        lds_barrier();
        ++c;
      }
    }
    // each head's sum to the output waves; the log-sum-exp or the split's (max, sum)
    if (h32 == 0) {
      sh.lsum[32 * wave + l32] = l_run;
      const int hq = hbase + 32 * wave + l32;
      if (hq < H) {
        if (a.n_split == 1) {
          if (a.lse) a.lse[rh0 + 32 * wave + l32] = l_run > 0.0f ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
        } else {
          const int64_t base = (int64_t)split * a.n_rows * H + rh0 + 32 * wave + l32;
          a.part_ml[base * 2] = m_run;
          a.part_ml[base * 2 + 1] = l_run;
        }
      }
    }
    lds_barrier();
  } else if (pv_wave) {
    // O^T tiles (channel tile 4pw + ct, head tile ht)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) acc[ct][ht] = v16f{};
#pragma unroll 1
    for (int i = 0; i < nsteps; ++i) {
      if (i >= 3) accumulate(i - 3);
      lds_barrier();
    }
    lds_barrier();                             // the sums are in LDS
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int hq = hbase + 32 * ht + l32;
      if (hq >= H) continue;
      const float l = sh.lsum[32 * ht + l32];
      const float inv = a.n_split == 1 ? (l > 0.0f ? 1.0f / l : 0.0f) : 1.0f;
      float* orow = a.n_split == 1 ? a.out + (rh0 + 32 * ht + l32) * kD
                                   : a.part_o + ((int64_t)split * a.n_rows * H + rh0 + 32 * ht + l32) * kD;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int cbase = 32 * (4 * pw + ct) + 4 * h32;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const v16f& o = acc[ct][ht];
          *reinterpret_cast<float4*>(orow + cbase + 8 * q4) =
              make_float4(o[4 * q4] * inv, o[4 * q4 + 1] * inv, o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv);
        }
      }
    }
  } else {
    // dequantising waves: chunk i is gathered four steps ahead into set
    // i % 4 and written into tile i % 4 at step i.  The loop is unrolled by
    // four so that the sets stay in registers; it leaves by a break after any
    // step, so every path back to its head has issued the four sets in order.
    TGather G0, G1, G2, G3;
    if (nsteps > 0) {
      gather(0, G0);
      gather(1, G1);
      gather(2, G2);
      gather(3, G3);
    }
    auto step = [&](int i, TGather& G, int buf) __attribute__((always_inline)) {
      if (i < nch) dequant(G, buf);
      gather(i + 4, G);
      lds_barrier();
    };
#pragma unroll 1
    for (int i = 0;; i += 4) {
      if (i >= nsteps) break;
      step(i, G0, 0);
      if (i + 1 >= nsteps) break;
      step(i + 1, G1, 1);
      if (i + 2 >= nsteps) break;
      step(i + 2, G2, 2);
      if (i + 3 >= nsteps) break;
      step(i + 3, G3, 3);
    }
    lds_barrier();
    __builtin_amdgcn_s_waitcnt(0);             // the trailing (dummy) gathers retired
  }
}

hipError_t launch_sparse_attn_tile(const AttnArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  if (a.keys_per_split > kTMaxKeys) return hipErrorInvalidValue;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&sparse_attn_tile_kernel),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)sizeof(TileShared));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(sparse_attn_tile_kernel,
                     dim3((unsigned)a.n_split, (unsigned)a.n_rows, (unsigned)((a.n_heads + kTHeads - 1) / kTHeads)),
                     dim3(kTThreads), sizeof(TileShared), stream, a);
  return hipGetLastError();
}

}  // namespace csa2
