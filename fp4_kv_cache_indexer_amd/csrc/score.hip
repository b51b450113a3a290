// Sparse indexer scores [0539edu §3: csa2.indexer (32 heads x 128) and its
// hierarchical block (2048 blocks x 8 positions)].
//
//   I_t = sum_h w_h * max(0, q_h . k_t), q/k FP8 E4M3, float32 accumulation.
//   The 128-byte keys stream straight from HBM into registers, are widened
//   to fp16 there (exact: every E4M3 value is an fp16 value) and meet the
//   queries in v_mfma_f32_16x16x32_f16, [32 heads x 128] x [128 x 16 entries]
//   per 8 MFMAs; the head reduction runs in the epilogue.  (gfx950's fp8
//   MFMAs were measured to sum their products with less than float32
//   precision -- up to ~1e-3 relative on heavy-tailed data -- which is as
//   wide as the top-k tie band; the fp16 MFMA matches a float32 FMA chain.)
//   Each workgroup also histograms the top 12 bits of the order key of its
//   scores in LDS and folds that into a per-row histogram for the top-k.
#include "append_dev.h"
#include "csa2_dev.h"
#include "csa2_launch.h"
#include "items.h"

namespace csa2 {

// ---------------------------------------------------------------------------
// score kernel
// ---------------------------------------------------------------------------

#ifndef CSA2_SCORE_TILES
#define CSA2_SCORE_TILES 4
#endif
#ifndef CSA2_SCORE_MINW
#define CSA2_SCORE_MINW 2
#endif
constexpr int kScoreThreads = 256;
constexpr int kScoreWaves = kScoreThreads / 64;
constexpr int kTilesPerIter = CSA2_SCORE_TILES;   // 16-item tiles per group
// Chosen by measurement on the 8 x 131072-block coarse scan: double-buffered
// groups of 4 tiles, register budget for 2 waves per SIMD (28.7 us vs
// 29.8-37 us for the single-buffered, larger-group and tighter-budget forms).
constexpr bool kScoreDB = true;
constexpr int kScoreMinW = CSA2_SCORE_MINW;
// Chunks of at most this many items stage their scores in LDS and write them
// in one coalesced pass at the end (measured 0.5-1.3 us less on the C3
// coarse scan than stores interleaved with the key stream); longer chunks
// store as they go.
constexpr int kScoreStage = 2048;

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Non-temporal variants for keys that are streamed once: the summary scan
// and the pool scan of the hierarchical indexer read faster with them; the
// flat scan over many sequences reads slower, and keeps the plain loads.
typedef unsigned int u4nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_nt(const uint8_t* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u4nt*>(p)));
}
template <bool NT>
__device__ __forceinline__ v8i load32k(const uint8_t* p) {
  const uint4 a = NT ? load16_nt(p) : *reinterpret_cast<const uint4*>(p);
  const uint4 b = NT ? load16_nt(p + 16) : *reinterpret_cast<const uint4*>(p + 16);
  v8i v;
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  return v;
}

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  v8i v;
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  return v;
}

// 8 FP4 channels (one word, channel 2j in the low nibble of byte j) times
// their E4M3 scale, as fp16: the unit-scale hardware decode is exact and the
// product has at most 6 significant bits within [2^-10, 2688], so it is exact.
__device__ __forceinline__ v8h fp4x8_to_f16(uint32_t w, _Float16 s) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  const v8h v = v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return v * s;
}

// 8 E4M3 bytes (two words, byte order = element order) widened to fp16.
__device__ __forceinline__ v8h fp8x8_to_f16(int w0, int w1) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w0, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w0, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w1, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w1, 1.0f, true);
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// max(0, x) on the bits (a negative float is a negative integer): one
// integer max, where a float max first quiets a NaN operand in an extra
// instruction.  -0 becomes +0.
__device__ __forceinline__ float relu0(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Sums across 16-lane rows without LDS: rows 0..3 of the result hold
// x.r0 + x.r1, y.r0 + y.r1, x.r2 + x.r3, y.r2 + y.r3 (one row swap between
// the operands, then one add).
__device__ __forceinline__ float row_pair_sum(float x, float y) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// ... and across the wave's halves: the lower half holds x.lo + x.hi, the
// upper half y.lo + y.hi.
__device__ __forceinline__ float half_pair_sum(float x, float y) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Adds a workgroup's LDS histogram (kHistBins counts, 8-byte aligned) into
// the row's histogram in memory: two adjacent bins per 64-bit atomic add
// (the low word is the even bin; no count reaches 2^32, so no carry crosses
// into the odd one), half the atomics of one per bin, for the pairs that
// counted anything.  Every workgroup of a row adds into the same words.
__device__ __forceinline__ void flush_hist(const uint32_t* lh, uint32_t* gh) {
  unsigned long long* g2 = reinterpret_cast<unsigned long long*>(gh);
  for (int b = threadIdx.x; b < kHistBins / 2; b += blockDim.x) {
    const uint2 c = *reinterpret_cast<const uint2*>(lh + 2 * b);
    if (c.x | c.y) atomicAdd(g2 + b, ((unsigned long long)c.y << 32) | c.x);
  }
}

// The append of one row inside the coarse scan's launch (its last column),
// for the (m, gate) forms a decode step uses.
__device__ __forceinline__ void fused_append_row(const AppendArgs& ap, int r, int t) {
  if (ap.m == 1) {
    if (ap.key_fp4) decode_append_row<1, false, 1>(ap, r, t); else decode_append_row<1, false, 0>(ap, r, t);
  } else if (ap.gate) {
    if (ap.key_fp4) decode_append_row<2, true, 1>(ap, r, t); else decode_append_row<2, true, 0>(ap, r, t);
  } else {
    if (ap.key_fp4) decode_append_row<2, false, 1>(ap, r, t); else decode_append_row<2, false, 0>(ap, r, t);
  }
}

// The refreshed summary of the block of entry e (sequence s) by lanes 0..31
// of wave 0, 4 channels each, into sp_key (bytes 4t..4t+3).
__device__ __forceinline__ void fused_block_summary(const AppendArgs& ap, int r, int64_t s, int64_t e,
                                                    uint8_t* sp_key) {
  const int t = threadIdx.x;
  if (t >= 32) return;
  uint32_t old_w[kBlockPos - 1], old_s[kBlockPos - 1];
  const int cnt = (int)(e - (e / kBlockPos) * kBlockPos) + 1;
  uint32_t out;
  if (ap.key_fp4) {
    append_members4<1>(ap, s, e, t, old_w, old_s);
    out = append_summary4<1>(old_w, old_s, cnt, append_key4<1>(ap.key + (int64_t)r * kIdxDim, t));
  } else {
    append_members4<0>(ap, s, e, t, old_w, old_s);
    out = append_summary4<0>(old_w, old_s, cnt, append_key4<0>(ap.key + (int64_t)r * kIdxDim, t));
  }
  *reinterpret_cast<uint32_t*>(sp_key + 4 * t) = out;
}

// DB: double-buffer the tile groups of a wave; MINW: waves per SIMD the
// register budget must allow.
// G > 0: the chunk is exactly G groups per wave and the group loop is fully
// unrolled (straight-line code lets the compiler keep the next group's loads
// in flight exactly); G == 0: runtime trip count.
// KF: key format, 0 = E4M3 (128 B per key), 1 = FP4 (64 B of codes + a
// 4-byte word of E4M3 scales, one per 32 channels).
// APP: the coarse stage of a decode step, which also runs the step's append
// (see ScoreArgs::fuse_append).
template <int MODE, int KF = 0, bool DB = false, int MINW = 4, int U = kTilesPerIter, int G = 0, bool APP = false>
__global__ __launch_bounds__(kScoreThreads, MINW) void index_score_kernel(ScoreArgs a) {
  a.im.mode = MODE;                              // lets the item mapping fold away
  // Block summaries (the long, HBM-bound coarse scan) are read in whole
  // cache lines and staged through LDS; the short gathers of the other
  // modes read straight into the operand layout (the staging's LDS round
  // trip costs them more than the halved line requests save).
  constexpr bool FULL = !KF && MODE == kItemsBlocks;
  // the histogram and the staged scores, each followed by one word per
  // thread for the lanes that count or stage nothing (no branch)
  __shared__ __align__(8) uint32_t hist[kHistBins + kScoreThreads];
  __shared__ float sscore[kScoreStage + kScoreThreads];
  __shared__ __align__(16) uint8_t sp_key[APP ? kIdxDim : 16];
  // staged keys pass through a wave-private buffer of two 16-key tiles
  __shared__ __align__(16) uint8_t kstage[FULL ? kScoreWaves * 2 * 16 * kIdxDim : 16];
  const int r = blockIdx.y;
  if (APP && blockIdx.x == gridDim.x - 1) {      // uniform: the row's append
    fused_append_row(a.app, r, threadIdx.x);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int32_t c0 = (int32_t)blockIdx.x * a.chunk;
  // Pool and candidate items are looked up in the row's list.  The first
  // group's lookups go out before the row's sequence and count are known
  // (clamped to the row's items, unconditional), so the two round trips
  // overlap.
  constexpr bool LIST = MODE == kItemsPool || MODE == kItemsCand;
  const int32_t* lrow = LIST ? a.im.list + (int64_t)r * a.im.list_len : nullptr;
  int32_t le0[U];
  if (LIST) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t ic = min(c0 + (wave * U + u) * 16 + n, a.im.n_items - 1);
      le0[u] = lrow[MODE == kItemsPool ? ic >> 3 : ic];
    }
  }
  int64_t seq;
  const int64_t nv = row_valid(a.im, r, &seq);
  // items stay below kMaxItems (2^24) per row: 32-bit item arithmetic
  const int32_t n_row = (int32_t)row_items(a.im, nv);
  if (c0 >= n_row) {                             // uniform for the workgroup
    if (LIST) {                                  // the lookups stay above the branch
#pragma unroll
      for (int u = 0; u < U; ++u) asm volatile("" ::"v"(le0[u]));
    }
    return;
  }
  const int32_t c1 = min(c0 + a.chunk, n_row);
  const bool stage = c1 - c0 <= kScoreStage;     // uniform
  // the block whose summary the row's append refreshes, when this chunk
  // holds it: scored from its new summary, recomputed here
  int32_t sp = -1;
  if (APP && a.app.block_keys) {
    int64_t aseq;
    const int64_t e = append_entry(a.app, r, aseq);
    if (e >= 0 && e / kBlockPos >= c0 && e / kBlockPos < c1) {
      sp = (int32_t)(e / kBlockPos);
      fused_block_summary(a.app, r, aseq, e, sp_key);   // ordered before the scoring by the barrier below
    }
  }

  // lane (n, g) owns channels 32g .. 32g+31 of key n: 32 E4M3 bytes, or 16
  // FP4 code bytes and the scale word (byte g)
  constexpr int kKeyBytes = KF ? kIdxDim / 2 : kIdxDim;
  const uint8_t* kbase = a.keys + seq * a.seq_rows * kKeyBytes + g * (KF ? 16 : 32);
  const uint8_t* krow = a.keys + seq * a.seq_rows * kKeyBytes;
  const uint8_t* sbase = KF ? a.key_scales + seq * a.seq_rows * 4 : nullptr;

  // MFMA A operands: indexer query rows n and 16+n, bytes [32g, 32g+32), as
  // four fp16 k-slices of 8.  The B operand (keys) uses the same byte split,
  // so each lane's query bytes meet the same key bytes and the four MFMAs
  // together form the full 128-term dot product.
  // The query and weight loads are issued first, then the first key group's,
  // and only then is the query converted (waiting for its own loads alone),
  // so the key stream starts without waiting a memory round trip.
  const uint8_t* qr = a.q + (int64_t)r * kIdxHeads * kIdxDim + g * 32;
  const v8i q0 = load32(qr + n * kIdxDim);
  const v8i q1 = load32(qr + (16 + n) * kIdxDim);
  float w0[4], w1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w0[i] = a.w ? a.w[r * kIdxHeads + 4 * g + i] : 1.0f;
    w1[i] = a.w ? a.w[r * kIdxHeads + 16 + 4 * g + i] : 1.0f;
  }
  float* srow = a.scores + (int64_t)r * a.row_stride;
  v8h qa0[4], qa1[4];                            // converted after the first key loads

  // A wave works on groups of U tiles of 16 items (U a multiple of 4).
  // Loads are unconditional (an invisible item reads a visible row and its
  // score is masked when written).
  const int32_t ntiles = (c1 - c0 + 15) / 16;
  const int32_t gstride = kScoreWaves * U;
  // Later groups' lookups are likewise issued together before any of their
  // key loads, so a group costs one lookup round trip -- a lookup behind a
  // branch, or after the previous tile's key loads, would wait for every
  // load issued before it.  Invisible list items read position 0.
  const int32_t safe_pos = LIST ? 0 : c0;
  auto load_group = [&](int32_t t0, v8i* kb, int32_t* pos, const int32_t* pre) {
    if (LIST) {
      int32_t le[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t ic = min(c0 + (t0 + u) * 16 + n, c1 - 1);
        le[u] = pre ? pre[u] : lrow[MODE == kItemsPool ? ic >> 3 : ic];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t item = c0 + (t0 + u) * 16 + n;
        const int64_t pp = MODE == kItemsPool ? (int64_t)le[u] * kBlockPos + (item & 7) : (int64_t)le[u];
        pos[u] = (item < c1 && le[u] >= 0 && pp < nv) ? (int32_t)pp : -1;
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t item = c0 + (t0 + u) * 16 + n;
        pos[u] = (item < c1) ? (int32_t)item_pos(a.im, r, item, nv) : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t p = (uint32_t)(pos[u] >= 0 ? pos[u] : safe_pos);
      if (KF) {
        constexpr bool NT = MODE != 0;
        const uint4 c = NT ? load16_nt(kbase + p * kKeyBytes) : *reinterpret_cast<const uint4*>(kbase + p * kKeyBytes);
        kb[u][0] = c.x; kb[u][1] = c.y; kb[u][2] = c.z; kb[u][3] = c.w;
        kb[u][4] = NT ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(sbase + p * 4))
                      : *reinterpret_cast<const uint32_t*>(sbase + p * 4);
      } else if (!FULL) {
        kb[u] = load32k<MODE != 0>(kbase + p * kKeyBytes);
      } else {
        // each load instruction reads 8 whole keys (lane L: key 8j + L / 8
        // of the tile, bytes 16 (L % 8)), one request per cache line
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int32_t it = c0 + (t0 + u) * 16 + 8 * j + (lane >> 3);
          const int32_t ps = it < c1 ? (int32_t)item_pos(a.im, r, it, nv) : -1;
          const uint64_t pj = (uint32_t)(ps >= 0 ? ps : safe_pos);
          const uint8_t* src = krow + pj * kIdxDim + 16 * (lane & 7);
          const uint4 c = MODE != 0 ? load16_nt(src) : *reinterpret_cast<const uint4*>(src);
          kb[u][4 * j] = c.x; kb[u][4 * j + 1] = c.y; kb[u][4 * j + 2] = c.z; kb[u][4 * j + 3] = c.w;
        }
      }
    }
  };
  // the loaded tiles into the operand layout (lane (n, g): bytes 32g .. +31
  // of key n), two at a time through the wave's buffer; key k's 16-byte
  // segment s sits at s ^ (k & 7) ^ ((k >> 3) & 1), so the writes (two keys
  // per 16 lanes) and the reads (16 keys, one segment) touch distinct banks.
  // The wave's own LDS accesses complete in order: no barrier.
  uint8_t* kst = kstage + (FULL ? wave * 2 * 16 * kIdxDim : 0);
  auto stage_group = [&](v8i* kb) {
#pragma unroll
    for (int h = 0; h < U; h += 2) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int kk = 8 * j + (lane >> 3);
          const int seg = (lane & 7) ^ (kk & 7) ^ ((kk >> 3) & 1);
          *reinterpret_cast<uint4*>(kst + s2 * 16 * kIdxDim + kk * kIdxDim + 16 * seg) =
              make_uint4(kb[h + s2][4 * j], kb[h + s2][4 * j + 1], kb[h + s2][4 * j + 2], kb[h + s2][4 * j + 3]);
        }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int sl = (2 * g) ^ (n & 7) ^ ((n >> 3) & 1), sh = (2 * g + 1) ^ (n & 7) ^ ((n >> 3) & 1);
        const uint4 lo = *reinterpret_cast<const uint4*>(kst + s2 * 16 * kIdxDim + n * kIdxDim + 16 * sl);
        const uint4 hi = *reinterpret_cast<const uint4*>(kst + s2 * 16 * kIdxDim + n * kIdxDim + 16 * sh);
        kb[h + s2] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
  };
  // a store at an offset past the row's buffer is dropped by the hardware
  const auto srows = __builtin_amdgcn_make_buffer_rsrc(srow, 0, (int)((int64_t)n_row * 4), 0x00020000);
  auto compute_group = [&](int32_t t0, v8i* kb, const int32_t* pos) {
    if (FULL) stage_group(kb);
    if (APP && sp >= 0) {                        // uniform: the refreshed block's key from LDS
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c0 + (t0 + u) * 16 + n == sp) {
          const uint4 lo = *reinterpret_cast<const uint4*>(sp_key + 32 * g);
          const uint4 hi = *reinterpret_cast<const uint4*>(sp_key + 32 * g + 16);
          kb[u] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      }
    }
#pragma unroll
    for (int u4 = 0; u4 < U; u4 += 4) {
      float p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // D[h][entry] = sum_k q[h][k] * key[entry][k]; lane: entry n, heads 4g+i
        v4f d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
        _Float16 ksc = (_Float16)0.0f;
        if (KF) ksc = (_Float16)e4m3_to_f32(((uint32_t)kb[u4 + u][4] >> (8 * g)) & 0xFFu);   // exact
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const v8h kh = KF ? fp4x8_to_f16((uint32_t)kb[u4 + u][v], ksc)
                            : fp8x8_to_f16(kb[u4 + u][2 * v], kb[u4 + u][2 * v + 1]);
          d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa0[v], kh, d0, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa1[v], kh, d1, 0, 0, 0);
        }
        float sp = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sp = fmaf(w0[i], relu0(d0[i]), sp);
          sp = fmaf(w1[i], relu0(d1[i]), sp);
        }
        p[u] = sp;
      }
      // transpose-reduce: lane (n, g) ends with the full score of tile
      // u4 + g, entry n (sum over the four head groups): row g of k0 holds
      // head groups (g & 2, +1) of tile (g & 1), of k1 those of tile 2 +
      // (g & 1); the halves then pair them
      const float k0 = row_pair_sum(p[0], p[1]), k1 = row_pair_sum(p[2], p[3]);
      const float sc = half_pair_sum(k0, k1);
      const int32_t item = c0 + (t0 + u4 + g) * 16 + n;
      const bool in = item < c1;
      bool vis;
      if (LIST) {                                // this lane's looked-up position (-1 past the chunk)
        const int32_t pg = g == 0 ? pos[u4] : g == 1 ? pos[u4 + 1] : g == 2 ? pos[u4 + 2] : pos[u4 + 3];
        vis = pg >= 0;
      } else {
        vis = in && item_pos(a.im, r, item, nv) >= 0;
      }
      const float out = vis ? sc : __uint_as_float(0x7FC00000u);   // NaN: not visible
      if (stage) {                               // uniform
        int si = in ? item - c0 : kScoreStage + (int)threadIdx.x;
        asm volatile("" : "+v"(si));             // a select, not a branch
        sscore[si] = out;
      } else {
        int off = in ? 4 * item : INT32_MAX;
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), srows, off, 0, 0);
      }
      uint32_t bin = vis ? order_key(sc) >> (32 - kHistBits) : kHistBins + threadIdx.x;
      asm volatile("" : "+v"(bin));
      atomicAdd(&hist[bin], 1u);
    }
  };
  v8i kA[U], kB[U];
  int32_t pA[U], pB[U];
  int32_t t0 = wave * U;
  // Group loads are unconditional (tiles past the chunk read a visible key
  // and are discarded): a load on one side of a branch makes the compiler's
  // later waits cover it, which would serialise the double buffer.
  if (G > 0 || DB) load_group(t0, kA, pA, le0);
  __builtin_amdgcn_sched_barrier(0);             // the key loads go out first
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    qa0[u] = fp8x8_to_f16(q0[2 * u], q0[2 * u + 1]);
    qa1[u] = fp8x8_to_f16(q1[2 * u], q1[2 * u + 1]);
  }
  for (int b = threadIdx.x; b < kHistBins; b += kScoreThreads) hist[b] = 0u;
  lds_barrier();                                 // the key loads stay in flight
  if (G > 0) {
    // straight-line: load group i+1 before computing group i
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int32_t ti = t0 + i * gstride;
      if (i + 1 < G) {
        if (i & 1) load_group(ti + gstride, kA, pA, nullptr); else load_group(ti + gstride, kB, pB, nullptr);
      }
      // keep the next group's loads above this group's arithmetic
      __builtin_amdgcn_sched_barrier(0);
      if (i & 1) compute_group(ti, kB, pB); else compute_group(ti, kA, pA);
    }
  } else if (DB) {
    // two groups per trip and no exit between them (a group past the chunk
    // is computed and discarded): one loop shape keeps the waits exact
    for (; t0 < ntiles; t0 += 2 * gstride) {
      const int32_t t1 = t0 + gstride;
      load_group(t1, kB, pB, nullptr);
      __builtin_amdgcn_sched_barrier(0);
      compute_group(t0, kA, pA);
      load_group(t1 + gstride, kA, pA, nullptr);
      __builtin_amdgcn_sched_barrier(0);
      compute_group(t1, kB, pB);
    }
  } else {
    for (; t0 < ntiles; t0 += gstride) {
      load_group(t0, kA, pA, nullptr);
      compute_group(t0, kA, pA);
    }
  }
  lds_barrier();
  if (stage)
    for (int32_t i = threadIdx.x; i < c1 - c0; i += kScoreThreads) srow[c0 + i] = sscore[i];
  flush_hist(hist, a.hist + (int64_t)r * kHistBins);
}

// ---------------------------------------------------------------------------
// row-group score kernel: many rows over one cache (a prefill chunk)
// ---------------------------------------------------------------------------

// When every row reads the same sequence's E4M3 keys in flat mode (the rows
// of one prefill chunk, each with its causal n_valid), a workgroup scores RG
// consecutive rows against each key tile it loads: the tile is read from
// memory and widened to fp16 once for all RG rows, which carry their own
// queries, weights, histograms and visible lengths.  Per row the MFMA
// operands, their order and the head reduction are those of
// index_score_kernel, so the scores are bit-identical.
#ifndef CSA2_ROW_GROUP
#define CSA2_ROW_GROUP 4
#endif
constexpr int kRowGroup = CSA2_ROW_GROUP;
constexpr int kRowTiles = kRowGroup >= 4 ? 2 : 4;   // 16-item tiles per group (registers)

template <int RG, int U>
__global__ __launch_bounds__(kScoreThreads, 2) void index_score_rows_kernel(ScoreArgs a) {
  static_assert(U == 2 || U == 4, "16-item tiles per group: 2 or 4");
  // the rows' histograms, then one word per thread for the counts of lanes
  // that count nothing (the epilogue has no branch)
  __shared__ __align__(8) uint32_t hist[RG * kHistBins + kScoreThreads];
  const int rbase = blockIdx.y * RG;
  // item counts stay below kMaxItems (2^24): 32-bit indices
  int32_t nv[RG];
  int32_t nmax = 0;
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    nv[i] = rbase + i < a.n_rows ? (int32_t)row_valid(a.im, rbase + i) : 0;   // the one sequence, or nothing
    nmax = max(nmax, nv[i]);
  }
  const int32_t c0 = (int32_t)blockIdx.x * a.chunk;
  if (c0 >= nmax) return;                        // uniform for the workgroup
  const int32_t c1 = min(c0 + a.chunk, nmax);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const uint8_t* kbase = a.keys + g * 32;        // sequence 0

  // queries and weights of the RG rows (rows past the end reuse the first)
  v8i qr0[RG], qr1[RG];
  float w0[RG][4], w1[RG][4];
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    const int r = rbase + i < a.n_rows ? rbase + i : rbase;
    const uint8_t* qr = a.q + (int64_t)r * kIdxHeads * kIdxDim + g * 32;
    qr0[i] = load32(qr + n * kIdxDim);
    qr1[i] = load32(qr + (16 + n) * kIdxDim);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w0[i][j] = a.w ? a.w[r * kIdxHeads + 4 * g + j] : 1.0f;
      w1[i][j] = a.w ? a.w[r * kIdxHeads + 16 + 4 * g + j] : 1.0f;
    }
  }

  const int32_t ntiles = (c1 - c0 + 15) / 16;
  const int32_t gstride = kScoreWaves * U;
  auto load_group = [&](int32_t t0, v8i* kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t item = c0 + (t0 + u) * 16 + n;
      const int32_t p = item < c1 ? item : c0;   // past the chunk: a visible key, discarded
      kb[u] = load32(kbase + (uint32_t)p * (uint32_t)kIdxDim);
    }
  };
  v8i kA[U], kB[U];
  int32_t t0 = wave * U;
  load_group(t0, kA);
  __builtin_amdgcn_sched_barrier(0);             // the key loads go out first
  v8h qa0[RG][4], qa1[RG][4];
#pragma unroll
  for (int i = 0; i < RG; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      qa0[i][v] = fp8x8_to_f16(qr0[i][2 * v], qr0[i][2 * v + 1]);
      qa1[i][v] = fp8x8_to_f16(qr1[i][2 * v], qr1[i][2 * v + 1]);
    }
  }
  for (int b = threadIdx.x; b < RG * kHistBins; b += kScoreThreads) hist[b] = 0u;
  lds_barrier();                                 // the key loads stay in flight
  // the workgroup's score rows: a store at an offset past the buffer's size
  // is dropped by the hardware, which masks the stores without a branch
  const auto srows = __builtin_amdgcn_make_buffer_rsrc(a.scores + (int64_t)rbase * a.row_stride, 0,
                                                       (int)((int64_t)RG * a.row_stride * 4), 0x00020000);

  // The two waves of a SIMD alternate: the one in its MFMA phase issues at a
  // raised priority, and the other's epilogue (transposes, stores, histogram
  // atomics) fills the issue slots between its MFMAs.
  auto compute_group = [&](int32_t tg, const v8i* kb) {
    __builtin_amdgcn_s_setprio(1);
    float p[RG][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v8h kh[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) kh[v] = fp8x8_to_f16(kb[u][2 * v], kb[u][2 * v + 1]);
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        v4f d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa0[i][v], kh[v], d0, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa1[i][v], kh[v], d1, 0, 0, 0);
        }
        float sp = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sp = fmaf(w0[i][j], relu0(d0[j]), sp);
          sp = fmaf(w1[i][j], relu0(d1[j]), sp);
        }
        p[i][u] = sp;
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // per row, the transpose-reduce of index_score_kernel: lane (n, g) ends
    // with the score of tile g (U = 4) or g & 1 (U = 2, lanes g >= 2 hold a
    // copy and store nothing), entry n; the adds pair the head groups as
    // index_score_kernel does, so the scores are bit-identical
    const int32_t item = c0 + (tg + (U == 4 ? g : (g & 1))) * 16 + n;
    // lanes holding a copy get an item no bound admits
    const int32_t item_o = (U == 4 || g < 2) ? item : INT32_MAX;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      float sc;
      if (U == 4) {
        sc = half_pair_sum(row_pair_sum(p[i][0], p[i][1]), row_pair_sum(p[i][2], p[i][3]));
      } else {
        const float k0 = row_pair_sum(p[i][0], p[i][1]);
        sc = half_pair_sum(k0, k0);
      }
      const bool own = item_o < min(c1, nv[i]);
      // the order key without order_key's -0 case: a score here is never
      // -0 (the sums start at +0, relu0 gives no -0, and a zero sum of
      // terms that are not -0 is +0 when rounding to nearest)
      const uint32_t u = __float_as_uint(sc);
      const uint32_t ok = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
      int off = own ? 4 * item + i * 4 * a.row_stride : INT32_MAX;
      uint32_t bin = own ? (uint32_t)(i * kHistBins) + (ok >> (32 - kHistBits)) : (uint32_t)(RG * kHistBins) + threadIdx.x;
      asm volatile("" : "+v"(off), "+v"(bin));  // selects, not branches
      // non-temporal: the block is read once, by the top-k after the scan,
      // and streaming it past the caches keeps the shared keys there
      __builtin_amdgcn_raw_buffer_store_b32(u, srows, off, 0, 2);
      atomicAdd(&hist[bin], 1u);
    }
  };
  // two groups per trip, no exit between them (a group past the chunk is
  // computed and discarded): the waits stay exact
  for (; t0 < ntiles; t0 += 2 * gstride) {
    const int32_t t1 = t0 + gstride;
    load_group(t1, kB);
    __builtin_amdgcn_sched_barrier(0);
    compute_group(t0, kA);
    load_group(t1 + gstride, kA);
    __builtin_amdgcn_sched_barrier(0);
    compute_group(t1, kB);
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    if (rbase + i >= a.n_rows) break;            // uniform
    flush_hist(hist + i * kHistBins, a.hist + (int64_t)(rbase + i) * kHistBins);
  }
}

bool score_rows_path(const ScoreArgs& a) {
  return a.im.mode == kItemsFlat && !a.key_fp4 && a.n_seq == 1 && a.n_rows >= kScoreRowsMin;
}

// Workgroups of one score kernel that fit on the device at once.
int score_resident_wgs() {
  static int cached = 0;
  if (cached) return cached;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, index_score_kernel<kItemsBlocks, 0, kScoreDB, kScoreMinW>,
                                                   kScoreThreads, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();
    return 1024;
  }
  cached = cus * per_cu;
  return cached;
}

hipError_t launch_index_score(const ScoreArgs& a, hipStream_t stream) {
  if (a.n_rows == 0 || a.im.n_items == 0) return hipSuccess;
  if (score_rows_path(a)) {
    // row groups over one cache: each group's items in chunks of whole
    // 256-item steps, as many as keep every resident slot busy
    ScoreArgs b = a;
    const int64_t groups = (a.n_rows + kRowGroup - 1) / kRowGroup;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      cus = 256;
    }
    const int64_t slots = (int64_t)cus * 2;      // two workgroups per CU
    const int64_t per_group = groups >= slots ? 1 : slots / groups;
    int64_t c = (a.im.n_items + per_group - 1) / per_group;
    c = (c + 255) / 256 * 256;
    b.chunk = (int32_t)c;
    const dim3 grid((unsigned)((a.im.n_items + c - 1) / c), (unsigned)groups), block(kScoreThreads);
    hipLaunchKernelGGL((index_score_rows_kernel<kRowGroup, kRowTiles>), grid, block, 0, stream, b);
    return hipGetLastError();
  }
  const int64_t chunks = ((int64_t)a.im.n_items + a.chunk - 1) / a.chunk;
  const dim3 grid((unsigned)(chunks + (a.fuse_append ? 1 : 0)), (unsigned)a.n_rows), block(kScoreThreads);
  // a chunk of exactly one group per wave (the 16384-position pool, short
  // rows) runs the straight-line form: no second, discarded group
  const bool one = a.chunk == kScoreWaves * kTilesPerIter * 16;
#define CSA2_SCORE(MM, KK)                                                                              \
  do {                                                                                                  \
    if (one)                                                                                            \
      hipLaunchKernelGGL((index_score_kernel<MM, KK, kScoreDB, kScoreMinW, kTilesPerIter, 1>), grid, block, \
                         0, stream, a);                                                                 \
    else                                                                                                \
      hipLaunchKernelGGL((index_score_kernel<MM, KK, kScoreDB, kScoreMinW>), grid, block, 0, stream, a);    \
  } while (0)
  if (a.im.mode == kItemsBlocks && a.fuse_append) {                // the coarse stage of a decode step
    if (one)
      hipLaunchKernelGGL((index_score_kernel<kItemsBlocks, 0, kScoreDB, kScoreMinW, kTilesPerIter, 1, true>), grid,
                         block, 0, stream, a);
    else
      hipLaunchKernelGGL((index_score_kernel<kItemsBlocks, 0, kScoreDB, kScoreMinW, kTilesPerIter, 0, true>), grid,
                         block, 0, stream, a);
  } else if (a.im.mode == kItemsBlocks) CSA2_SCORE(kItemsBlocks, 0);      // block summaries are E4M3
  else if (a.key_fp4) {
    if (a.im.mode == kItemsFlat) CSA2_SCORE(kItemsFlat, 1);
    else if (a.im.mode == kItemsPool) CSA2_SCORE(kItemsPool, 1);
    else CSA2_SCORE(kItemsCand, 1);
  } else {
    if (a.im.mode == kItemsFlat) CSA2_SCORE(kItemsFlat, 0);
    else if (a.im.mode == kItemsPool) CSA2_SCORE(kItemsPool, 0);
    else CSA2_SCORE(kItemsCand, 0);
  }
#undef CSA2_SCORE
  return hipGetLastError();
}

}  // namespace csa2
