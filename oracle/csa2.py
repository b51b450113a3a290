"""The CSA2 decode hot path, step by step, as plain NumPy (float64).

Steps and where the pages state them:

1. ``pool``            -- the main key compressor folds every m tokens into one
   entry with weights that depend on the context rather than a uniform mean
   [nxbn §4.2];
   m = 2 in the encoder layers, m = 1 in the decoder layers [0539edu §3],
   [daiw table "four factors", row "sequence length"].  Read as a per-channel
   softmax over the m tokens of a group of caller-supplied gate logits; no
   logits means equal weights (the mean).
2. ``quantize_fp4``    -- main KV stored as FP4 E2M1 with one E4M3 scale per
   16 channels and no second-level scale [0539edu §3].  Scale = amax/6 rounded
   to E4M3 (6 is the largest E2M1 magnitude); each value rounded to the
   nearest E2M1 multiple of the scale, ties to the even code.
3. ``dequantize_fp4``  -- value = E2M1(code) * E4M3(scale).
4. ``block_summary``   -- hierarchical indexer blocks of 8 positions
   [0539edu §3, ``positions_per_block``]; a block's key is the mean of its
   member keys rounded to E4M3.
5. ``index_scores``    -- multi-head indexer, 32 heads x 128 dims
   [0539edu §3, ``csa2.indexer``]; heads combined as sum_h w_h * ReLU(q_h . k).
6. ``topk_select``     -- top_k = 512 [0539edu §3]; ties go to the lower index;
   output ascending, padded with -1.
7. ``indexer_topk_hier`` -- coarse-to-fine: keep at most 2048 blocks
   (``max_blocks``), expand to their 8 positions each (a candidate pool of at
   most 16384), score those exactly, keep top_k [0539edu §3 and the paragraph
   on ``candidate_pool_size`` after the TOML listing].
8. ``sparse_attn``     -- one 512-dim latent shared by all query heads
   [daiw table "four factors", row "entry dimension"], used as both key and
   value; selected global entries attended jointly with the 128-token FP8
   sliding window [0539edu §3 ``swa_window_size``], [daiw "cost factors"
   paragraph on local window + compressed global context]; one softmax over
   all keys, scale 1/sqrt(512) unless given.
9. ``layer_group``     -- Full / Reuse / Reindex layers: Reuse layers reuse the
   main KV and top-k indices, Reindex layers issue new indexer queries over the
   shared cache [0539edu §1, §3 (``csa2.decoder.groups``)].
10. ``prefill_row_view`` -- a prefill query at position p sees an entry once all
   of its m tokens are at or before p, and the SWA tokens [p-127, p].

Test infrastructure only (see the package docstring).
"""

import math

import numpy as np

from .formats import (
    E2M1_MAGNITUDES,
    bf16_bits_to_f64,
    e2m1_decode,
    e4m3_decode,
    e4m3_rne_sat,
)

LATENT_DIM = 512
SCALE_GROUP = 16
IDX_HEADS = 32
IDX_DIM = 128
BLOCK_POS = 8
IDX_FP4_GROUP = 32          # channels per E4M3 scale of an FP4 index key


# ---------------------------------------------------------------------------
# 1-3. cache write: pooling, FP4 quantisation, dequantisation
# ---------------------------------------------------------------------------


def pool(x, z, m):
    """Fold every m consecutive tokens into one entry.

    x: float64 [T, C] token latents; z: float64 [T, C] gate logits or None;
    T must be a multiple of m.  Returns the pooled entries rounded to float32
    (the precision in which the quantiser takes its decisions) as float64
    values, shape [T/m, C].

    For m = 1 the entry is the token itself.  Otherwise, per channel, the
    weights are the softmax over the m tokens of the group of that channel's
    logits (equal weights when z is None) [nxbn §4.2].
    """
    x = np.asarray(x, dtype=np.float64)
    T, C = x.shape
    if T % m:
        raise ValueError("pool: token count must be a multiple of m")
    xg = x.reshape(T // m, m, C)
    if m == 1:
        y = xg[:, 0, :]
    elif z is None:
        y = xg.mean(axis=1)
    else:
        zg = np.asarray(z, dtype=np.float64).reshape(T // m, m, C)
        e = np.exp(zg - zg.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        y = (p * xg).sum(axis=1)
    return y.astype(np.float32).astype(np.float64)


def quantize_fp4(y, chunk=8192, group=SCALE_GROUP):
    """Quantise entries y [E, C] (float32 values, given as float64) to packed
    FP4 codes and E4M3 scales [0539edu §3, nxbn §3.1].

    Per group of `group` channels (16 for the main KV): amax = max |y|; scale = E4M3(amax / 6) with the
    division done in float32 (6 is the largest E2M1 magnitude); a zero scale
    gives all-zero codes; otherwise each |y| becomes the nearest point of
    {0, .5, 1, 1.5, 2, 3, 4, 6} * scale, an exact tie keeping the even code;
    the sign is kept except on zero; values beyond 6 * scale take the top of
    the grid.  (After that clip the distances are exact in float64: the grid
    points have at most 7 significant bits and |y| at most 24.)

    Returns codes uint8 [E, C/2] (channel 2j in the low nibble of byte j,
    channel 2j+1 in the high nibble) and scales uint8 [E, C/group].
    """
    y = np.asarray(y, dtype=np.float64)
    E, C = y.shape
    G = C // group
    packed = np.empty((E, C // 2), dtype=np.uint8)
    scales = np.empty((E, G), dtype=np.uint8)
    even = (np.arange(8) % 2 == 0)
    for e0 in range(0, E, chunk):
        yg = y[e0:e0 + chunk].reshape(-1, G, group)
        amax = np.abs(yg).max(axis=2).astype(np.float32)
        s_code = e4m3_rne_sat((amax / np.float32(6.0)).astype(np.float64))
        s = e4m3_decode(s_code)
        grid = E2M1_MAGNITUDES[None, None, None, :] * s[:, :, None, None]
        # beyond the top of the grid the nearest point is the top (6 * scale);
        # clipping first keeps every distance exact in float64
        a = np.minimum(np.abs(yg), 6.0 * s[:, :, None])
        d = np.abs(a[..., None] - grid)                   # [e, G, 16, 8]
        ties = d == d.min(axis=3, keepdims=True)
        even_tie = ties & even
        mag = np.where(even_tie.any(axis=3), even_tie.argmax(axis=3), ties.argmax(axis=3))
        mag = np.where(s[:, :, None] == 0.0, 0, mag)
        nib = mag + 8 * ((yg < 0) & (mag != 0))
        nib = nib.reshape(-1, C)
        packed[e0:e0 + chunk] = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        scales[e0:e0 + chunk] = s_code
    return packed, scales


def unpack_fp4(codes):
    """Packed bytes [E, C/2] -> nibble codes [E, C] (low nibble first)."""
    codes = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.int64)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def dequantize_fp4(codes, scales, group=SCALE_GROUP):
    """FP4 entries back to float64: E2M1(code) * E4M3(scale of its group)."""
    v = e2m1_decode(unpack_fp4(codes))
    s = e4m3_decode(scales)
    return v * np.repeat(s, group, axis=1)


def kv_compress_quantize(x_bits, z_bits, m):
    """Cache write for one sequence: bf16 tokens [T, 512] (+ bf16 gate logits
    or None) -> FP4 codes [T/m, 256], scales [T/m, 32].  A trailing partial
    group of fewer than m tokens is not emitted."""
    x = bf16_bits_to_f64(x_bits)
    T = (x.shape[0] // m) * m
    z = None if z_bits is None else bf16_bits_to_f64(z_bits)[:T]
    y = pool(x[:T], z, m)
    return quantize_fp4(y)


# ---------------------------------------------------------------------------
# 4. block summaries
# ---------------------------------------------------------------------------


def block_summary(keys):
    """keys uint8 E4M3 [N, 128] -> block keys uint8 [ceil(N/8), 128].

    Each block's key is the mean of the decoded keys of its (up to 8) members,
    computed as an exact sum divided by the member count in float32, then
    rounded to E4M3.  (Any sum of at most 8 E4M3 values is exact in float32:
    it is a multiple of 2**-9 below 2**12, so only the division rounds.)
    FP4 keys (Fp4Keys) go to block_summary_fp4.
    """
    if isinstance(keys, Fp4Keys):
        return block_summary_fp4(keys.codes, keys.scales)
    k = e4m3_decode(keys)
    N, D = k.shape
    nb = (N + BLOCK_POS - 1) // BLOCK_POS
    pad = np.zeros((nb * BLOCK_POS, D))
    pad[:N] = k
    ssum = pad.reshape(nb, BLOCK_POS, D).sum(axis=1).astype(np.float32)
    count = np.minimum(BLOCK_POS, N - np.arange(nb) * BLOCK_POS).astype(np.float32)
    mean = ssum / count[:, None]
    return e4m3_rne_sat(mean.astype(np.float64))


# ---------------------------------------------------------------------------
# 4b. FP4 index keys: 128 x E2M1 + one E4M3 scale per 32 channels = 68 B/entry
# ---------------------------------------------------------------------------
#
# [daiw "four generations" table: 890 B/token of global cache; "four factors"
# table: FP4 main KV with E4M3 scales] -- with 2.5 entries per token and a
# 288-byte FP4 main entry, 170 B/token = 68 B/entry are left for the index
# key: 128 FP4 codes (64 B) and 4 B of scale, read here as one E4M3 scale per
# 32 channels, quantised by the same rule as the main KV.


class Fp4Keys:
    """FP4 index keys (codes [N, 64], scales [N, 4]); indexable like E4M3
    keys [N, 128], so every indexer function below takes either."""

    def __init__(self, codes, scales):
        self.codes = np.asarray(codes, dtype=np.uint8)
        self.scales = np.asarray(scales, dtype=np.uint8)

    @property
    def shape(self):
        return (self.codes.shape[0], IDX_DIM)

    def __getitem__(self, sel):
        return Fp4Keys(self.codes[sel], self.scales[sel])

    def decode(self):
        return index_key_decode_fp4(self.codes, self.scales)


def index_key_quantize_fp4(k_bits):
    """bf16 index keys [N, 128] -> FP4 codes uint8 [N, 64], scales uint8 [N, 4]."""
    return quantize_fp4(bf16_bits_to_f64(k_bits), group=IDX_FP4_GROUP)


def index_key_decode_fp4(codes, scales):
    """FP4 index keys back to float64 [N, 128]."""
    return dequantize_fp4(codes, scales, group=IDX_FP4_GROUP)


def block_summary_fp4(codes, scales):
    """Block keys (E4M3 [ceil(N/8), 128]) of FP4 index keys: the mean of the
    members' decoded values, as their sum divided by the member count in
    float32, rounded to E4M3.  (The decoded values are multiples of 2**-10
    below 2**12 in magnitude, so float32 partial sums are exact while below
    2**14; a block that reaches 2**14 has a mean beyond 448 in magnitude and
    saturates either way.  The sum is formed in float32 in member order.)"""
    k = index_key_decode_fp4(codes, scales).astype(np.float32)
    N, D = k.shape
    nb = (N + BLOCK_POS - 1) // BLOCK_POS
    ssum = np.zeros((nb, D), dtype=np.float32)
    for j in range(BLOCK_POS):
        rows = np.arange(nb) * BLOCK_POS + j
        ok = rows < N
        ssum[ok] = ssum[ok] + k[rows[ok]]
    count = np.minimum(BLOCK_POS, N - np.arange(nb) * BLOCK_POS).astype(np.float32)
    return e4m3_rne_sat((ssum / count[:, None]).astype(np.float64))


# ---------------------------------------------------------------------------
# 5-7. indexer and top-k
# ---------------------------------------------------------------------------


def index_scores_dec(q, w, kd):
    """I_t = sum_h w_h * max(0, q_h . k_t), all in float64, for decoded keys
    kd float [N, 128].  q uint8 E4M3 [32, 128]; w float [32] or None (ones)."""
    qd = e4m3_decode(q)
    wd = np.ones(qd.shape[0]) if w is None else np.asarray(w, dtype=np.float64)
    dots = qd @ np.asarray(kd, dtype=np.float64).T    # [32, N]
    return (wd[:, None] * np.maximum(dots, 0.0)).sum(axis=0)


def index_scores(q, w, keys):
    """I_t = sum_h w_h * max(0, q_h . k_t), all in float64.

    q uint8 E4M3 [32, 128]; w float [32] or None (all ones); keys uint8 E4M3
    [N, 128].  Returns float64 [N].
    """
    if isinstance(keys, Fp4Keys):
        return index_scores_dec(q, w, keys.decode())
    return index_scores_dec(q, w, e4m3_decode(keys))


def topk_select(scores, ids, k):
    """Top-k of (score, id) pairs: order by score descending, then id
    ascending; keep the first min(k, n); return the ids ascending, padded
    with -1 to length k."""
    scores = np.asarray(scores, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -scores))
    keep = np.sort(ids[order[:min(k, len(ids))]])
    out = np.full(k, -1, dtype=np.int64)
    out[:len(keep)] = keep
    return out


def indexer_topk_flat(q, w, keys, k, n_valid=None):
    """Flat indexer: score entries [0, n_valid) and keep the top k."""
    N = keys.shape[0] if n_valid is None else int(n_valid)
    s = index_scores(q, w, keys[:N])
    return topk_select(s, np.arange(N), k)


def indexer_topk_pool(q, w, keys, cand, k, n_valid=None):
    """Indexer restricted to a candidate list of entry ids (ids outside
    [0, n_valid) and -1 are skipped)."""
    N = keys.shape[0] if n_valid is None else int(n_valid)
    cand = np.asarray(cand, dtype=np.int64)
    cand = cand[(cand >= 0) & (cand < N)]
    s = index_scores(q, w, keys[cand])
    return topk_select(s, cand, k)


def coarse_blocks(q, w, block_keys, n_valid, keep_blocks):
    """Coarse stage: score the blocks that hold at least one visible entry and
    keep the first min(keep_blocks, #blocks) by (score desc, block id asc).
    Returns (kept block ids ascending, all block scores)."""
    nb = (int(n_valid) + BLOCK_POS - 1) // BLOCK_POS
    sb = index_scores(q, w, block_keys[:nb])
    kept = topk_select(sb, np.arange(nb), min(keep_blocks, nb))
    return kept, sb


def pool_positions(blocks, n_valid):
    """Expand block ids to their member positions below n_valid (ascending)."""
    blocks = np.asarray(blocks, dtype=np.int64)
    blocks = blocks[blocks >= 0]
    pos = (blocks[:, None] * BLOCK_POS + np.arange(BLOCK_POS)[None, :]).reshape(-1)
    return pos[pos < int(n_valid)]


def indexer_topk_hier(q, w, keys, block_keys, k, n_valid=None, keep_blocks=2048):
    """Coarse-to-fine indexer.  Returns (top-k ids, kept blocks)."""
    N = keys.shape[0] if n_valid is None else int(n_valid)
    kept, _ = coarse_blocks(q, w, block_keys, N, keep_blocks)
    cand = pool_positions(kept, N)
    return indexer_topk_pool(q, w, keys, cand, k, N), kept


# ---------------------------------------------------------------------------
# 8. joint sparse + sliding-window attention
# ---------------------------------------------------------------------------


def sparse_attn(q_bits, codes, scales, idx, swa=None, swa_slots=(), sm_scale=None):
    """One query row.

    q_bits: uint16 bf16 bits [H, 512]; codes/scales: the row's FP4 cache
    [N, 256] / [N, 32]; idx: selected entry ids (-1 skipped); swa: uint8 E4M3
    [cap, 512] and swa_slots the slots of the window.  Keys and values are
    the same vectors: the dequantised entries followed by the window tokens.
    Returns (O float64 [H, 512], LSE float64 [H]); with no key, O = 0 and
    LSE = -inf.
    """
    q = bf16_bits_to_f64(q_bits)
    H, D = q.shape
    scale = 1.0 / math.sqrt(D) if (sm_scale is None or sm_scale <= 0) else float(sm_scale)
    idx = np.asarray(idx, dtype=np.int64)
    idx = idx[idx >= 0]
    parts = []
    if len(idx):
        parts.append(dequantize_fp4(codes[idx], scales[idx]))
    slots = np.asarray(list(swa_slots), dtype=np.int64)
    if len(slots):
        parts.append(e4m3_decode(swa[slots]))
    if not parts:
        return np.zeros((H, D)), np.full(H, -np.inf)
    K = np.concatenate(parts, axis=0)                 # [n_keys, 512]
    s = (q @ K.T) * scale                             # [H, n_keys]
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    l = e.sum(axis=1, keepdims=True)
    O = (e / l) @ K
    lse = (mx + np.log(l))[:, 0]
    return O, lse


def swa_slots(start, length, cap):
    """Ring-buffer slots of a window: (start + j) mod cap for j < length."""
    return [(int(start) + j) % int(cap) for j in range(int(length))]


# ---------------------------------------------------------------------------
# 9. layer groups
# ---------------------------------------------------------------------------


def layer_group(modes, q_attn, q_idx, w_idx, codes, scales, keys, swa, slots, k,
                block_keys=None, keep_blocks=2048, n_valid=None, sm_scale=None,
                reindex_in_pool=False):
    """Run one row through a group of layers with modes in {full, reuse,
    reindex}.  Full and Reindex layers select with their own indexer query
    over the shared keys; Reuse layers attend with the last selection.  The
    main KV and index keys are shared by the group; each layer has its own
    query and its own sliding window (swa[L]).  Returns [(idx, O, LSE)] per
    layer.

    reindex_in_pool (with block_keys): a Reindex layer selects only among the
    candidate pool -- the kept blocks' positions -- of the latest Full layer,
    instead of running its own coarse stage [0539edu §3: the 16384-position
    pool bounds the indexer's work per query; ai-feeds Method: index reuse
    across layers]."""
    idx = None
    pool_blocks = None
    out = []
    for L, mode in enumerate(modes):
        if mode in ("full", "reindex"):
            if block_keys is None:
                idx = indexer_topk_flat(q_idx[L], w_idx[L], keys, k, n_valid)
            elif mode == "reindex" and reindex_in_pool:
                if pool_blocks is None:
                    raise ValueError("a pool-restricted reindex layer needs an earlier full layer")
                N = keys.shape[0] if n_valid is None else int(n_valid)
                idx = indexer_topk_pool(q_idx[L], w_idx[L], keys, pool_positions(pool_blocks, N), k, N)
            else:
                idx, kept = indexer_topk_hier(q_idx[L], w_idx[L], keys, block_keys, k,
                                              n_valid, keep_blocks)
                if mode == "full":
                    pool_blocks = kept
        elif mode == "reuse":
            if idx is None:
                raise ValueError("a reuse layer needs an earlier full/reindex layer")
        else:
            raise ValueError(mode)
        O, lse = sparse_attn(q_attn[L], codes, scales, idx, swa[L], slots, sm_scale)
        out.append((idx.copy(), O, lse))
    return out


# ---------------------------------------------------------------------------
# 10. prefill rows
# ---------------------------------------------------------------------------


def prefill_row_view(p, m, window=128):
    """For a prefill query at token position p: the number of visible entries
    (entry i covers tokens [m*i, m*i + m) and is visible when m*i + m - 1 <= p)
    and the window's token range [max(0, p - window + 1), p]."""
    n_valid = (int(p) + 1) // int(m)
    lo = max(0, int(p) - window + 1)
    return n_valid, lo, int(p) - lo + 1
