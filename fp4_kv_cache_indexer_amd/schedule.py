"""The CSA2 layer schedule of the 40-layer model and what one decode step
runs per layer [0539edu §3: the csa2 block of the inference configuration,
encoder and decoder groups; the paragraph after the TOML listing on the
candidate pool].

* Encoder (20 layers, compression ratio 2): the first two layers attend to
  their sliding window only; the other 18 form three groups of six, each a
  Full layer (builds a global cache and selects its entries) followed by
  five Reuse layers (same cache and selection, their own queries).
* Decoder (20 layers, compression ratio 1): five groups of four; the first
  group is Full + 3 Reuse, the other four Reindex + 3 Reuse.  A Reindex layer
  selects anew with its own indexer queries, over the decoder cache, within
  the candidate pool the decoder's Full layer kept.

So four layers build a global cache (three encoder caches at m = 2, one
decoder cache at m = 1) and every layer keeps its own 128-token window.
"""

from dataclasses import dataclass

WINDOW = 128


@dataclass(frozen=True)
class Layer:
    index: int
    side: str        # "encoder" | "decoder"
    mode: str        # "swa_only" | "full" | "reuse" | "reindex"
    m: int           # compression ratio of the side's caches
    cache: int       # global cache the layer attends to (-1: window only)
    group: int       # layer group (-1: window only)


def csa2_layers():
    """The 40 layers in order."""
    out = []

    def add(side, mode, m, cache, group):
        out.append(Layer(len(out), side, mode, m, cache, group))

    for _ in range(2):
        add("encoder", "swa_only", 2, -1, -1)
    for g in range(3):
        add("encoder", "full", 2, g, g)
        for _ in range(5):
            add("encoder", "reuse", 2, g, g)
    for g in range(5):
        add("decoder", "full" if g == 0 else "reindex", 1, 3, 3 + g)
        for _ in range(3):
            add("decoder", "reuse", 1, 3, 3 + g)
    return out


def cache_ratios(layers):
    """Compression ratio of each global cache, by cache id."""
    ratios = {}
    for ly in layers:
        if ly.mode == "full":
            ratios[ly.cache] = ly.m
    return [ratios[c] for c in sorted(ratios)]


def global_bytes_per_token(layers, main_entry_bytes, index_entry_bytes):
    """Global-cache bytes per token: every cache holds one entry per m tokens."""
    return sum((main_entry_bytes + index_entry_bytes) / m for m in cache_ratios(layers))


def decode_layers(layers, caches, rings, swa_len, q, q_idx, top_k=512, keep_blocks=2048, out=None, lse=None,
                  sel=None, blocks=None, ws_idx=None, ws_pool=None, ws_attn=None):
    """One token through every layer's selection and attention, for a batch
    of sequences (row b is sequence b of every cache and window).

    caches   -- per cache id, a dict: codes [B, N, 256], scales [B, N, 32],
                keys (E4M3 [B, N, 128] or FP4 codes [B, N, 64]), key_scales
                (FP4: [B, N, 4], else None), summ (block keys
                [B, ceil(N/8), 128] for a hierarchical Full layer, else None)
    rings    -- the layers' windows, uint8 [L, B, cap, 512]; swa_len int32 [B]
    q        -- per layer, bf16 [B, H, 512]; q_idx -- per Full/Reindex layer
                index, E4M3 [B, 32, 128]
    out, lse -- per layer output buffers (allocated when None; may alias)
    sel      -- per layer group, int32 [B, top_k] selections (allocated when None)
    blocks   -- per cache id with a hierarchical Full layer, int32
                [B, keep_blocks]: its kept blocks, the pool its Reindex
                layers select within (allocated when None)
    ws_*     -- workspaces per cache id (indexer, pool indexer) and for the
                attention; allocated per call when None
    Full layers select over their cache (coarse-to-fine when it has block
    keys), Reindex layers within the pool of their cache's Full layer (over
    the whole cache when that layer was flat), Reuse layers attend with their
    group's selection, window-only layers attend to their window alone.
    Returns (out, lse, sel, blocks)."""
    import torch

    from . import csa2 as C

    B = rings.shape[1]
    dev = rings.device
    L = len(layers)
    out = out if out is not None else [None] * L
    lse = lse if lse is not None else [None] * L
    sel = sel if sel is not None else {}
    blocks = blocks if blocks is not None else {}
    ws_idx = ws_idx or {}
    ws_pool = ws_pool or {}
    for ly in layers:
        ring = rings[ly.index]
        if ly.mode == "swa_only":
            out[ly.index], lse[ly.index] = C.sparse_attn_decode(
                q[ly.index], None, None, None, swa=ring, swa_len=swa_len, out=out[ly.index], lse=lse[ly.index],
                workspace=ws_attn)
            continue
        c = caches[ly.cache]
        if ly.group not in sel:
            sel[ly.group] = torch.empty((B, top_k), dtype=torch.int32, device=dev)
        idx = sel[ly.group]
        hier = c.get("summ") is not None
        if ly.mode == "full":
            if hier and ly.cache not in blocks:
                blocks[ly.cache] = torch.empty((B, keep_blocks), dtype=torch.int32, device=dev)
            C.indexer_topk(q_idx[ly.index], c["keys"], top_k, block_keys=c.get("summ"), keep_blocks=keep_blocks,
                           out_idx=idx, out_blocks=blocks.get(ly.cache) if hier else None,
                           workspace=ws_idx.get(ly.cache), key_scales=c.get("key_scales"))
        elif ly.mode == "reindex":
            if hier:
                C.indexer_topk(q_idx[ly.index], c["keys"], top_k, cand_blocks=blocks[ly.cache], out_idx=idx,
                               workspace=ws_pool.get(ly.cache), key_scales=c.get("key_scales"))
            else:
                C.indexer_topk(q_idx[ly.index], c["keys"], top_k, out_idx=idx, workspace=ws_idx.get(ly.cache),
                               key_scales=c.get("key_scales"))
        out[ly.index], lse[ly.index] = C.sparse_attn_decode(
            q[ly.index], c["codes"], c["scales"], idx, swa=ring, swa_len=swa_len, out=out[ly.index],
            lse=lse[ly.index], workspace=ws_attn)
    return out, lse, sel, blocks
