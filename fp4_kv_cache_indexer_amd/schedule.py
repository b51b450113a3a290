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
