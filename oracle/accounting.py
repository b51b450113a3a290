"""Global-KV byte accounting of the CSA2 cache.

* Cache size is roughly sequence length x layers that store a cache x numbers
  per entry x bytes per number [daiw table "four factors", the formula above
  it]; the worked example of [nxbn §2.1] applies it to a dense 64-layer
  model.
* Sequence compression divides the entry count by m (m = 2 in the encoder,
  1 in the decoder) and only the layers that build a cache store one
  [daiw table "four factors"]; in the layer schedule of [0539edu §3] those are
  the ``full`` layers (Reuse and Reindex layers read the group's cache).
* An FP4 E2M1 entry of d channels with one E4M3 scale per 16 channels takes
  d/2 + d/16 bytes [0539edu §3].

Test infrastructure only (see the package docstring).
"""

from fractions import Fraction


def kv_bytes(seq_len, layers, numbers_per_entry, bytes_per_number):
    """The four-factor cache size: product of the factors."""
    return seq_len * layers * numbers_per_entry * bytes_per_number


def fp4_entry_bytes(dim, group=16, scale_bytes=1):
    """Bytes of one FP4 entry: half a byte per channel plus one scale per group."""
    if dim % group or dim % 2:
        raise ValueError("dim must be a multiple of the scale group and of 2")
    return dim // 2 + (dim // group) * scale_bytes


def fp8_entry_bytes(dim):
    """Bytes of one FP8 entry: one byte per channel."""
    return dim


def cache_layers(schedule):
    """The compression ratios of the layers that build a global cache.

    ``schedule`` is a list of (mode, m) per layer, mode in
    {"swa_only", "full", "reuse", "reindex"}.
    """
    return [m for mode, m in schedule if mode == "full"]


def bytes_per_token(schedule, main_entry_bytes, index_entry_bytes=0):
    """Global-KV bytes per token: sum over cache-building layers of
    (main entry + index-key entry) / m, as an exact fraction."""
    return sum(Fraction(main_entry_bytes + index_entry_bytes, m) for m in cache_layers(schedule))


def schedule_from_config(cfg):
    """Expand the ``csa2`` block of the inference configuration of
    [0539edu §3] (a dict with ``encoder``/``decoder``) into a per-layer list
    of (mode, m)."""
    out = []
    for part in ("encoder", "decoder"):
        p = cfg[part]
        m = int(p["compression_ratio"])
        n_groups_layers = sum(int(g["size"]) for g in p["groups"])
        lead = int(p["layers"]) - n_groups_layers
        if lead:
            if p.get("first_two_layers") != "swa_only" or lead != 2:
                raise ValueError("unexpected leading layers")
            out += [("swa_only", m)] * lead
        for g in p["groups"]:
            if len(g["modes"]) != int(g["size"]):
                raise ValueError("group size does not match its modes")
            out += [(mode, m) for mode in g["modes"]]
    return out
