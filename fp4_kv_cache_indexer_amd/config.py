"""CSA2 configuration: the cache and indexer keys of the pages' inference
configuration, carried down to the integers the C ABI takes
[0539edu §3: the kv_cache block (global_kv_dtype, global_kv_scale,
swa_kv_dtype, swa_window_size) and the csa2 block (encoder/decoder layer
groups and compression ratios, indexer query_heads / head_dim / top_k and its
hierarchical max_blocks / positions_per_block / candidate_pool_size)].

``Csa2Config.from_dict`` reads that configuration (as JSON-like dicts; keys
other than these are ignored), ``validate`` rejects what the kernels do not
implement, and ``indexer_kwargs`` / ``attn_kwargs`` / ``cache_kwargs`` give
the keyword arguments of the binding's calls.  ``layers`` expands the
encoder and decoder groups into the per-layer table ``schedule`` drives.

One key is not on the pages: ``index_key_dtype``, the storage of the index
keys -- "e4m3" (128 B per entry, the default) or "fp4_e2m1" (64 code bytes +
4 E4M3 scales, the 68 B per entry that closes 890 B/token of global cache).
"""

from dataclasses import dataclass, field
from typing import Tuple

from . import schedule as _schedule

LATENT_DIM = 512          # one latent per entry, shared by all query heads [daiw "four factors"]
SCALE_GROUP = 16          # channels per E4M3 scale (e4m3_per_16_channel)
MAX_TOPK = 2048           # largest top_k / keep_blocks the kernels select
KEY_E4M3, KEY_FP4 = 0, 1  # CSA2_KEY_* of include/csa2.h

_MODES = ("full", "reuse", "reindex")


class ConfigError(ValueError):
    pass


@dataclass(frozen=True)
class Hierarchical:
    enabled: bool = True
    max_blocks: int = 2048
    positions_per_block: int = 8
    candidate_pool_size: int = 16384


@dataclass(frozen=True)
class Indexer:
    query_heads: int = 32
    head_dim: int = 128
    top_k: int = 512
    hierarchical: Hierarchical = field(default_factory=Hierarchical)


@dataclass(frozen=True)
class Group:
    modes: Tuple[str, ...]


@dataclass(frozen=True)
class Side:
    layers: int
    compression_ratio: int
    groups: Tuple[Group, ...]
    swa_only_layers: int = 0      # leading layers with the window only ("first_two_layers": "swa_only")


@dataclass(frozen=True)
class Csa2Config:
    global_kv_dtype: str = "fp4_e2m1"
    global_kv_scale: str = "e4m3_per_16_channel"
    swa_kv_dtype: str = "fp8"
    swa_window_size: int = 128
    index_key_dtype: str = "e4m3"
    indexer: Indexer = field(default_factory=Indexer)
    encoder: Side = field(default_factory=lambda: Side(
        20, 2, tuple(Group(("full",) + ("reuse",) * 5) for _ in range(3)), swa_only_layers=2))
    decoder: Side = field(default_factory=lambda: Side(
        20, 1, (Group(("full",) + ("reuse",) * 3),) + tuple(Group(("reindex",) + ("reuse",) * 3) for _ in range(4))))

    # -- reading ------------------------------------------------------------

    @classmethod
    def from_dict(cls, d):
        """Build from the configuration's dicts: ``kv_cache`` and ``csa2``
        (with ``encoder``, ``decoder`` and ``indexer``).  Missing keys keep
        the defaults, which are the pages' values."""
        kv = d.get("kv_cache", {})
        cs = d.get("csa2", {})
        ix = cs.get("indexer", {})
        hi = ix.get("hierarchical", {})
        base = cls()

        def side(sd, dflt):
            if not sd:
                return dflt
            groups = tuple(Group(tuple(g["modes"])) for g in sd.get("groups", []))
            for g, gd in zip(groups, sd.get("groups", [])):
                if "size" in gd and gd["size"] != len(g.modes):
                    raise ConfigError(f"group size {gd['size']} != {len(g.modes)} modes")
            swa_only = 2 if sd.get("first_two_layers") == "swa_only" else int(sd.get("swa_only_layers", 0))
            return Side(int(sd.get("layers", dflt.layers)), int(sd.get("compression_ratio", dflt.compression_ratio)),
                        groups or dflt.groups, swa_only)

        hb = base.indexer.hierarchical
        cfg = cls(
            global_kv_dtype=kv.get("global_kv_dtype", base.global_kv_dtype),
            global_kv_scale=kv.get("global_kv_scale", base.global_kv_scale),
            swa_kv_dtype=kv.get("swa_kv_dtype", base.swa_kv_dtype),
            swa_window_size=int(kv.get("swa_window_size", base.swa_window_size)),
            index_key_dtype=d.get("index_key_dtype", base.index_key_dtype),
            indexer=Indexer(
                query_heads=int(ix.get("query_heads", base.indexer.query_heads)),
                head_dim=int(ix.get("head_dim", base.indexer.head_dim)),
                top_k=int(ix.get("top_k", base.indexer.top_k)),
                hierarchical=Hierarchical(
                    enabled=bool(hi.get("enabled", hb.enabled)),
                    max_blocks=int(hi.get("max_blocks", hb.max_blocks)),
                    positions_per_block=int(hi.get("positions_per_block", hb.positions_per_block)),
                    candidate_pool_size=int(hi.get("candidate_pool_size", hb.candidate_pool_size)))),
            encoder=side(cs.get("encoder"), base.encoder),
            decoder=side(cs.get("decoder"), base.decoder))
        cfg.validate()
        return cfg

    # -- checking -----------------------------------------------------------

    def validate(self):
        """Raise ConfigError for a configuration the kernels do not implement."""
        def need(ok, msg):
            if not ok:
                raise ConfigError(msg)

        need(self.global_kv_dtype == "fp4_e2m1", f"global_kv_dtype {self.global_kv_dtype!r}: only fp4_e2m1")
        need(self.global_kv_scale == f"e4m3_per_{SCALE_GROUP}_channel",
             f"global_kv_scale {self.global_kv_scale!r}: only e4m3_per_16_channel")
        need(self.swa_kv_dtype in ("fp8", "fp8_e4m3", "e4m3"), f"swa_kv_dtype {self.swa_kv_dtype!r}: only fp8 (E4M3)")
        need(self.swa_window_size >= 1, "swa_window_size must be positive")
        need(self.index_key_dtype in ("e4m3", "fp4_e2m1"), f"index_key_dtype {self.index_key_dtype!r}")
        ix, hb = self.indexer, self.indexer.hierarchical
        need(ix.query_heads == 32 and ix.head_dim == 128,
             f"indexer {ix.query_heads}x{ix.head_dim}: the kernels implement 32 heads x 128 dims")
        need(1 <= ix.top_k <= MAX_TOPK, f"top_k {ix.top_k} outside [1, {MAX_TOPK}]")
        if hb.enabled:
            need(hb.positions_per_block == 8, f"positions_per_block {hb.positions_per_block}: the block keys are 8 wide")
            need(1 <= hb.max_blocks <= MAX_TOPK, f"max_blocks {hb.max_blocks} outside [1, {MAX_TOPK}]")
            need(hb.candidate_pool_size == hb.max_blocks * hb.positions_per_block,
                 f"candidate_pool_size {hb.candidate_pool_size} != max_blocks x positions_per_block")
        for name, sd in (("encoder", self.encoder), ("decoder", self.decoder)):
            need(sd.compression_ratio in (1, 2, 4), f"{name} compression_ratio {sd.compression_ratio}: 1, 2 or 4")
            n = sd.swa_only_layers + sum(len(g.modes) for g in sd.groups)
            need(n == sd.layers, f"{name}: {n} layers in its groups, {sd.layers} declared")
            for g in sd.groups:
                need(g.modes and g.modes[0] in ("full", "reindex"), f"{name}: a group starts with full or reindex")
                need(all(m in _MODES for m in g.modes) and all(m == "reuse" for m in g.modes[1:]),
                     f"{name}: group modes {g.modes}")
            need(sd.groups[0].modes[0] == "full" if sd.groups else True, f"{name}: the first group builds the cache")

    # -- ABI integers -------------------------------------------------------

    @property
    def key_format(self):
        return KEY_FP4 if self.index_key_dtype == "fp4_e2m1" else KEY_E4M3

    def index_entry_bytes(self):
        return 64 + 4 if self.key_format == KEY_FP4 else 128

    def main_entry_bytes(self):
        return LATENT_DIM // 2 + LATENT_DIM // SCALE_GROUP

    def indexer_kwargs(self, hierarchical=None):
        """Keyword arguments of csa2.indexer_topk for a Full layer's
        selection: top_k and, when hierarchical, keep_blocks (block_keys and
        the key buffers are the caller's tensors)."""
        h = self.indexer.hierarchical.enabled if hierarchical is None else hierarchical
        kw = dict(top_k=self.indexer.top_k)
        if h:
            kw["keep_blocks"] = self.indexer.hierarchical.max_blocks
        return kw

    def attn_kwargs(self):
        """Keyword arguments of csa2.sparse_attn_decode: the window bound."""
        return dict(swa_max=self.swa_window_size)

    def cache_kwargs(self, side):
        """Keyword arguments of csa2.kv_compress_quantize / decode_append for
        the caches of one side ("encoder" or "decoder"): the ratio m."""
        return dict(m=(self.encoder if side == "encoder" else self.decoder).compression_ratio)

    # -- layer table --------------------------------------------------------

    def layers(self):
        """Per-layer table (schedule.Layer): window-only layers first, then
        each group's layers; each encoder group builds its own cache, the
        decoder's groups share one (Reindex re-selects over it)."""
        out = []

        def add(side, mode, m, cache, group):
            out.append(_schedule.Layer(len(out), side, mode, m, cache, group))

        n_cache = n_group = 0
        for name, sd in (("encoder", self.encoder), ("decoder", self.decoder)):
            for _ in range(sd.swa_only_layers):
                add(name, "swa_only", sd.compression_ratio, -1, -1)
            side_cache = None
            for g in sd.groups:
                if g.modes[0] == "full":
                    side_cache = n_cache
                    n_cache += 1
                for mode in g.modes:
                    add(name, mode, sd.compression_ratio, side_cache, n_group)
                n_group += 1
        return out

    def global_bytes_per_token(self):
        """Global cache per token: every cache-building layer holds one
        (main + index) entry per m tokens."""
        return _schedule.global_bytes_per_token(self.layers(), self.main_entry_bytes(), self.index_entry_bytes())
