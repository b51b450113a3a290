"""The package's layer schedule against the oracle's expansion of the
pages' configuration (tests/golden/pages_config.json)."""

import json
import os

from fp4_kv_cache_indexer_amd import schedule as S
from oracle import accounting as A

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_schedule_matches_pages_config():
    with open(os.path.join(GOLD, "pages_config.json")) as f:
        cfg = json.load(f)["csa2"]
    want = A.schedule_from_config(cfg)
    layers = S.csa2_layers()
    assert [(ly.mode, ly.m) for ly in layers] == want
    assert [ly.index for ly in layers] == list(range(40))


def test_caches_and_groups():
    layers = S.csa2_layers()
    assert S.cache_ratios(layers) == [2, 2, 2, 1]
    # every Reuse/Reindex layer reads the cache its group's Full layer built,
    # and the Reindex layers read the decoder cache
    full_of = {ly.group: ly.cache for ly in layers if ly.mode == "full"}
    for ly in layers:
        if ly.mode == "reuse":
            assert ly.cache == [x for x in layers if x.group == ly.group][0].cache
        if ly.mode == "reindex":
            assert ly.cache == full_of[3] and ly.side == "decoder"
        if ly.mode == "swa_only":
            assert ly.cache == -1
    # the FP4 main entry (288 B) and FP4 index key (68 B) give 890 B/token
    assert S.global_bytes_per_token(layers, 288, 68) == 890
    assert S.global_bytes_per_token(layers, 288, 128) == 1040
