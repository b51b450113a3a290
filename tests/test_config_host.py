"""The configuration module (no GPU): the pages' configuration parses into
the ABI integers and the 40-layer table the schedule uses, and settings the
kernels do not implement are refused [0539edu §3]."""

import json
import os

import pytest

from fp4_kv_cache_indexer_amd import config as CF
from fp4_kv_cache_indexer_amd import schedule as SCH
from oracle import accounting as A

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_config.json")


def pages():
    with open(GOLDEN) as f:
        return json.load(f)


def test_pages_configuration_to_abi_integers():
    cfg = CF.Csa2Config.from_dict(pages())
    assert cfg == CF.Csa2Config()                         # the defaults are the pages' values
    assert cfg.indexer_kwargs() == dict(top_k=512, keep_blocks=2048)
    assert cfg.indexer_kwargs(hierarchical=False) == dict(top_k=512)
    assert cfg.attn_kwargs() == dict(swa_max=128)
    assert cfg.cache_kwargs("encoder") == dict(m=2) and cfg.cache_kwargs("decoder") == dict(m=1)
    assert cfg.key_format == CF.KEY_E4M3 and cfg.main_entry_bytes() == A.fp4_entry_bytes(512) == 288


def test_layer_table_equals_the_schedule():
    cfg = CF.Csa2Config.from_dict(pages())
    assert cfg.layers() == SCH.csa2_layers()
    assert len(cfg.layers()) == 40


def test_bytes_per_token_with_each_index_key():
    d = pages()
    assert CF.Csa2Config.from_dict(d).global_bytes_per_token() == 2.5 * (288 + 128)      # 1040
    d["index_key_dtype"] = "fp4_e2m1"
    cfg = CF.Csa2Config.from_dict(d)
    assert cfg.key_format == CF.KEY_FP4 and cfg.global_bytes_per_token() == 890.0


@pytest.mark.parametrize("path,value", [
    (("kv_cache", "global_kv_dtype"), "fp8"),
    (("kv_cache", "global_kv_scale"), "e4m3_per_32_channel"),
    (("csa2", "indexer", "query_heads"), 64),
    (("csa2", "indexer", "top_k"), 4096),
    (("csa2", "indexer", "hierarchical", "candidate_pool_size"), 8192),
    (("csa2", "indexer", "hierarchical", "positions_per_block"), 16),
    (("csa2", "encoder", "compression_ratio"), 3),
    (("csa2", "decoder", "layers"), 24),
])
def test_unsupported_settings_are_refused(path, value):
    d = pages()
    node = d
    for k in path[:-1]:
        node = node[k]
    node[path[-1]] = value
    with pytest.raises(CF.ConfigError):
        CF.Csa2Config.from_dict(d)


def test_group_size_must_match_its_modes():
    d = pages()
    d["csa2"]["decoder"]["groups"][1]["size"] = 5
    with pytest.raises(CF.ConfigError):
        CF.Csa2Config.from_dict(d)
