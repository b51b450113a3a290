"""Pins for the byte accounting against the figures the pages print
(tests/golden/pages_figures.json, tests/golden/pages_config.json)."""

import json
import os
from fractions import Fraction

from oracle import accounting as A

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_schedule_from_pages_config():
    cfg = load("pages_config.json")["csa2"]
    sch = A.schedule_from_config(cfg)
    assert len(sch) == 40
    assert sch[:2] == [("swa_only", 2)] * 2
    # four layers build a global cache: 3 encoder Full (m=2), 1 decoder Full (m=1)
    assert A.cache_layers(sch) == [2, 2, 2, 1]
    fig = load("pages_figures.json")["cache_layers_v41"]
    assert len(A.cache_layers(sch)) == fig["layers_producing_global_kv"]
    assert sum(1 for mode, _ in sch if mode == "reindex") == 4


def test_fp4_entry_and_890_bytes_per_token():
    cfg = load("pages_config.json")
    sch = A.schedule_from_config(cfg["csa2"])
    dim = load("pages_figures.json")["cache_layers_v41"]["latent_dim_shared_by_all_heads"]
    entry = A.fp4_entry_bytes(dim, group=16)
    assert entry == 288
    main = A.bytes_per_token(sch, entry)
    assert main == 720                                       # 1.5 + 1 entries/token x 288 B
    total = load("pages_figures.json")["global_kv_bytes_per_token"]["DeepSeek-V4.1-Flash"]
    # the remainder is the index keys: 2.5 entries/token share 170 B -> 68 B per
    # entry, e.g. 128 channels of FP4 plus a 4-byte scale
    idx_entry = A.fp4_entry_bytes(128, group=128, scale_bytes=4)
    assert idx_entry == 68
    assert A.bytes_per_token(sch, entry, idx_entry) == total
    # the FP8 128-dim index key of the kernels' layout would give 1040 B/token
    assert A.bytes_per_token(sch, entry, A.fp8_entry_bytes(128)) == 1040


def test_fp4_nearly_halves_fp8_main_kv():
    r = Fraction(A.fp4_entry_bytes(512), A.fp8_entry_bytes(512))
    assert r == Fraction(9, 16) and 0.5 < r < 0.6


def test_generation_ratios():
    fig = load("pages_figures.json")
    b = fig["global_kv_bytes_per_token"]
    r = fig["step_ratios"]
    assert round(b["DeepSeek-V1"] / b["DeepSeek-V3.2"], 1) == r["V1_to_V3.2"]
    assert round(b["DeepSeek-V3.2"] / b["DeepSeek-V4-Flash"], 1) == r["V3.2_to_V4-Flash"]
    assert round(b["DeepSeek-V4-Flash"] / b["DeepSeek-V4.1-Flash"], 1) == r["V4-Flash_to_V4.1-Flash"]
    assert round(b["DeepSeek-V1"] / b["DeepSeek-V4.1-Flash"]) == r["V1_to_V4.1-Flash_overall"]
    p = fig["v4flash_vs_v32_kv_percent"]
    assert round(100 * b["DeepSeek-V4-Flash"] / b["DeepSeek-V3.2"], 1) == p["computed_from_table"]
    assert round(100 * b["DeepSeek-V4-Flash"] / b["DeepSeek-V3.2"]) == p["stated"]
    gb = fig["per_million_tokens_GB"]
    for model, bytes_tok in b.items():
        if model.startswith("_"):
            continue
        v = A.kv_bytes(1_000_000, 1, bytes_tok, 1) / 1e9
        assert abs(v - gb[model]) <= 0.5 * 10 ** -(len(str(gb[model]).split(".")[-1]) if "." in str(gb[model]) else 0) + 1e-9


def test_dense_worked_example():
    ex = load("pages_figures.json")["dense_kv_worked_example"]
    per_layer = A.kv_bytes(1, 1, 2 * ex["kv_heads"] * ex["head_dim"], ex["bytes_per_number"])
    assert per_layer == ex["bytes_per_token_per_layer"]
    assert A.kv_bytes(1, ex["layers"], 2 * ex["kv_heads"] * ex["head_dim"],
                      ex["bytes_per_number"]) == ex["bytes_per_token"]
    total = A.kv_bytes(ex["context_tokens"], ex["layers"], 2 * ex["kv_heads"] * ex["head_dim"],
                       ex["bytes_per_number"])
    assert total == ex["total_GB"] * 2 ** 30
