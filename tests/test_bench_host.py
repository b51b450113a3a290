"""Host checks of bench.py's oracle leg for the prefill step (no GPU): the
bounded sample runs the oracle on a small prefill shape and reports a rate
over the whole step with the sample it took."""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _bf16_bits(a):
    u = np.asarray(a, np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_prefill_cpu_baseline_small_shape():
    rng = np.random.default_rng(3)
    T, m, R, H, k, W = 2048, 2, 64, 16, 64, 128
    w = dict(T=T, m=m, R=R, H=H, k=k, W=W)
    xb, zb = _bf16_bits(rng.standard_normal((T, 512))), _bf16_bits(rng.standard_normal((T, 512)))
    kb = rng.integers(0, 0x70, (T // m, 128), dtype=np.uint8)
    qi = rng.integers(0, 0x70, (R, 32, 128), dtype=np.uint8)
    hw = rng.random((R, 32)) * 0.75 + 0.25
    qb = _bf16_bits(rng.standard_normal((R, H, 512)))
    base = T - R - (W - 1)
    sw = rng.integers(0, 0x70, (T - base, 512), dtype=np.uint8)
    res = bench.cpu_baseline_prefill(w, xb, zb, kb, qi, hw, qb, sw, base, 0.0, write_stride=8, row_stride=16)
    assert res["kind"] == "oracle" and res["unit"] == "queries/s"
    assert res["value"] > 0 and res["cores"] >= 1
    # at least two rows are always sampled; the cache write covers 1 in 8 entries
    assert "of 2 rows strided by 16" in res["sample"]
    assert "1 in 8 entries (128 entries" in res["sample"]
