"""Attention geometry invariance: the same rows through the 16-head (narrow)
and 64-head (tile) kernels, each at two key-split counts (one split
included), pinned with
csa2_attn_plan_override.  Every geometry must meet the oracle's attention
tolerance on the same inputs; the spread between geometries is printed.

Inputs: 6 rows over 3 sequences of 8192 FP4 entries (outlier channels),
64 heads, top-512 ids drawn per row (a few -1 slots, skipped), windows of
128, 97 and 0 tokens in a ring of 128 with rotated starts (ragged tails in
the last chunk of every split)."""

import numpy as np
import pytest
import torch

from fp4_kv_cache_indexer_amd import csa2 as C
from fp4_kv_cache_indexer_amd import synth
from oracle import csa2 as O
from parity import check_close, dev, host, say

pytestmark = pytest.mark.gpu

GEOMETRIES = [(16, 1), (16, 5), (64, 1), (64, 4)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    C.lib()
    yield
    C.attn_plan_override(0, 0)
    torch.cuda.synchronize()


def test_attention_geometry_invariance():
    S, N, H, k, R = 3, 8192, 64, 512, 6
    c = synth.make_decode_case(seed=3, cfg=2, S=S, N=N, H=H, top_k=k, R=R, outliers=True)
    codes, scales = C.kv_compress_quantize(dev(c.x_bits), 1)
    rng = np.random.default_rng(7)
    idx_h = np.stack([rng.choice(N, size=k, replace=False) for _ in range(R)]).astype(np.int32)
    idx_h[1, ::37] = -1                                    # skipped slots
    swa_len_h = np.array([128, 97, 0, 128, 97, 128], dtype=np.int32)
    swa_start_h = np.array([0, 5, 0, 120, 31, 64], dtype=np.int32)
    idx, swa_len, swa_start = dev(idx_h), dev(swa_len_h), dev(swa_start_h)
    q, swa, row_seq = dev(c.q), dev(c.swa), dev(c.row_seq)
    codes_h, scales_h = host(codes), host(scales)

    refs = []
    for r in range(R):
        s = int(c.row_seq[r])
        slots = O.swa_slots(int(swa_start_h[r]), int(swa_len_h[r]), 128)
        refs.append(O.sparse_attn(c.q[r], codes_h[s], scales_h[s], idx_h[r], c.swa[s], slots))

    outs = {}
    try:
        for hpw, ns in GEOMETRIES:
            C.attn_plan_override(hpw, ns)
            ws_bytes = C.sparse_attn_workspace(q, idx, swa=swa, swa_len=swa_len, codes=codes)
            assert (ws_bytes > 0) == (ns > 1), f"workspace {ws_bytes} for {ns} splits"
            out, lse = C.sparse_attn_decode(q, codes, scales, idx, swa=swa, swa_start=swa_start,
                                            swa_len=swa_len, row_seq=row_seq)
            torch.cuda.synchronize()
            go, gl = host(out), host(lse)
            worst = 0.0
            for r in range(R):
                worst = max(worst, check_close(go[r], refs[r][0], f"{hpw} heads/wg, {ns} splits, row {r} out"))
                check_close(gl[r], refs[r][1], f"{hpw} heads/wg, {ns} splits, row {r} lse")
            say(f"  {hpw} heads per workgroup, {ns} splits: worst {worst:.3g} of the oracle bound")
            outs[(hpw, ns)] = go.astype(np.float64)
    finally:
        C.attn_plan_override(0, 0)

    scale = max(np.abs(o).max() for o in outs.values())
    base = outs[GEOMETRIES[0]]
    for g, o in outs.items():
        say(f"  max |{g} - {GEOMETRIES[0]}| = {np.abs(o - base).max() / scale:.3g} of max |out|")
