"""Matrix-core precision of the indexer's head scores: the 128-term E4M3 dot
products through the fp16 MFMA (the scans' arithmetic) and the fp8 MFMA,
against the exact sums.

Every product of two E4M3 values is exact in float64, and so is every sum of
128 of them (the products span 2^-18 .. 2^18 with 8 significant bits), so
numpy's float64 matmul of the decoded values is the exact dot product.  The
error of a float32 summation of n terms is at most about n * 2^-24 times the
sum of their magnitudes; the fp16 path (four MFMA steps of 32 exact
products) must stay inside that bound.  The fp8 path's error is measured
and printed: it is the evidence for keeping the scans on fp16.

Inputs: 256 queries x 1024 keys of 128 dims, E4M3 of N(0,1) and of
Student-t(3) with 8 dims scaled by 8 (heavy tails)."""

import numpy as np
import pytest
import torch

from fp4_kv_cache_indexer_amd import csa2 as C
from fp4_kv_cache_indexer_amd import synth
from oracle import formats as F
from parity import dev, host, say

pytestmark = pytest.mark.gpu

F32_SUM_BOUND = 128 * 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    C.lib()


@pytest.mark.parametrize("dist", ["normal", "t3"])
def test_fp16_path_exact_to_float32_and_fp8_path_measured(dist):
    g = synth.rng(5, 3, synth.T_QIDX)
    och = np.arange(0, 128, 16) if dist == "t3" else None
    q = synth.to_e4m3(synth.latent_np(g, (256, 128), dist, och))
    k = synth.to_e4m3(synth.latent_np(g, (1024, 128), dist, och))
    o16, o8 = C.mfma_dot_probe(dev(q), dev(k))
    torch.cuda.synchronize()
    qf, kf = F.e4m3_decode(q).astype(np.float64), F.e4m3_decode(k).astype(np.float64)
    exact = qf @ kf.T
    mag = np.abs(qf) @ np.abs(kf).T
    mag = np.where(mag > 0, mag, 1.0)
    e16 = np.abs(host(o16).astype(np.float64) - exact) / mag
    e8 = np.abs(host(o8).astype(np.float64) - exact) / mag
    say(f"  {dist}: fp16 path max {e16.max():.3g}, median {np.median(e16):.3g} of sum |q_i k_i|; "
        f"fp8 path max {e8.max():.3g}, median {np.median(e8):.3g}, "
        f"{np.mean(e8 > F32_SUM_BOUND) * 100:.1f}% of pairs beyond the float32 bound {F32_SUM_BOUND:.3g}")
    assert e16.max() <= F32_SUM_BOUND, "fp16 matrix-core path outside the float32 summation bound"
    assert e8.max() < 2.0 ** -6, "fp8 path error larger than ever measured"
