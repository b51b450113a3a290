"""The timing probes behind the scan and attention designs run and read what
they claim: the block-summary scan's two load shapes (half lines per lane,
whole lines per instruction), plain or non-temporal, read the same bytes the
same number of times, so the XOR of all their output words agrees; the
MFMA/vector-issue and gather probes complete.  Their timings are printed by
`bench.py --probe scan|mfma-valu|gather`."""

import functools

import pytest
import torch

from fp4_kv_cache_indexer_amd import csa2 as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    C.lib()


def xor_all(t):
    return functools.reduce(lambda a, b: a ^ b, t.cpu().tolist(), 0)


@pytest.mark.parametrize("n_keys,chunk", [(1000, 256), (4096, 1376), (333, 16)])
def test_scan_probe_shapes_read_the_same_bytes(n_keys, chunk):
    g = torch.Generator(device="cuda").manual_seed(n_keys)
    keys = torch.randint(0, 256, (3, n_keys, 128), dtype=torch.uint8, device="cuda", generator=g)
    folds = {(full, nt): xor_all(C.probe_scan_read(keys, chunk, full, nt))
             for full in (False, True) for nt in (False, True)}
    torch.cuda.synchronize()
    assert len(set(folds.values())) == 1, folds


def test_mfma_valu_and_gather_probes_run():
    for nv in (0, 8):
        out = C.probe_mfma_valu(nv, 256, 4, 2)
        assert torch.isfinite(out).all()
    codes = torch.randint(0, 256, (1000, 256), dtype=torch.uint8, device="cuda")
    scales = torch.randint(0, 256, (1000, 32), dtype=torch.uint8, device="cuda")
    ids = torch.randint(-5, 1005, (6, 512), dtype=torch.int32, device="cuda")   # clamped into [0, 1000)
    for whole in (False, True):
        C.probe_gather(codes, scales, ids, 3, whole)
    torch.cuda.synchronize()
