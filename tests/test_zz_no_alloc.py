"""The indexer entry point that allocates nothing (csa2_indexer_topk_static)
against csa2_indexer_topk with a caller workspace: bit-equal ids, scores
and kept blocks over consecutive calls that share the static scratch (a
large hierarchical call, a smaller flat one, the large one again), and a
request beyond the static size refused before anything runs."""

import numpy as np
import pytest
import torch

from fp4_kv_cache_indexer_amd import csa2 as C
from fp4_kv_cache_indexer_amd import synth
from oracle import csa2 as O
from parity import check_topk, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    C.lib()
    yield
    torch.cuda.synchronize()


def case(seed, S, N, R, row_seq, n_valid):
    g = np.random.default_rng(seed)
    keys = synth.to_e4m3(g.standard_normal((S, N, 128)).astype(np.float32))
    q = synth.to_e4m3(g.standard_normal((R, 32, 128)).astype(np.float32))
    w = g.uniform(0.25, 1.0, (R, 32)).astype(np.float32)
    return dict(keys=dev(keys), q=dev(q), w=dev(w), row_seq=dev(np.asarray(row_seq, np.int32)),
                n_valid=dev(np.asarray(n_valid, np.int32)), host_keys=keys)


def both(c, k, hier=None):
    """The same selection through both entry points; returns their outputs."""
    R = c["q"].shape[0]
    outs = []
    for static in (False, True):
        out_score = torch.full((R, k), -7.0, dtype=torch.float32, device="cuda")
        out_blocks = torch.full((R, hier), -7, dtype=torch.int32, device="cuda") if hier else None
        kw = dict(head_w=c["w"], row_seq=c["row_seq"], n_valid=c["n_valid"], out_score=out_score)
        if hier:
            kw.update(block_keys=c["summ"], keep_blocks=hier, out_blocks=out_blocks)
        f = C.indexer_topk_static if static else C.indexer_topk
        idx = f(c["q"], c["keys"], k, **kw)
        torch.cuda.synchronize()
        outs.append((host(idx), host(out_score), None if out_blocks is None else host(out_blocks)))
    return outs


def test_static_scratch_equals_workspace_entry_point():
    big = case(61, 4, 200003, 8, [0, 1, 2, 3, 3, 2, -1, 0], [200003, 150001, 200003, 7, 0, 99999, 5, 123457])
    big["summ"] = C.index_block_summary(big["keys"])
    small = case(62, 2, 5000, 3, [1, 0, 1], [5000, 4097, 300])
    need = [C.indexer_topk_workspace(big["q"], big["keys"], 512, block_keys=big["summ"], keep_blocks=512),
            C.indexer_topk_workspace(small["q"], small["keys"], 256)]
    say(f"scratch needed: hierarchical call {need[0]} B, flat call {need[1]} B (static {C.STATIC_SCRATCH_BYTES} B)")
    assert need[1] < need[0] <= C.STATIC_SCRATCH_BYTES
    got = {}
    for name, c, k, hier in (("hierarchical", big, 512, 512), ("flat, smaller", small, 256, None),
                             ("hierarchical again", big, 512, 512)):
        say(f"  {name}")
        (ia, sa, ba), (ib, sb, bb) = both(c, k, hier)
        assert np.array_equal(ia, ib), name
        assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32)), name
        if hier:
            assert np.array_equal(ba, bb), name
        got[name] = ib
    # the flat call is also the oracle's selection
    for r in range(3):
        s, nv = int(host(small["row_seq"])[r]), int(host(small["n_valid"])[r])
        sc = O.index_scores(host(small["q"])[r], host(small["w"])[r], small["host_keys"][s][:nv])
        check_topk(got["flat, smaller"][r], O.topk_select(sc, np.arange(nv), 256), np.arange(nv), sc, 256,
                   f"flat row {r}")


def test_static_scratch_refuses_larger_requests():
    # 64 rows of flat 262144-entry scans need far more than the static array
    q = torch.zeros((64, 32, 128), dtype=torch.uint8, device="cuda")
    keys = torch.zeros((64, 262144, 128), dtype=torch.uint8, device="cuda")
    assert C.indexer_topk_workspace(q, keys, 512) > C.STATIC_SCRATCH_BYTES
    with pytest.raises(C.Csa2Error) as e:
        C.indexer_topk_static(q, keys, 512)
    assert e.value.status == 3 and "static" in str(e.value)
