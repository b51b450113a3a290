"""Top-k rows whose threshold bin holds more scores than the row select keeps
in LDS (12,288), in one-stage calls that allocate no candidate area: the
select resolves such a row from its stored scores.  Expected ids follow from
the method's tie rule (equal scores go to the lower index), so they are exact:

* a row of zero queries scores every visible key 0: its top-k is the first k
  positions (flat) or the k lowest candidate ids (candidate lists);
* a row whose single non-zero query dim meets keys whose matching dim is 1.0
  or 1.5 (all other key dims zero): every score is 32 * w_sum * that value,
  so about 70 % of the keys tie at the top.

Paths: 4 rows (per-row scan) and 256 rows (row-group scan) over 32,768
entries; a call of 4,100 rows over 524,288 entries whose last pass through
the score block holds fewer rows than the others; candidate lists of 20,000
ids."""

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


def tie_keys(g, N):
    """Keys whose dim 0 is 1.0 (30 %) or 1.5 (70 %), other dims zero."""
    k = np.zeros((N, 128), np.float32)
    k[:, 0] = np.where(g.random(N) < 0.7, 1.5, 1.0)
    return synth.to_e4m3(k)


def normal_q(g, R):
    return synth.to_e4m3(g.standard_normal((R, 32, 128)).astype(np.float32))


def run(q, keys, k, w=None, **kw):
    R = q.shape[0]
    out_score = torch.empty((R, k), dtype=torch.float32, device="cuda")
    idx = C.indexer_topk(dev(q), dev(keys), k, head_w=None if w is None else dev(w), out_score=out_score, **kw)
    torch.cuda.synchronize()
    return host(idx), host(out_score)


def expect_flat(q, w, keys, k, nv=None):
    nv = keys.shape[0] if nv is None else nv
    sc = O.index_scores(q, w, keys[:nv])
    return O.topk_select(sc, np.arange(nv), k), sc


@pytest.mark.parametrize("R", [4, 256])
def test_flat_rows_of_ties(R):
    """Sequence 0 holds normal keys, sequence 1 the tied keys; 32,768 entries
    each (the most a row selects without the filter stage)."""
    N, k = 32768, 512
    say(f"indexer flat: {R} rows over {N} entries with zero-query and tied rows, k={k}")
    g = np.random.default_rng(101 + R)
    keys = np.stack([synth.to_e4m3(g.standard_normal((N, 128)).astype(np.float32)), tie_keys(g, N)])
    q = normal_q(g, R)
    w = g.uniform(0.25, 1.0, (R, 32)).astype(np.float32)
    zero_rows = [0, R // 2, R - 1]
    q[zero_rows] = 0
    tie_row = 1
    q[tie_row] = 0
    q[tie_row, :, 0] = synth.to_e4m3(np.ones(32, np.float32))
    rs = np.zeros(R, np.int32)
    rs[tie_row] = 1
    gi, gsc = run(q, keys, k, w=w, row_seq=dev(rs))
    for r in zero_rows:
        assert np.array_equal(gi[r], np.arange(k)), f"row {r}: zero queries must keep positions 0..{k - 1}"
        assert np.all(gsc[r] == 0.0), f"row {r}: scores"
    ref, sc = expect_flat(q[tie_row], w[tie_row], keys[1], k)
    assert np.array_equal(gi[tie_row], np.sort(ref)), "tied row: ids differ from the lowest tied positions"
    assert np.all(gsc[tie_row] == gsc[tie_row][0]), "tied row: one score"
    assert abs(gsc[tie_row][0] - sc[ref[0]]) <= 2e-6 * abs(sc[ref[0]]), "tied row: score value"
    for r in (2, R // 2 + 1):                       # ordinary rows still agree
        ref, sc = expect_flat(q[r], w[r], keys[0], k)
        check_topk(gi[r], ref, np.arange(N), sc, k, f"row {r}")


def test_short_last_pass():
    """4,100 rows over 524,288 entries: the score rows take passes of 257
    rows through one score block, the last holding 245 -- fewer than a pass
    that may filter, in a call that allocated no candidate area for it.
    Zero-query rows in the first and the last pass."""
    N, R, k = 524288, 4100, 256
    say(f"indexer flat: {R} rows over {N} entries in passes, k={k}")
    g = np.random.default_rng(7)
    keys = synth.to_e4m3(g.standard_normal((N, 128)).astype(np.float32))
    q = normal_q(g, R)
    zero_rows = [3, R - 2]
    q[zero_rows] = 0
    gi, _ = run(q, keys[None], k, row_seq=dev(np.zeros(R, np.int32)))
    for r in zero_rows:
        assert np.array_equal(gi[r], np.arange(k)), f"row {r}"
    for r in (0, R - 1):
        ref, sc = expect_flat(q[r], None, keys, k)
        check_topk(gi[r], ref, np.arange(N), sc, k, f"row {r}")


def test_candidate_lists_of_ties():
    N, n_cand, k = 30000, 20000, 512
    say(f"indexer candidates: {n_cand} ids over {N} entries, zero-query row, k={k}")
    g = np.random.default_rng(5)
    keys = synth.to_e4m3(g.standard_normal((2, N, 128)).astype(np.float32))
    q = normal_q(g, 2)
    q[0] = 0
    cand = np.stack([g.permutation(N)[:n_cand] for _ in range(2)]).astype(np.int32)
    cand[:, ::41] = -1
    gi, gsc = run(q, keys, k, cand=dev(cand))
    ids0 = np.sort(cand[0][cand[0] >= 0])
    assert np.array_equal(gi[0], ids0[:k]), "zero-query row: the lowest candidate ids"
    assert np.all(gsc[0] == 0.0)
    ids1 = cand[1][cand[1] >= 0]
    sc = O.index_scores(q[1], None, keys[1][ids1])
    check_topk(gi[1], O.topk_select(sc, ids1, k), ids1, sc, k, "row 1")
