"""Pins for the oracle's indexer and top-k: brute force on tiny inputs with
pure-Python loops, constructed ties, invariances, and the identity of the
hierarchical and flat selections when the pool covers every entry."""

import numpy as np

from oracle import csa2 as O
from oracle import formats as F
from fp4_kv_cache_indexer_amd.synth import to_e4m3


def small(seed, N, heads=32, dim=128):
    g = np.random.default_rng(seed)
    q = to_e4m3(g.standard_normal((heads, dim)).astype(np.float32))
    k = to_e4m3(g.standard_normal((N, dim)).astype(np.float32))
    w = g.uniform(0.25, 1.0, heads).astype(np.float32)
    return q, w, k


def brute_scores(q, w, keys):
    qd, kd = F.e4m3_decode(q), F.e4m3_decode(keys)
    out = []
    for t in range(kd.shape[0]):
        tot = 0.0
        for h in range(qd.shape[0]):
            d = 0.0
            for i in range(qd.shape[1]):
                d += qd[h, i] * kd[t, i]
            tot += float(w[h]) * (d if d > 0 else 0.0)
        out.append(tot)
    return np.array(out)


def brute_topk(scores, ids, k):
    pairs = sorted(zip(scores.tolist(), ids.tolist()), key=lambda p: (-p[0], p[1]))
    sel = sorted(i for _, i in pairs[:k])
    return sel + [-1] * (k - len(sel))


def test_scores_brute_force():
    q, w, k = small(10, 12, heads=4, dim=16)
    assert np.allclose(O.index_scores(q, w, k), brute_scores(q, w, k), rtol=1e-12, atol=1e-12)
    # a key orthogonal-ish / all-negative dots gives exactly 0
    kneg = to_e4m3(-np.abs(F.e4m3_decode(q[:1])).astype(np.float32))
    qpos = to_e4m3(np.abs(F.e4m3_decode(q)).astype(np.float32))
    assert O.index_scores(qpos, w, kneg)[0] == 0.0


def test_relu_per_head_not_linear():
    # one head positive, one negative: the ReLU keeps only the positive one
    q = to_e4m3(np.array([[1.0, 0.0], [-1.0, 0.0]], dtype=np.float32))
    k = to_e4m3(np.array([[2.0, 5.0]], dtype=np.float32))
    assert O.index_scores(q, np.array([1.0, 1.0]), k)[0] == 2.0
    assert O.index_scores(q, np.array([0.5, 3.0]), k)[0] == 1.0


def test_topk_brute_force_with_ties():
    g = np.random.default_rng(11)
    for trial in range(20):
        n = int(g.integers(1, 40))
        k = int(g.integers(1, 20))
        s = g.integers(0, 5, n).astype(np.float64)   # many exact ties
        ids = np.arange(n)
        got = O.topk_select(s, ids, k).tolist()
        assert got == brute_topk(s, ids, k)


def test_flat_topk_brute_force_duplicated_keys():
    q, w, k = small(12, 48)
    k[20:30] = k[5]          # equal scores: lower indices must win
    k[40:48] = k[1]
    s = brute_scores(q, w, k)
    for kk in (1, 5, 8, 16, 47, 48, 60):
        assert O.indexer_topk_flat(q, w, k, kk).tolist() == brute_topk(s, np.arange(48), kk)


def test_n_valid_and_padding():
    q, w, k = small(13, 30)
    out = O.indexer_topk_flat(q, w, k, 16, n_valid=10)
    assert out[:10].tolist() == list(range(10)) and (out[10:] == -1).all()
    out = O.indexer_topk_flat(q, w, k, 4, n_valid=0)
    assert (out == -1).all()


def test_uniform_weight_scale_invariance():
    q, _, k = small(14, 200)
    a = O.indexer_topk_flat(q, np.ones(32), k, 17)
    b = O.indexer_topk_flat(q, np.full(32, 3.5), k, 17)
    assert np.array_equal(a, b)


def test_permutation_equivariance():
    q, w, k = small(15, 120)
    perm = np.random.default_rng(0).permutation(120)
    a = O.indexer_topk_flat(q, w, k, 20)
    b = O.indexer_topk_flat(q, w, k[perm], 20)
    assert np.array_equal(np.sort(perm[b]), a)


def test_hierarchical_equals_flat_when_pool_covers_all():
    q, w, k = small(16, 203)
    bk = O.block_summary(k)
    flat = O.indexer_topk_flat(q, w, k, 32)
    hier, kept = O.indexer_topk_hier(q, w, k, bk, 32, keep_blocks=26)
    assert len(kept) == 26 and np.array_equal(hier, flat)
    # with a smaller budget the result comes from the kept blocks only
    hier, kept = O.indexer_topk_hier(q, w, k, bk, 32, keep_blocks=5)
    assert set((hier // 8).tolist()) <= set(kept.tolist())


def test_hierarchical_coarse_brute_force():
    q, w, k = small(17, 90)
    bk = O.block_summary(k)
    sb = brute_scores(q, w, bk)
    kept, _ = O.coarse_blocks(q, w, bk, 90, 4)
    assert kept.tolist() == brute_topk(sb, np.arange(len(sb)), 4)
    # blocks holding no visible entry are not candidates
    kept, _ = O.coarse_blocks(q, w, bk, 17, 10)
    assert kept.max() <= 2
    cand = O.pool_positions(kept, 17)
    assert cand.max() == 16 and np.all(np.diff(cand) > 0)


def test_pool_restricted_selection_brute_force():
    q, w, k = small(18, 64)
    cand = np.array([3, 9, 10, 11, 40, 63, -1, 70])
    s = brute_scores(q, w, k)
    valid = np.array([3, 9, 10, 11, 40, 63])
    got = O.indexer_topk_pool(q, w, k, cand, 4).tolist()
    assert got == brute_topk(s[valid], valid, 4)
