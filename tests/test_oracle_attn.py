"""Pins for the oracle's joint sparse + sliding-window attention: dense
attention through PyTorch's scaled_dot_product_attention (an independent
library routine) when the selection covers every entry, single-key and
empty cases, set invariance, layer reuse, prefill visibility."""

import math

import numpy as np
import torch

from oracle import csa2 as O
from oracle import formats as F
from fp4_kv_cache_indexer_amd import synth


def case(N=96, H=8, cap=40, seed=20):
    c = synth.make_decode_case(seed=seed, cfg=99, S=1, N=N, H=H, swa_cap=cap, swa_len=cap,
                               outliers=True)
    codes, scales = O.kv_compress_quantize(c.x_bits[0], None, 1)
    return c, codes, scales


def sdpa(q, K, scale):
    qt = torch.from_numpy(q)[None]          # [1, H, D] as (batch, L, E) with L = H rows
    kt = torch.from_numpy(K)[None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)
    lse = torch.logsumexp(qt @ kt.transpose(1, 2) * scale, dim=-1)
    return out[0].numpy(), lse[0].numpy()


def test_sparse_covering_all_equals_dense_sdpa():
    c, codes, scales = case()
    idx = O.indexer_topk_flat(c.q_idx[0], c.w_idx[0], c.keys[0], 128)  # k >= N: every entry
    assert (idx[:96] == np.arange(96)).all()
    slots = O.swa_slots(0, 40, 40)
    Ox, lse = O.sparse_attn(c.q[0], codes, scales, idx, c.swa[0], slots)
    K = np.concatenate([O.dequantize_fp4(codes, scales), F.e4m3_decode(c.swa[0])])
    q = F.bf16_bits_to_f64(c.q[0])
    Oref, lref = sdpa(q, K, 1 / math.sqrt(512))
    assert np.allclose(Ox, Oref, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, lref, rtol=1e-12, atol=1e-12)


def test_single_key_and_empty():
    c, codes, scales = case()
    Ox, lse = O.sparse_attn(c.q[0], codes, scales, [7, -1, -1], c.swa[0], [])
    v = O.dequantize_fp4(codes[7:8], scales[7:8])[0]
    assert np.array_equal(Ox, np.tile(v, (8, 1)))
    q = F.bf16_bits_to_f64(c.q[0])
    assert np.allclose(lse, q @ v / math.sqrt(512), rtol=1e-13)
    Ox, lse = O.sparse_attn(c.q[0], codes, scales, [-1, -1], c.swa[0], [])
    assert (Ox == 0).all() and np.isneginf(lse).all()


def test_swa_only_and_global_only_are_dense_sdpa():
    c, codes, scales = case()
    q = F.bf16_bits_to_f64(c.q[0])
    Ox, _ = O.sparse_attn(c.q[0], codes, scales, [-1] * 4, c.swa[0], O.swa_slots(30, 20, 40))
    slots = [(30 + j) % 40 for j in range(20)]
    Oref, _ = sdpa(q, F.e4m3_decode(c.swa[0][slots]), 1 / math.sqrt(512))
    assert np.allclose(Ox, Oref, rtol=1e-12, atol=1e-12)
    sel = np.array([90, 3, 44, -1, 17])
    Ox, _ = O.sparse_attn(c.q[0], codes, scales, sel, c.swa[0], [], sm_scale=0.125)
    Oref, _ = sdpa(q, O.dequantize_fp4(codes[[90, 3, 44, 17]], scales[[90, 3, 44, 17]]), 0.125)
    assert np.allclose(Ox, Oref, rtol=1e-12, atol=1e-12)


def test_key_set_invariance():
    c, codes, scales = case()
    a, la = O.sparse_attn(c.q[0], codes, scales, [5, 9, 60, -1], c.swa[0], O.swa_slots(0, 12, 40))
    b, lb = O.sparse_attn(c.q[0], codes, scales, [-1, 60, 5, 9], c.swa[0], O.swa_slots(28, 12, 40)[::-1])
    # the same keys in another order (slots 28..39 hold other tokens, so compare
    # against a ring that wraps onto the same tokens)
    b2, lb2 = O.sparse_attn(c.q[0], codes, scales, [-1, 60, 5, 9], c.swa[0],
                            list(reversed(O.swa_slots(0, 12, 40))))
    assert np.allclose(a, b2, rtol=1e-12, atol=1e-12) and np.allclose(la, lb2, rtol=1e-12)
    assert not np.allclose(a, b)


def test_layer_group_reuse_and_reindex():
    c, codes, scales = case(N=200, H=4)
    g = np.random.default_rng(3)
    L = 4
    q_attn = [c.q[0]] * L
    q_idx = [c.q_idx[0], None, c.q_idx[0], None]
    w_idx = [c.w_idx[0], None, c.w_idx[0], None]
    swa = [c.swa[0]] * L
    out = O.layer_group(["full", "reuse", "reindex", "reuse"], q_attn, q_idx, w_idx,
                        codes, scales, c.keys[0], swa, O.swa_slots(0, 40, 40), 32)
    # same queries everywhere -> every layer equals the Full layer
    for idx, Ox, lse in out[1:]:
        assert np.array_equal(idx, out[0][0]) and np.array_equal(Ox, out[0][1])
    # a Reindex layer with a new indexer query selects anew; the Reuse after it follows it
    q2 = synth.to_e4m3(g.standard_normal((32, 128)).astype(np.float32))
    out = O.layer_group(["full", "reuse", "reindex", "reuse"], q_attn, [c.q_idx[0], None, q2, None],
                        w_idx, codes, scales, c.keys[0], swa, O.swa_slots(0, 40, 40), 32)
    assert np.array_equal(out[2][0], O.indexer_topk_flat(q2, w_idx[2], c.keys[0], 32))
    assert np.array_equal(out[3][0], out[2][0]) and not np.array_equal(out[2][0], out[0][0])


def test_layer_group_reindex_in_pool():
    """A Reindex layer restricted to the Full layer's pool: brute force over
    the pool's positions, and equal to the unrestricted (hierarchical)
    Reindex when the pool covers every entry."""
    c, codes, scales = case(N=203, H=4)
    g = np.random.default_rng(5)
    keys = c.keys[0]
    bk = O.block_summary(keys)
    q1, q2 = c.q_idx[0], synth.to_e4m3(g.standard_normal((32, 128)).astype(np.float32))
    w = g.uniform(0.25, 1.0, 32)
    modes = ["full", "reuse", "reindex"]
    L = len(modes)
    args = dict(q_attn=[c.q[0]] * L, q_idx=[q1, None, q2], w_idx=[w, None, w], codes=codes, scales=scales,
                keys=keys, swa=[c.swa[0]] * L, slots=O.swa_slots(0, 40, 40), k=16, block_keys=bk)
    out = O.layer_group(modes, keep_blocks=6, reindex_in_pool=True, **args)
    # brute force: the Full layer's six best blocks (ties to the lower id),
    # their positions, then the reindex query's best 16 there
    sb = [sum(wi * max(0.0, float(np.dot(F.e4m3_decode(q2b), F.e4m3_decode(kb))))
              for wi, q2b in zip(w, q1)) for kb in bk]
    blocks = sorted(sorted(range(len(bk)), key=lambda b: (-sb[b], b))[:6])
    pool = [8 * b + i for b in blocks for i in range(8) if 8 * b + i < len(keys)]
    sp = {p: sum(wi * max(0.0, float(np.dot(F.e4m3_decode(qr), F.e4m3_decode(keys[p]))))
                 for wi, qr in zip(w, q2)) for p in pool}
    want = sorted(sorted(pool, key=lambda p: (-sp[p], p))[:16])
    assert out[2][0].tolist() == want
    # restricting to a pool that covers everything changes nothing
    full = O.layer_group(modes, keep_blocks=26, reindex_in_pool=True, **args)
    free = O.layer_group(modes, keep_blocks=26, reindex_in_pool=False, **args)
    assert np.array_equal(full[2][0], free[2][0]) and np.array_equal(full[2][1], free[2][1])


def test_prefill_row_view():
    assert O.prefill_row_view(0, 2) == (0, 0, 1)
    assert O.prefill_row_view(1, 2) == (1, 0, 2)
    assert O.prefill_row_view(2, 2) == (1, 0, 3)
    assert O.prefill_row_view(5, 1) == (6, 0, 6)
    assert O.prefill_row_view(200, 2) == (100, 73, 128)
    # the visible entries are exactly those whose m tokens are all <= p
    for m in (1, 2, 4):
        for p in range(40):
            nv = O.prefill_row_view(p, m)[0]
            assert all((m * i + m - 1 <= p) == (i < nv) for i in range(20))
