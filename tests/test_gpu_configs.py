"""GPU parity at the full sizes of the five workload configurations.

Every test runs the HIP path over the whole configuration, with the same
entry points and launch shapes the benchmark uses, and checks sampled
outputs against the oracle: sampled cache entries (the oracle quantises the
same seeded tokens itself), sampled indexer rows (the oracle scores every
visible entry of the row and selects its own top-k) and the attention of
those rows (the oracle quantises the selected entries and attends over them
with the row's window).  Inputs never come from the HIP path; where the
GPU's selection legitimately differs from the oracle's (a swap inside the
1e-5 tie band, accepted by check_topk first), the next stage is judged on
the GPU's choice: the fine top-k on the pool of the blocks the GPU kept, the
attention over the entries the GPU selected -- the oracle still computes
both from the seeded inputs.

Inputs are drawn on the device with seeded generators (synth.latent_dev and
torch_gen), one sequence at a time; the oracle reads slices of those same
inputs, regenerated from their seeds where a full tensor would not fit on
the host.

  C1  1 query, N=4096, m=1, 16 heads, flat top-512, SWA 128, outlier channels
  C2  batch 32, 131072 tokens pooled at m=2 (gated) -> 65536 entries, t3 KV,
      64 heads, flat top-512
  C3  batch 8 at 1M entries, hierarchical (2048 blocks -> 16384 pool),
      top-512, 64 heads -- the benchmark's step
  C4  batch 64, 262144 entries, layer group full/reuse x3/reindex/reuse x3
  C5  cache write of 1M tokens at m=2, then a 4096-query prefill chunk at
      the end of the context (all 4096 rows run; 33 of them, every 128th and
      the last, are checked) with causal top-512 + SWA 128
  C4 with pool-restricted Reindex: the Full layer selects hierarchically and
      the Reindex layer scores only the Full layer's 16384-position pool
"""

import numpy as np
import pytest
import torch

from fp4_kv_cache_indexer_amd import csa2 as C
from fp4_kv_cache_indexer_amd import synth
from oracle import accounting as A
from oracle import csa2 as O
from oracle import formats as F
from parity import check_close, check_topk, dev, host, near_boundary, say

pytestmark = pytest.mark.gpu

D = 512


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    C.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class Cache:
    """Seeded token latents of S sequences (drawn per sequence on the
    device), their FP4 cache written by the HIP path, and host access to
    any tokens for the oracle."""

    def __init__(self, seed, cfg, S, T, m, dist="normal", outliers=False, gate=False):
        self.seed, self.cfg, self.S, self.T, self.m = seed, cfg, S, T, m
        self.dist, self.gate = dist, gate
        self.och = synth.outlier_channels_np(seed, cfg) if outliers else None
        self.N = T // m
        self.codes = torch.empty((S, self.N, D // 2), dtype=torch.uint8, device="cuda")
        self.scales = torch.empty((S, self.N, D // 16), dtype=torch.uint8, device="cuda")
        for s in range(S):
            x, z = self.tokens_dev(s)
            C.kv_compress_quantize(x[None], m, gate=None if z is None else z[None],
                                   codes=self.codes[s:s + 1], scales=self.scales[s:s + 1])
            del x, z
        release()

    def tokens_dev(self, s):
        x = synth.latent_dev((self.T, D), synth.torch_gen(self.seed, self.cfg, synth.T_LATENT, s),
                             self.dist, self.och).to(torch.bfloat16)
        z = None
        if self.gate:
            z = synth.latent_dev((self.T, D), synth.torch_gen(self.seed, self.cfg, synth.T_GATE, s)).to(torch.bfloat16)
        return x, z

    def entry_tokens(self, s, entries):
        """bf16 bits of the tokens of the given entries (m consecutive tokens
        each, in entry order), and of their gate logits."""
        x, z = self.tokens_dev(s)
        tok = (np.asarray(entries, dtype=np.int64)[:, None] * self.m + np.arange(self.m)[None, :]).ravel()
        t = torch.as_tensor(tok, device="cuda")
        xb = synth.bf16_host_bits(x[t])
        zb = None if z is None else synth.bf16_host_bits(z[t])
        del x, z
        return xb, zb

    def oracle_entries(self, s, entries):
        xb, zb = self.entry_tokens(s, entries)
        return O.kv_compress_quantize(xb, zb, self.m)

    def oracle_sparse(self, s, entries):
        """Oracle codes/scales of the whole sequence, filled only at
        `entries`, and whether the HIP cache holds the same bytes there.
        Without gates they must be equal; with gates a group may differ only
        on a quantiser decision boundary (then the two sides attend over
        slightly different keys and the row's attention is not compared)."""
        codes, scales, boundary = self.oracle_union(s, entries)
        return codes, scales, not boundary

    def oracle_union(self, s, entries):
        """As oracle_sparse for the union of several rows' selections: the
        oracle bytes at `entries` and the set of entries whose bytes differ
        on a decision boundary (empty without gates)."""
        entries = np.unique(np.asarray(entries, dtype=np.int64))
        entries = entries[entries >= 0]
        codes = np.zeros((self.N, D // 2), np.uint8)
        scales = np.zeros((self.N, D // 16), np.uint8)
        boundary = set()
        if len(entries):
            c, sc = self.oracle_entries(s, entries)
            codes[entries], scales[entries] = c, sc
            t = torch.as_tensor(entries, device="cuda")
            gc, gs = host(self.codes[s][t]), host(self.scales[s][t])
            bad = np.unique(np.concatenate([
                np.nonzero((gc != c).reshape(len(entries), 32, 8).any(axis=2).ravel())[0],
                np.nonzero((gs != sc).ravel())[0]]))
            if len(bad):
                assert self.gate, f"seq {s}: {len(bad)} selected groups differ (must be bit-exact)"
                xb, zb = self.entry_tokens(s, entries)
                y = O.pool(F.bf16_bits_to_f64(xb), F.bf16_bits_to_f64(zb), self.m)
                for gidx in bad:
                    e, gg = divmod(int(gidx), 32)
                    assert near_boundary(y[e, gg * 16:(gg + 1) * 16]), f"seq {s} entry {entries[e]} off-boundary"
                    boundary.add(int(entries[e]))
                say(f"  seq {s}: {len(bad)} selected groups on a decision boundary")
        return codes, scales, boundary

    def check_sampled(self, seqs, n_sample, rng):
        """Sampled cache entries against the oracle: bit-exact, except groups
        on a quantiser decision boundary when gates are pooled in float32."""
        mism = total = 0
        for s in seqs:
            ent = np.sort(rng.choice(self.N, size=min(n_sample, self.N), replace=False))
            rc, rs = self.oracle_entries(s, ent)
            gc = host(self.codes[s][torch.as_tensor(ent, device="cuda")])
            gs = host(self.scales[s][torch.as_tensor(ent, device="cuda")])
            bad = np.unique(np.concatenate([
                np.nonzero((gc != rc).reshape(len(ent), 32, 8).any(axis=2).ravel())[0],
                np.nonzero((gs != rs).ravel())[0]]))
            total += len(ent) * 32
            if not self.gate:
                assert len(bad) == 0, f"seq {s}: {len(bad)} groups differ (must be bit-exact)"
                continue
            xb, zb = self.entry_tokens(s, ent)
            y = O.pool(F.bf16_bits_to_f64(xb), F.bf16_bits_to_f64(zb), self.m)
            for gidx in bad:
                e, gg = divmod(int(gidx), 32)
                assert near_boundary(y[e, gg * 16:(gg + 1) * 16]), f"seq {s} entry {ent[e]} group {gg} off-boundary"
            mism += len(bad)
        say(f"  cache: {total} sampled groups, {mism} boundary mismatches")
        assert mism <= max(2, total * 1e-3)


def index_keys(seed, cfg, S, N):
    keys = torch.empty((S, N, 128), dtype=torch.uint8, device="cuda")
    for s in range(S):
        keys[s] = synth.to_e4m3(torch.randn((N, 128), generator=synth.torch_gen(seed, cfg, synth.T_KEYS, s),
                                            device="cuda"))
    return keys


def queries(seed, cfg, R, H, layer=0, swa_rows=None, dist="normal", och=None, cap=128):
    q_idx = synth.to_e4m3(torch.randn((R, 32, 128), generator=synth.torch_gen(seed, cfg, synth.T_QIDX, layer),
                                      device="cuda"))
    w = torch.rand((R, 32), generator=synth.torch_gen(seed, cfg, synth.T_WIDX, layer), device="cuda") * 0.75 + 0.25
    q = torch.randn((R, H, D), generator=synth.torch_gen(seed, cfg, synth.T_QATTN, layer),
                    device="cuda").to(torch.bfloat16)
    S = R if swa_rows is None else swa_rows
    swa = synth.to_e4m3(synth.latent_dev((S, cap, D), synth.torch_gen(seed, cfg, synth.T_SWA, layer), dist, och))
    return q_idx, w, q, swa


def check_rows(rows, gi, gsc_rows, q_idx_h, w_h, keys_of, n_valid_of, k, what):
    """Flat top-k of sampled rows against the oracle; returns the oracle ids."""
    refs = {}
    for r in rows:
        keys_h = keys_of(r)
        nv = n_valid_of(r)
        sc = O.index_scores(q_idx_h[r], w_h[r], keys_h[:nv])
        ref = O.topk_select(sc, np.arange(nv), k)
        check_topk(gi[r], ref, np.arange(nv), sc, k, f"{what} row {r}")
        sel = gi[r][gi[r] >= 0]
        if gsc_rows is not None and len(sel):
            err = np.abs(gsc_rows[r][:len(sel)] - sc[sel])
            assert np.all(err <= 2e-6 * np.abs(sc[sel]) + 1e-5), f"{what} row {r} scores"
        refs[r] = ref
    return refs


def judge_attention(cache, s, sel, q_bits, swa_h, slots, go, gl, what, boundary=None):
    """Attention of one row over the selection the GPU made, once check_topk
    has accepted it (equal to the oracle's, or differing only by swaps inside
    the tie band): the oracle quantises those entries itself and attends over
    them with the row's window.  Returns False, without comparing, when a
    selected group sits on a quantiser decision boundary (gated pooling)."""
    sel = np.asarray(sel, dtype=np.int64)
    if boundary is None:
        codes_o, scales_o, boundary = cache.oracle_union(s, sel)
    else:
        codes_o, scales_o = boundary[0], boundary[1]
        boundary = boundary[2]
    if boundary & set(sel[sel >= 0].tolist()):
        return False
    Ox, lx = O.sparse_attn(q_bits, codes_o, scales_o, sel, swa_h, slots)
    worst = check_close(go, Ox, f"{what} out")
    check_close(gl, lx, f"{what} lse")
    judge_attention.worst = max(getattr(judge_attention, "worst", 0.0), worst)
    return True


def test_c1_single_query_4096():
    say("C1: 1 query, N=4096, m=1, H=16, flat top-512, SWA 128, outliers x8")
    c = synth.make_decode_case(seed=0, cfg=0, S=1, N=4096, H=16, outliers=True)
    codes, scales = C.kv_compress_quantize(dev(c.x_bits), 1)
    rc, rs = O.kv_compress_quantize(c.x_bits[0], None, 1)
    torch.cuda.synchronize()
    assert np.array_equal(host(codes)[0], rc) and np.array_equal(host(scales)[0], rs)
    out_score = torch.empty((1, 512), dtype=torch.float32, device="cuda")
    idx = C.indexer_topk(dev(c.q_idx), dev(c.keys), 512, head_w=dev(c.w_idx), out_score=out_score)
    out, lse = C.sparse_attn_decode(dev(c.q), codes, scales, idx, swa=dev(c.swa), swa_len=dev(c.swa_len))
    torch.cuda.synchronize()
    gi = host(idx)
    refs = check_rows([0], gi, host(out_score), c.q_idx, c.w_idx, lambda r: c.keys[0], lambda r: 4096, 512, "C1")
    assert np.array_equal(gi[0], refs[0])
    Ox, lx = O.sparse_attn(c.q[0], rc, rs, refs[0], c.swa[0], O.swa_slots(0, 128, 128))
    check_close(host(out)[0], Ox, "C1 out")
    check_close(host(lse)[0], lx, "C1 lse")


def test_c2_batch32_m2_flat():
    say("C2: batch 32, 131072 tokens at m=2 (gated, t3) -> 65536 entries, H=64, flat top-512")
    seed, cfg, S, T, H, k = 0, 1, 32, 131072, 64, 512
    cache = Cache(seed, cfg, S, T, 2, dist="t3", gate=True)
    cache.check_sampled([0, 31], 512, np.random.default_rng(21))
    N = cache.N
    keys = index_keys(seed, cfg, S, N)
    q_idx, w, q, swa = queries(seed, cfg, S, H, dist="t3")
    swa_len = torch.full((S,), 128, dtype=torch.int32, device="cuda")
    out_score = torch.empty((S, k), dtype=torch.float32, device="cuda")
    say("  indexer + attention, 32 rows")
    idx = C.indexer_topk(q_idx, keys, k, head_w=w, out_score=out_score)
    out, lse = C.sparse_attn_decode(q, cache.codes, cache.scales, idx, swa=swa, swa_len=swa_len)
    torch.cuda.synchronize()
    gi, gsc, go, gl = host(idx), host(out_score), host(out), host(lse)
    rows = list(range(S))                                  # every row of the batch
    q_idx_h, w_h, q_h, swa_h = host(q_idx), host(w), synth.bf16_host_bits(q), host(swa)
    check_rows(rows, gi, gsc, q_idx_h, w_h, lambda r: host(keys[r]), lambda r: N, k, "C2")
    compared = 0
    judge_attention.worst = 0.0
    for r in rows:
        compared += judge_attention(cache, r, gi[r], q_h[r], swa_h[r], O.swa_slots(0, 128, 128), go[r], gl[r],
                                    f"C2 row {r}")
    say(f"  attention compared on {compared} of {len(rows)} rows (others hold a boundary group); "
        f"worst output error {judge_attention.worst:.3g} of the bound (64 heads: one fp16 P term)")
    assert compared >= len(rows) // 2


def test_c3_hierarchical_1m_bench_shape():
    say("C3: batch 8 at 1M entries, hierarchical keep 2048 -> pool 16384, top-512, H=64 (benchmark step)")
    seed, cfg, S, N, H, k, keep = 0, 2, 8, 1 << 20, 64, 512, 2048
    cache = Cache(seed, cfg, S, N, 1)
    cache.check_sampled([0, 7], 512, np.random.default_rng(23))
    keys = index_keys(seed, cfg, S, N)
    summ = C.index_block_summary(keys)
    q_idx, w, q, swa = queries(seed, cfg, S, H)
    swa_len = torch.full((S,), 128, dtype=torch.int32, device="cuda")
    blocks = torch.empty((S, keep), dtype=torch.int32, device="cuda")
    out_score = torch.empty((S, k), dtype=torch.float32, device="cuda")
    say("  hierarchical indexer + attention, 8 rows")
    idx = C.indexer_topk(q_idx, keys, k, head_w=w, block_keys=summ, keep_blocks=keep, out_blocks=blocks,
                         out_score=out_score)
    out, lse = C.sparse_attn_decode(q, cache.codes, cache.scales, idx, swa=swa, swa_len=swa_len)
    torch.cuda.synchronize()
    gi, gb, go, gl = host(idx), host(blocks), host(out), host(lse)
    q_idx_h, w_h, q_h, swa_h = host(q_idx), host(w), synth.bf16_host_bits(q), host(swa)
    compared = 0
    for r in range(S):                                     # every row of the batch
        keys_h = host(keys[r])
        bk = O.block_summary(keys_h)
        assert np.array_equal(host(summ[r]), bk), f"row {r} block summaries"
        _, ref_blocks = O.indexer_topk_hier(q_idx_h[r], w_h[r], keys_h, bk, k, N, keep)
        sb = O.index_scores(q_idx_h[r], w_h[r], bk)
        check_topk(gb[r], ref_blocks, np.arange(len(bk)), sb, keep, f"C3 row {r} blocks")
        # the fine stage is judged on the pool the GPU kept: a coarse swap
        # inside the tie band legitimately changes the pool
        pool = O.pool_positions(gb[r], N)
        sc = O.index_scores(q_idx_h[r], w_h[r], keys_h[pool])
        ref_idx = O.topk_select(sc, pool, k)
        check_topk(gi[r], ref_idx, pool, sc, k, f"C3 row {r} fine")
        assert judge_attention(cache, r, gi[r], q_h[r], swa_h[r], O.swa_slots(0, 128, 128), go[r], gl[r],
                               f"C3 row {r}")
        compared += 1
    assert compared == S


def test_c4_layer_group_batch64():
    say("C4: batch 64, 262144 entries, layers full/reuse x3/reindex/reuse x3, H=64")
    seed, cfg, S, N, H, k = 0, 3, 64, 262144, 64, 512
    modes = ["full", "reuse", "reuse", "reuse", "reindex", "reuse", "reuse", "reuse"]
    cache = Cache(seed, cfg, S, N, 1)
    cache.check_sampled([0, 63], 256, np.random.default_rng(24))
    keys = index_keys(seed, cfg, S, N)
    swa_len = torch.full((S,), 128, dtype=torch.int32, device="cuda")
    rows = tuple(range(0, S, 9)) + (S - 1,)                # 8 rows spread over the batch
    layers = []
    idx = None
    for L, mode in enumerate(modes):
        q_idx, w, q, swa = queries(seed, cfg, S, H, layer=L + 1)
        say(f"  layer {L} ({mode})")
        if mode in ("full", "reindex"):
            idx = C.indexer_topk(q_idx, keys, k, head_w=w)
        out, lse = C.sparse_attn_decode(q, cache.codes, cache.scales, idx, swa=swa, swa_len=swa_len)
        torch.cuda.synchronize()
        layers.append(dict(gi=host(idx)[list(rows)], go=host(out)[list(rows)], gl=host(lse)[list(rows)],
                           q_idx=host(q_idx)[list(rows)], w=host(w)[list(rows)],
                           q=synth.bf16_host_bits(q)[list(rows)], swa=host(swa)[list(rows)]))
        del q_idx, w, q, swa, out, lse
    compared = 0
    for j, r in enumerate(rows):
        keys_h = host(keys[r])
        own = {}
        for L in (0, 4):
            sc = O.index_scores(layers[L]["q_idx"][j], layers[L]["w"][j], keys_h)
            own[L] = O.topk_select(sc, np.arange(N), k)
            check_topk(layers[L]["gi"][j], own[L], np.arange(N), sc, k, f"C4 row {r} layer {L}")
        gsel = {L: layers[L]["gi"][j] for L in (0, 4)}
        codes_o, scales_o, same = cache.oracle_sparse(r, np.concatenate([own[0], own[4], gsel[0], gsel[4]]))
        assert same
        ref = O.layer_group(modes, [l["q"][j] for l in layers], [l["q_idx"][j] for l in layers],
                            [l["w"][j] for l in layers], codes_o, scales_o, keys_h,
                            [l["swa"][j] for l in layers], O.swa_slots(0, 128, 128), k)
        for L in range(len(modes)):
            ref_idx, Ox, lx = ref[L]
            src = 0 if L < 4 else 4
            assert np.array_equal(ref_idx, own[src])
            assert np.array_equal(layers[L]["gi"][j], gsel[src]), "reuse keeps the ids"
            if not np.array_equal(gsel[src], ref_idx):
                # a tie swap inside the band: the layer attends over the
                # GPU's (validated) selection
                Ox, lx = O.sparse_attn(layers[L]["q"][j], codes_o, scales_o, gsel[src], layers[L]["swa"][j],
                                       O.swa_slots(0, 128, 128))
            check_close(layers[L]["go"][j], Ox, f"C4 row {r} layer {L} out")
            check_close(layers[L]["gl"][j], lx, f"C4 row {r} layer {L} lse")
            compared += 1
    assert compared == len(rows) * len(modes)


def test_c5_cache_write_and_prefill_chunk():
    say("C5: cache write of 1M tokens at m=2 (gated), prefill chunk of 4096 queries")
    seed, cfg, T, m, H, k = 0, 4, 1 << 20, 2, 64, 512
    cache = Cache(seed, cfg, 1, T, m, gate=True)
    N = cache.N
    cache.check_sampled([0], 2048, np.random.default_rng(25))
    # bytes one cache entry occupies, as laid out by the library, equal the
    # oracle's accounting of an FP4 entry (codes + one E4M3 scale per 16 channels)
    assert cache.codes.shape[-1] + cache.scales.shape[-1] == A.fp4_entry_bytes(D)
    keys = index_keys(seed, cfg, 1, N)
    chunk = 4096
    pos = np.arange(T - chunk, T)                            # every row of the chunk
    R = len(pos)
    nv = (pos + 1) // m                                      # entries whose tokens all precede the query
    cap = chunk + 127                                        # window ring over the chunk's tokens
    base = T - cap
    x, _ = cache.tokens_dev(0)
    swa = synth.to_e4m3(x[base:].float())[None]              # the window holds the tokens in FP8
    del x
    lo = pos - 127
    swa_start = (lo - base).astype(np.int32)
    swa_len = np.full(R, 128, np.int32)
    q_idx, w, q, _ = queries(seed, cfg, R, H, swa_rows=1)
    row_seq = torch.zeros(R, dtype=torch.int32, device="cuda")
    say(f"  prefill rows R={R}: flat top-512 over causal prefixes of ~{N} entries + SWA")
    idx = C.indexer_topk(q_idx, keys, k, head_w=w, row_seq=row_seq, n_valid=dev(nv.astype(np.int32)))
    # every window is 128 tokens: swa_max keeps each row in one key split
    out, lse = C.sparse_attn_decode(q, cache.codes, cache.scales, idx, swa=swa, swa_start=dev(swa_start),
                                    swa_len=dev(swa_len), row_seq=row_seq, swa_max=128)
    torch.cuda.synchronize()
    gi, go, gl = host(idx), host(out), host(lse)
    q_idx_h, w_h, q_h, swa_h = host(q_idx), host(w), synth.bf16_host_bits(q), host(swa[0])
    keys_h = host(keys[0])
    rows = list(range(0, R, 128)) + [R - 1]                # 33 rows, every 128th and the last
    views = {r: O.prefill_row_view(int(pos[r]), m) for r in rows}
    check_rows(rows, gi, None, q_idx_h, w_h, lambda r: keys_h, lambda r: views[r][0], k, "C5")
    union = cache.oracle_union(0, np.concatenate([gi[r] for r in rows]))
    compared = 0
    for r in rows:
        assert views[r][0] == nv[r] and views[r][1] == lo[r] and views[r][2] == 128
        slots = range(int(lo[r] - base), int(lo[r] - base) + 128)
        compared += judge_attention(cache, 0, gi[r], q_h[r], swa_h, slots, go[r], gl[r], f"C5 row {r}",
                                    boundary=union)
    say(f"  attention compared on {compared} of {len(rows)} rows (others hold a boundary group)")
    assert compared >= len(rows) // 2


def test_c4_reindex_in_pool():
    say("C4 with pool-restricted Reindex: batch 64, 262144 entries, Full hierarchical (keep 2048), "
        "Reindex over the Full layer's pool")
    seed, cfg, S, N, H, k, keep = 0, 3, 64, 262144, 64, 512, 2048
    cache = Cache(seed, cfg, S, N, 1)
    keys = index_keys(seed, cfg, S, N)
    summ = C.index_block_summary(keys)
    swa_len = torch.full((S,), 128, dtype=torch.int32, device="cuda")
    blocks = torch.empty((S, keep), dtype=torch.int32, device="cuda")
    q1, w1, qa1, swa1 = queries(seed, cfg, S, H, layer=1)
    q5, w5, qa5, swa5 = queries(seed, cfg, S, H, layer=5)
    say("  Full layer (hierarchical) and pool-restricted Reindex layer")
    idx1 = C.indexer_topk(q1, keys, k, head_w=w1, block_keys=summ, keep_blocks=keep, out_blocks=blocks)
    idx5 = C.indexer_topk(q5, keys, k, head_w=w5, cand_blocks=blocks)
    out5, lse5 = C.sparse_attn_decode(qa5, cache.codes, cache.scales, idx5, swa=swa5, swa_len=swa_len)
    torch.cuda.synchronize()
    gb, gi5, go5, gl5 = host(blocks), host(idx5), host(out5), host(lse5)
    compared = 0
    for r in (0, 9, 18, 27, 36, 41, 54, 63):
        keys_h = host(keys[r])
        bk = O.block_summary(keys_h)
        qi = [host(q1[r]), None, None, None, host(q5[r])]
        wi = [host(w1[r]), None, None, None, host(w5[r])]
        _, kept = O.indexer_topk_hier(qi[0], wi[0], keys_h, bk, k, N, keep)
        sb = O.index_scores(qi[0], wi[0], bk)
        check_topk(gb[r], kept, np.arange(len(bk)), sb, keep, f"row {r} full-layer blocks")
        # the Reindex layer is judged on the pool the GPU's Full layer kept
        pool = O.pool_positions(gb[r], N)
        sc = O.index_scores(qi[4], wi[4], keys_h[pool])
        ref5 = O.indexer_topk_pool(qi[4], wi[4], keys_h, pool, k, N)
        check_topk(gi5[r], ref5, pool, sc, k, f"row {r} reindex in pool")
        codes_o, scales_o, same = cache.oracle_sparse(r, np.concatenate([ref5, gi5[r]]))
        assert same
        if np.array_equal(gb[r], kept):
            modes = ["full", "reuse", "reuse", "reuse", "reindex"]
            qa = [synth.bf16_host_bits(qa1[r])] * 4 + [synth.bf16_host_bits(qa5[r])]
            sw = [host(swa1[r])] * 4 + [host(swa5[r])]
            ref = O.layer_group(modes, qa, qi, wi, codes_o, scales_o, keys_h, sw, O.swa_slots(0, 128, 128), k,
                                block_keys=bk, keep_blocks=keep, reindex_in_pool=True)
            assert np.array_equal(ref[4][0], ref5)
        Ox, lx = O.sparse_attn(synth.bf16_host_bits(qa5[r]), codes_o, scales_o, gi5[r], host(swa5[r]),
                               O.swa_slots(0, 128, 128))
        check_close(go5[r], Ox, f"row {r} reindex out")
        check_close(gl5[r], lx, f"row {r} reindex lse")
        compared += 1
    assert compared == 8
