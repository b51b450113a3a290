"""Decode-time append (csa2_decode_append) against the oracle's bulk
definitions: appending a token stream one position at a time must leave the
caches that the bulk cache write, index-key rounding, block summaries and
window of the same stream give."""

import numpy as np
import pytest
import torch

from fp4_kv_cache_indexer_amd import csa2 as C
from fp4_kv_cache_indexer_amd import synth
from oracle import csa2 as O
from oracle import formats as F
from parity import dev, host, near_boundary, say

pytestmark = pytest.mark.gpu

SWA_CAP = 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    C.lib()
    yield
    torch.cuda.synchronize()


def token_stream(seed, S, T, gate):
    """bf16 tokens [S, T, 512] (with zero, huge and tiny tokens), gate logits
    and index keys [S, T, 128]."""
    g = np.random.default_rng(seed)
    x = (g.standard_normal((S, T, 512)) * np.exp(g.uniform(-2, 2, (S, T, 1)))).astype(np.float32)
    x[0, 0] = 0.0
    x[1, 1] = 3.0e38 * np.sign(x[1, 1])          # saturates E4M3 in the window
    x[2, 2] = 1e-30
    z = g.standard_normal((S, T, 512)).astype(np.float32) if gate else None
    k = (g.standard_normal((S, T, 128)) * np.exp(g.uniform(-3, 3, (S, T, 1)))).astype(np.float32)
    k[0, -1] = 0.0
    return (synth.to_bf16_bits(x), None if z is None else synth.to_bf16_bits(z), synth.to_bf16_bits(k))


class Caches:
    def __init__(self, S, N, m, fp4, gate):
        u8 = dict(dtype=torch.uint8, device="cuda")
        self.codes = torch.zeros((S, N, 256), **u8)
        self.scales = torch.zeros((S, N, 32), **u8)
        self.keys = torch.zeros((S, N, 64 if fp4 else 128), **u8)
        self.kscales = torch.zeros((S, N, 4), **u8) if fp4 else None
        self.summ = torch.zeros((S, (N + 7) // 8, 128), **u8)
        self.swa = torch.zeros((S, SWA_CAP, 512), **u8)
        bf = dict(dtype=torch.bfloat16, device="cuda")
        self.pend_x = torch.zeros((S, max(m - 1, 1), 512), **bf)
        self.pend_z = torch.zeros((S, max(m - 1, 1), 512), **bf) if gate else None
        self.m = m

    def append(self, x, z, k, pos, row_seq):
        C.decode_append(dev(x).view(torch.bfloat16), dev(pos.astype(np.int64)), self.codes, self.scales,
                        dev(k).view(torch.bfloat16), self.keys, m=self.m,
                        gate=None if z is None else dev(z).view(torch.bfloat16),
                        pend_x=self.pend_x if self.m > 1 else None,
                        pend_gate=self.pend_z if (self.m > 1 and z is not None) else None,
                        key_scales=self.kscales, block_keys=self.summ, swa=self.swa,
                        row_seq=dev(row_seq.astype(np.int32)))


def e4m3_of_bf16(bits):
    return F.e4m3_rne_sat(F.bf16_bits_to_f64(bits)).astype(np.uint8)


def check_against_bulk(c, x, z, k, T, m, fp4, gate, label):
    S, N = c.codes.shape[0], c.codes.shape[1]
    E = T // m
    gc, gs, gk = host(c.codes), host(c.scales), host(c.keys)
    gks = None if c.kscales is None else host(c.kscales)
    gsum, gswa = host(c.summ), host(c.swa)
    mism = 0
    for s in range(S):
        # main KV entries: the bulk write of the stream
        rc, rs = O.kv_compress_quantize(x[s, :E * m], None if z is None else z[s, :E * m], m)
        bad = np.unique(np.concatenate([
            np.nonzero((gc[s, :E] != rc).reshape(E, 32, 8).any(axis=2).ravel())[0],
            np.nonzero((gs[s, :E] != rs).ravel())[0]]))
        if m == 1 or not gate:
            assert len(bad) == 0, f"{label} seq {s}: {len(bad)} groups differ"
        else:
            y = O.pool(F.bf16_bits_to_f64(x[s, :E * m]), F.bf16_bits_to_f64(z[s, :E * m]), m)
            for gi in bad:
                e, gg = divmod(int(gi), 32)
                assert near_boundary(y[e, gg * 16:(gg + 1) * 16]), f"{label} seq {s} entry {e} off-boundary"
            mism += len(bad)
        assert not gc[s, E:].any() and not gs[s, E:].any(), f"{label}: entries past the stream written"
        # index keys: entry e takes the key of the token that completes it
        kin = k[s, m - 1::m][:E]
        if fp4:
            rk, rks = O.index_key_quantize_fp4(kin)
            assert np.array_equal(gk[s, :E], rk) and np.array_equal(gks[s, :E], rks), f"{label} seq {s} FP4 keys"
            ref_keys = O.Fp4Keys(rk, rks)
        else:
            rk = e4m3_of_bf16(kin)
            assert np.array_equal(gk[s, :E], rk), f"{label} seq {s} E4M3 keys"
            ref_keys = rk
        # block summaries over the entries written so far
        nb = (E + 7) // 8
        assert np.array_equal(gsum[s, :nb], O.block_summary(ref_keys)), f"{label} seq {s} summaries"
        assert not gsum[s, nb:].any()
        # window ring: slot p % cap holds the last token written there
        for slot in range(SWA_CAP):
            ps = [p for p in range(T) if p % SWA_CAP == slot]
            want = e4m3_of_bf16(x[s, ps[-1]]) if ps else np.zeros(512, np.uint8)
            assert np.array_equal(gswa[s, slot], want), f"{label} seq {s} window slot {slot}"
        # the open group's tokens wait in the pending buffer
        for j in range(T % m):
            got = c.pend_x[s, j].view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(got, x[s, E * m + j]), f"{label} seq {s} pending {j}"
    return mism


@pytest.mark.parametrize("m,gate,fp4", [(1, False, False), (1, False, True), (2, True, False),
                                        (2, True, True), (2, False, False), (4, True, True)])
def test_decode_append_equals_bulk_write(m, gate, fp4):
    S = 3
    E = 43                                    # 6 blocks, the last ragged
    T = E * m + (m - 1)                       # and an open group at the end
    N = E + 5
    say(f"decode_append m={m} gate={gate} fp4={fp4}: {T} tokens, {E} entries, ring {SWA_CAP}")
    x, z, k = token_stream(100 + 10 * m + gate + 2 * fp4, S, T, gate)
    c = Caches(S, N, m, fp4, gate)
    order = np.array([2, 0, 1])               # rows map to sequences out of order
    for p in range(T):
        c.append(x[order, p], None if z is None else z[order, p], k[order, p], np.full(S, p), order)
    torch.cuda.synchronize()
    mism = check_against_bulk(c, x, z, k, T, m, fp4, gate, f"m={m}")
    say(f"  boundary mismatches {mism}")
    assert mism <= 2


def test_decode_append_staggered_rows_and_skips():
    """One call mixes rows that open, continue and complete groups; rows with
    an unknown sequence, a negative position or an entry past the capacity
    write nothing."""
    m, S = 2, 4
    x, z, k = token_stream(7, S, 40, True)
    N = 12
    c = Caches(S, N, m, False, True)
    start = np.array([0, 1, 3, 2])            # sequence s has seen start[s] tokens before
    # bring every sequence to its own start, then advance all together
    for s in range(S):
        for p in range(start[s]):
            c.append(x[[s], p], z[[s], p], k[[s], p], np.array([p]), np.array([s]))
    for step in range(18):
        pos = start + step
        c.append(x[np.arange(S), pos], z[np.arange(S), pos], k[np.arange(S), pos], pos, np.arange(S))
    torch.cuda.synchronize()
    before = [t.clone() for t in (c.codes, c.scales, c.keys, c.summ, c.swa, c.pend_x)]
    # skipped rows: sequence -1, sequence 9, negative position, entry N (past the capacity)
    c.append(x[:4, 0], z[:4, 0], k[:4, 0], np.array([5, 5, -1, 2 * N + 1]), np.array([-1, 9, 0, 1]))
    torch.cuda.synchronize()
    for a, b in zip(before, (c.codes, c.scales, c.keys, c.summ, c.swa, c.pend_x)):
        assert torch.equal(a, b)
    # each sequence now holds its own stream of start[s] + 18 tokens
    for s in range(S):
        T = int(start[s]) + 18
        sub = Caches.__new__(Caches)
        sub.codes, sub.scales, sub.keys, sub.kscales = c.codes[s:s + 1], c.scales[s:s + 1], c.keys[s:s + 1], None
        sub.summ, sub.swa, sub.pend_x, sub.m = c.summ[s:s + 1], c.swa[s:s + 1], c.pend_x[s:s + 1], m
        assert check_against_bulk(sub, x[s:s + 1], z[s:s + 1], k[s:s + 1], T, m, False, True, f"seq {s}") <= 1


def test_window_append_many_rings():
    """Window-only rows (layers without a cache of their own) write slot
    pos % cap of their ring and nothing else."""
    L, S, cap, T = 5, 3, 8, 19
    x, _, _ = token_stream(9, L * S, T, False)
    ring = torch.zeros((L * S, cap, 512), dtype=torch.uint8, device="cuda")
    order = np.random.default_rng(3).permutation(L * S)
    for p in range(T):
        C.window_append(dev(x[order, p]).view(torch.bfloat16), dev(np.full(L * S, p, np.int64)), ring,
                        row_seq=dev(order.astype(np.int32)))
    torch.cuda.synchronize()
    got = host(ring)
    for r in range(L * S):
        for slot in range(cap):
            last = max(p for p in range(T) if p % cap == slot)
            assert np.array_equal(got[r, slot], e4m3_of_bf16(x[r, last])), (r, slot)


@pytest.mark.parametrize("m,gate,fp4", [(1, False, False), (1, False, True), (2, True, False), (2, True, True),
                                        (2, False, False)])
def test_append_indexer_fused_equals_sequential(m, gate, fp4):
    """csa2_append_indexer_topk over one decode step (the append runs inside
    the coarse scan's launch and the scan scores the refreshed block from a
    summary it computes itself) leaves the same caches and gives the same
    selection, bit for bit, as csa2_decode_append followed by
    csa2_indexer_topk, from the same cache state.  Row r is sequence r; the
    rows' tokens complete the last entry of a block, one inside a block, the
    first of a new block, none (an open group at m = 2, or position -1) or
    belong to no sequence (r >= n_seq).  A call with row_seq buffers (where
    a row may read a sequence another row appends to) takes the sequential
    form: its rows 1 and 4 share a sequence, row 4 appending nothing."""
    say(f"append + indexer fused vs sequential: m={m} gate={gate} fp4={fp4}")
    S, N, k, keep = 5, 2003, 96, 60
    R = 6
    g = np.random.default_rng(90 + m + 2 * fp4 + 4 * gate)
    gt = torch.Generator(device="cuda")
    gt.manual_seed(93 + m)
    base = Caches(S, N, m, fp4, gate)
    base.codes.copy_(torch.randint(0, 256, base.codes.shape, generator=gt, device="cuda", dtype=torch.uint8))
    base.scales.copy_(synth.to_e4m3(torch.randn(base.scales.shape, generator=gt, device="cuda")))
    kb = torch.randn((S, N, 128), generator=gt, device="cuda").to(torch.bfloat16)
    if fp4:
        C.index_key_quantize(kb, codes=base.keys, scales=base.kscales)
        C.index_block_summary_fp4(base.keys, base.kscales, summ=base.summ)
    else:
        base.keys.copy_(synth.to_e4m3(kb.float()))
        C.index_block_summary(base.keys, summ=base.summ)
    base.swa.copy_(torch.randint(0, 120, base.swa.shape, generator=gt, device="cuda", dtype=torch.uint8))
    base.pend_x.copy_(torch.randn(base.pend_x.shape, generator=gt, device="cuda").to(torch.bfloat16))
    if base.pend_z is not None:
        base.pend_z.copy_(torch.randn(base.pend_z.shape, generator=gt, device="cuda").to(torch.bfloat16))
    ent = np.array([N - 1, 8 * 100 + 3, 8 * 150, 8 * 40 + 5, 0, 17])
    pos = ent * m + (m - 1)
    if m > 1:
        pos[3] -= 1                                          # the first token of its group: nothing completes
    pos[4] = -1
    row_map = np.array([0, 1, 2, 3, 1, -1])                  # the row_seq form's mapping
    torch.cuda.synchronize()
    xt = synth.to_bf16_bits(g.standard_normal((R, 512)).astype(np.float32))
    zt = synth.to_bf16_bits(g.standard_normal((R, 512)).astype(np.float32)) if gate else None
    kt = synth.to_bf16_bits(g.standard_normal((R, 128)).astype(np.float32))
    q = dev(synth.to_e4m3(g.standard_normal((R, 32, 128)).astype(np.float32)))
    w = dev(g.uniform(0.25, 1.0, (R, 32)).astype(np.float32))
    nv = dev(np.array([N, 8 * 100 + 4, 8 * 150 + 1, N, N, N], np.int32))

    def clone(c):
        d = Caches(S, N, m, fp4, gate)
        for name in ("codes", "scales", "keys", "kscales", "summ", "swa", "pend_x", "pend_z"):
            if getattr(c, name) is not None:
                getattr(d, name).copy_(getattr(c, name))
        return d

    def run(form, row_seq):
        c = clone(base)
        rs = None if row_seq is None else dev(row_seq.astype(np.int32))
        args = dict(m=m, gate=None if zt is None else dev(zt).view(torch.bfloat16),
                    pend_x=c.pend_x if m > 1 else None, pend_gate=c.pend_z if (m > 1 and gate) else None,
                    key_scales=c.kscales, swa=c.swa)
        out_score = torch.zeros((R, k), dtype=torch.float32, device="cuda")
        blocks = torch.zeros((R, keep), dtype=torch.int32, device="cuda")
        xd, kd, pd = dev(xt).view(torch.bfloat16), dev(kt).view(torch.bfloat16), dev(pos.astype(np.int64))
        if form == "sequential":
            C.decode_append(xd, pd, c.codes, c.scales, kd, c.keys, row_seq=rs, block_keys=c.summ, **args)
            idx = C.indexer_topk(q, c.keys, k, head_w=w, row_seq=rs, n_valid=nv, block_keys=c.summ,
                                 keep_blocks=keep, out_score=out_score, out_blocks=blocks, key_scales=c.kscales)
        else:
            idx = C.append_indexer_topk(xd, pd, c.codes, c.scales, kd, q, c.keys, k, c.summ, row_seq=rs, head_w=w,
                                        n_valid=nv, keep_blocks=keep, out_score=out_score, out_blocks=blocks,
                                        **args)
        torch.cuda.synchronize()
        return (form, c, host(idx), host(out_score), host(blocks))

    pairs = [(run("sequential", None), run("fused", None)),
             (run("sequential", row_map), run("fused call with row_seq", row_map))]
    for (_, ref_c, ref_i, ref_s, ref_b), (form, c, gi, gs, gb) in pairs:
        for name in ("codes", "scales", "keys", "kscales", "summ", "swa", "pend_x", "pend_z"):
            if getattr(c, name) is not None:
                assert torch.equal(getattr(c, name), getattr(ref_c, name)), f"{form}: {name}"
        assert np.array_equal(gi, ref_i), f"{form}: ids"
        assert np.array_equal(gs.view(np.uint32), ref_s.view(np.uint32)), f"{form}: scores"
        assert np.array_equal(gb, ref_b), f"{form}: kept blocks"
        assert (ref_i[:4, 0] >= 0).all() and (ref_i[5] == -1).all()
        # the step changed the caches: the appended rows' summaries moved
        assert not torch.equal(ref_c.summ, base.summ)
