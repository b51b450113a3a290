"""GPU parity: every C-ABI entry point against the oracle on seeded inputs,
at sizes the oracle finishes in seconds, spanning several tiles/workgroups,
ragged tails and the degenerate cases of the method."""

import numpy as np
import pytest
import torch

from fp4_kv_cache_indexer_amd import csa2 as C
from fp4_kv_cache_indexer_amd import synth
from oracle import csa2 as O
from oracle import formats as F
from parity import check_close, check_topk, dev, host, near_boundary, say

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    C.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# cache write
# ---------------------------------------------------------------------------


def cache_case(seed, S, T, dist="normal", gate=False):
    g = synth.rng(seed, 7, synth.T_LATENT)
    x = synth.latent_np(g, (S, T, 512), dist, synth.outlier_channels_np(seed, 7))
    # edge rows: zeros, tiny, huge, mixed
    x[0, 0] = 0.0
    x[0, 1] = 1e-30
    x[0, 2] = 3.0e38 * np.sign(x[0, 2])
    x[0, 3, :16] = [1e-38] * 8 + [-2e-38] * 8
    xb = synth.to_bf16_bits(x)
    zb = synth.to_bf16_bits(synth.rng(seed, 7, synth.T_GATE).standard_normal((S, T, 512)).astype(np.float32)) if gate else None
    return xb, zb


@pytest.mark.parametrize("m,gate,S,T", [(1, False, 2, 1000), (2, False, 2, 1026), (2, True, 3, 2048),
                                        (4, True, 1, 1024), (4, False, 1, 1030)])
def test_kv_compress_quantize(m, gate, S, T):
    say(f"kv_compress_quantize m={m} gate={gate} S={S} T={T}")
    xb, zb = cache_case(11 + m, S, T, "t3" if gate else "normal", gate)
    codes, scales = C.kv_compress_quantize(dev(xb), m, gate=None if zb is None else dev(zb))
    torch.cuda.synchronize()
    gc, gs = host(codes), host(scales)
    E = T // m
    total = mism = 0
    for s in range(S):
        rc, rs = O.kv_compress_quantize(xb[s], None if zb is None else zb[s], m)
        assert rc.shape == gc[s].shape == (E, 256)
        bad_groups = np.unique(np.concatenate([
            np.nonzero((gc[s] != rc).reshape(E, 32, 8).any(axis=2).ravel())[0],
            np.nonzero((gs[s] != rs).ravel())[0]]))
        total += E * 32
        if m == 1 or (m == 2 and not gate):
            assert len(bad_groups) == 0, f"seq {s}: {len(bad_groups)} groups differ (must be bit-exact)"
            continue
        # pooled values are computed in float32 on the GPU: a group may only
        # differ where the oracle's value sits on a decision boundary
        x = F.bf16_bits_to_f64(xb[s])
        z = None if zb is None else F.bf16_bits_to_f64(zb[s])
        y = O.pool(x[:E * m], None if z is None else z[:E * m], m)
        for gidx in bad_groups:
            e, gg = divmod(int(gidx), 32)
            assert near_boundary(y[e, gg * 16:(gg + 1) * 16]), f"seq {s} entry {e} group {gg} differs off-boundary"
        mism += len(bad_groups)
    say(f"  groups {total}, boundary mismatches {mism}")
    assert mism <= max(2, total * 1e-3)


def test_kv_compress_quantize_append_in_place():
    say("kv_compress_quantize append with out_seq_stride")
    xb, _ = cache_case(5, 3, 64, "normal")
    full_c, full_s = C.kv_compress_quantize(dev(xb), 1)
    codes = torch.zeros((3, 100, 256), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((3, 100, 32), dtype=torch.uint8, device="cuda")
    # write tokens 10..13 of every sequence into entries 50..53 of a 100-entry cache
    xt = dev(xb)[:, 10:14].contiguous()
    C.kv_compress_quantize(xt, 1, codes=codes[:, 50:], scales=scales[:, 50:], out_seq_stride=100)
    torch.cuda.synchronize()
    assert torch.equal(codes[:, 50:54], full_c[:, 10:14]) and torch.equal(scales[:, 50:54], full_s[:, 10:14])
    assert int(codes[:, :50].sum()) == 0 and int(codes[:, 54:].sum()) == 0


@pytest.mark.parametrize("N", [4096, 4093, 8, 5])
def test_block_summary(N):
    say(f"index_block_summary N={N}")
    g = np.random.default_rng(N)
    keys = synth.to_e4m3(g.standard_normal((3, N, 128)).astype(np.float32) * 4)
    summ = C.index_block_summary(dev(keys))
    torch.cuda.synchronize()
    gsum = host(summ)
    for s in range(3):
        assert np.array_equal(gsum[s], O.block_summary(keys[s])), s
    # refresh one block after changing its last key
    keys2 = keys.copy()
    keys2[:, N - 1] = synth.to_e4m3(g.standard_normal((3, 128)).astype(np.float32))
    nb = (N + 7) // 8
    C.index_block_summary(dev(keys2), summ=summ, blk_begin=nb - 1, blk_end=nb)
    torch.cuda.synchronize()
    gsum = host(summ)
    for s in range(3):
        assert np.array_equal(gsum[s], O.block_summary(keys2[s])), s


# ---------------------------------------------------------------------------
# indexer
# ---------------------------------------------------------------------------


def run_indexer(case, top_k, **kw):
    q = dev(case["q"])
    keys = dev(case["keys"])
    args = dict(head_w=dev(case["w"]) if case.get("w") is not None else None)
    if case.get("row_seq") is not None:
        args["row_seq"] = dev(case["row_seq"].astype(np.int32))
    if case.get("n_valid") is not None:
        args["n_valid"] = dev(case["n_valid"].astype(np.int32))
    R = case["q"].shape[0]
    out_score = torch.empty((R, top_k), dtype=torch.float32, device="cuda")
    args.update(kw)
    idx = C.indexer_topk(q, keys, top_k, out_score=out_score, **args)
    torch.cuda.synchronize()
    return host(idx), host(out_score)


def idx_case(seed, S, N, R, w=True, row_seq=None, n_valid=None, dup=False):
    g = np.random.default_rng(seed)
    keys = synth.to_e4m3(g.standard_normal((S, N, 128)).astype(np.float32))
    if dup:   # exact ties: copies of a few keys spread over the cache
        for s in range(S):
            src = g.integers(0, N, 16)
            for j, t in enumerate(src):
                keys[s, g.integers(0, N, 40)] = keys[s, t]
    q = synth.to_e4m3(g.standard_normal((R, 32, 128)).astype(np.float32))
    ww = g.uniform(0.25, 1.0, (R, 32)).astype(np.float32) if w else None
    return dict(keys=keys, q=q, w=ww, row_seq=row_seq, n_valid=n_valid)


def check_flat_rows(case, gi, gsc, top_k):
    R = case["q"].shape[0]
    S, N = case["keys"].shape[:2]
    diffs = 0
    for r in range(R):
        s = r if case["row_seq"] is None else int(case["row_seq"][r])
        nv = N if case["n_valid"] is None else int(case["n_valid"][r])
        w = None if case["w"] is None else case["w"][r]
        sc = O.index_scores(case["q"][r], w, case["keys"][s][:nv])
        ref = O.topk_select(sc, np.arange(nv), top_k)
        diffs += check_topk(gi[r], ref, np.arange(nv), sc, top_k, f"row {r}")
        sel = gi[r][gi[r] >= 0]
        err = np.abs(gsc[r][:len(sel)] - sc[sel])
        if len(sel):
            say(f"  row {r}: score max abs err {err.max():.3e}, max rel {np.max(err / np.abs(sc[sel]).clip(1e-30)):.3e}")
        assert np.all(err <= 2e-6 * np.abs(sc[sel]) + 1e-5), f"row {r} scores"
    return diffs


def test_indexer_rows_in_passes():
    """A one-stage call whose score block would pass 512 MiB runs its rows in
    passes through one block: 600 rows over a 262,144-entry cache take two
    passes of 300 rows; bit-equal to two calls of 300 rows (one pass each)
    and to the oracle on sampled rows (ragged visible lengths, one empty row).
    With row_seq NULL, the second pass's rows keep their own sequences (past
    the one-sequence cache: nothing)."""
    say("indexer flat, 600 rows over one 262144-entry cache, in two passes")
    N, R, k = 262144, 600, 512
    g = np.random.default_rng(31)
    nv = g.integers(N // 2, N + 1, R)
    nv[:3] = [N, 1, 0]
    rs = np.zeros(R, np.int64)
    case = idx_case(41, 1, N, R, row_seq=rs, n_valid=nv)
    ws = C.indexer_topk_workspace(dev(case["q"]), dev(case["keys"]), k)
    assert ws < (R // 2 + 8) * N * 4 + (64 << 20), f"workspace {ws} not sized for one pass of {R // 2} rows"
    gi, gsc = run_indexer(case, k)
    parts = []
    for lo, hi in ((0, 300), (300, R)):
        parts.append(run_indexer(dict(case, q=case["q"][lo:hi], w=case["w"][lo:hi], row_seq=rs[lo:hi],
                                      n_valid=nv[lo:hi]), k))
    assert np.array_equal(gi, np.concatenate([parts[0][0], parts[1][0]]))
    assert np.array_equal(gsc.view(np.uint32), np.concatenate([parts[0][1], parts[1][1]]).view(np.uint32))
    assert (gi[2] == -1).all() and gi[1][0] == 0 and (gi[1][1:] == -1).all()
    sample = [0, 3, 299, 300, 599]
    sub = dict(case, q=case["q"][sample], w=case["w"][sample], row_seq=rs[sample], n_valid=nv[sample])
    check_flat_rows(sub, gi[sample], gsc[sample], k)
    gi2, _ = run_indexer(dict(case, row_seq=None, n_valid=None), k)
    one, _ = run_indexer(dict(case, q=case["q"][:1], w=case["w"][:1], row_seq=None, n_valid=None), k)
    assert np.array_equal(gi2[0], one[0])
    assert (gi2[1:] == -1).all()


def test_indexer_flat_single_query_4096():
    say("indexer flat N=4096 R=1 k=512")
    case = idx_case(1, 1, 4096, 1, w=False)
    gi, gsc = run_indexer(case, 512)
    check_flat_rows(case, gi, gsc, 512)


def test_indexer_flat_rows_ragged():
    say("indexer flat S=3 R=6 ragged n_valid")
    case = idx_case(2, 3, 5000, 6, row_seq=np.array([0, 1, 2, 0, 2, 1]),
                    n_valid=np.array([5000, 100, 0, 3001, 513, 512]))
    gi, gsc = run_indexer(case, 512)
    check_flat_rows(case, gi, gsc, 512)
    assert (gi[2] == -1).all() and (gi[1][100:] == -1).all()


def test_indexer_row_groups_one_cache():
    """Many rows over a one-sequence cache (a prefill chunk) take the
    row-group scan: bit-equal to the per-row scan of the same rows (issued
    in calls of fewer rows) and to the oracle on sampled rows; ragged and
    empty visible lengths, sequences outside the cache, an odd row count."""
    say("indexer flat, one cache, 301 rows (row groups) against the per-row scan and the oracle")
    N, R, k = 6007, 301, 96
    g = np.random.default_rng(11)
    nv = g.integers(0, N + 1, R)
    nv[:6] = [N, 0, 1, 15, 17, N - 1]
    rs = np.zeros(R, np.int64)
    rs[[7, 150, 299]] = [1, -1, 5]                       # outside the cache: nothing visible
    case = idx_case(21, 1, N, R, row_seq=rs, n_valid=nv)
    gi, gsc = run_indexer(case, k)                        # R >= 256 rows over one sequence
    parts = []
    for lo, hi in ((0, 150), (150, R)):                   # the same rows below the row-group threshold
        sub = dict(case, q=case["q"][lo:hi], w=case["w"][lo:hi], row_seq=rs[lo:hi], n_valid=nv[lo:hi])
        parts.append(run_indexer(sub, k))
    assert np.array_equal(gi, np.concatenate([parts[0][0], parts[1][0]]))
    assert np.array_equal(gsc.view(np.uint32), np.concatenate([parts[0][1], parts[1][1]]).view(np.uint32))
    for r in (7, 150, 299):
        assert (gi[r] == -1).all()
    sample = [0, 1, 2, 3, 4, 5, 100, 257, R - 1]
    sub = dict(case, q=case["q"][sample], w=case["w"][sample], row_seq=rs[sample], n_valid=nv[sample])
    check_flat_rows(sub, gi[sample], gsc[sample], k)


def test_indexer_flat_ties_and_topk_range():
    for k in (1, 7, 512, 2048):
        say(f"indexer flat ties k={k}")
        case = idx_case(3 + k, 2, 3000, 2, dup=True)
        gi, gsc = run_indexer(case, k)
        check_flat_rows(case, gi, gsc, k)


def test_indexer_hierarchical():
    say("indexer hierarchical S=2 N=20003 keep=300 k=512")
    case = idx_case(4, 2, 20003, 3, row_seq=np.array([0, 1, 1]), n_valid=np.array([20003, 20003, 9001]))
    bk = np.stack([O.block_summary(case["keys"][s]) for s in range(2)])
    blocks = torch.empty((3, 300), dtype=torch.int32, device="cuda")
    gi, gsc = run_indexer(case, 512, block_keys=dev(bk), keep_blocks=300, out_blocks=blocks)
    gb = host(blocks)
    for r in range(3):
        s = int(case["row_seq"][r])
        nv = int(case["n_valid"][r])
        q, w = case["q"][r], case["w"][r]
        nb = (nv + 7) // 8
        sb = O.index_scores(q, w, bk[s][:nb])
        ref_idx, ref_blocks = O.indexer_topk_hier(q, w, case["keys"][s], bk[s], 512, nv, 300)
        check_topk(gb[r], ref_blocks, np.arange(nb), sb, 300, f"row {r} blocks")
        # the fine stage on the pool the GPU kept (a near-tie at the coarse
        # boundary may change it legitimately)
        pool = O.pool_positions(gb[r], nv)
        sc = O.index_scores(q, w, case["keys"][s][pool])
        check_topk(gi[r], O.topk_select(sc, pool, 512), pool, sc, 512, f"row {r} fine")
        check_topk_valid(gi[r], gb[r], q, w, case["keys"][s], nv, 512, f"row {r} fine")
        if np.array_equal(gb[r], ref_blocks):
            assert np.array_equal(O.topk_select(sc, pool, 512), ref_idx)


def check_topk_valid(ids, kept_blocks, q, w, keys, nv, k, what):
    """Property check of a selection made from a pool of kept blocks: ids
    ascending, inside the pool, and no pool entry outside the selection
    scores above the lowest selected one by more than the tie band."""
    pool = set(O.pool_positions(kept_blocks, nv).tolist())
    ids = np.asarray(ids)
    sel = ids[ids >= 0]
    assert np.all(np.diff(sel) > 0) and set(sel.tolist()) <= pool, what
    assert len(sel) == min(k, len(pool)), what
    rest = np.array(sorted(pool - set(sel.tolist())), dtype=np.int64)
    if len(rest) and len(sel):
        lo = O.index_scores(q, w, keys[sel]).min()
        hi = O.index_scores(q, w, keys[rest]).max()
        assert hi <= lo + 1e-5 * abs(lo), what


def test_indexer_hierarchical_covering_pool_equals_flat():
    say("indexer hierarchical with a covering pool == flat")
    case = idx_case(5, 1, 4000, 2)
    bk = O.block_summary(case["keys"][0])[None]
    gi_h, _ = run_indexer(case, 256, block_keys=dev(bk), keep_blocks=500)
    gi_f, _ = run_indexer(case, 256)
    assert np.array_equal(gi_h, gi_f)


def test_indexer_candidates():
    say("indexer candidate lists")
    case = idx_case(6, 2, 3000, 2, n_valid=np.array([3000, 2000]))
    g = np.random.default_rng(0)
    cand = np.stack([g.permutation(3000)[:700] for _ in range(2)]).astype(np.int32)
    cand[:, ::37] = -1
    gi, gsc = run_indexer(case, 128, cand=dev(cand))
    for r in range(2):
        nv = int(case["n_valid"][r])
        ids = cand[r][(cand[r] >= 0) & (cand[r] < nv)]
        sc = O.index_scores(case["q"][r], case["w"][r], case["keys"][r][ids])
        check_topk(gi[r], O.topk_select(sc, ids, 128), ids, sc, 128, f"row {r}")


def test_indexer_flat_long_rows():
    """Rows longer than one workgroup streams (2^18 items) with few rows take
    the multi-workgroup filter + select path."""
    say("indexer flat N=300000 R=2 k=2048 (filter + select path)")
    case = idx_case(12, 1, 300000, 2, row_seq=np.array([0, 0]), n_valid=np.array([300000, 262145]))
    gi, gsc = run_indexer(case, 2048)
    check_flat_rows(case, gi, gsc, 2048)


def test_indexer_flat_long_rows_mixed_lengths():
    """The filter + select path with rows of very different lengths in one
    call: the select maps its candidate slots by the launch's chunk count
    (74 here), so a 10-chunk row leaves most threads idle, and a row that
    sees nothing writes -1."""
    say("indexer flat N=300000 R=3 k=2048, n_valid 300000 / 40000 / 0")
    case = idx_case(13, 1, 300000, 3, row_seq=np.array([0, 0, 0]), n_valid=np.array([300000, 40000, 0]))
    gi, gsc = run_indexer(case, 2048)
    check_flat_rows(case, gi, gsc, 2048)


def test_indexer_block_pool():
    """Block-pool mode: select among the positions of given blocks (ascending
    lists with -1 holes and blocks past n_valid), ragged rows."""
    say("indexer block pool: S=2 N=20003 R=3, 300-block lists")
    case = idx_case(31, 2, 20003, 3, row_seq=np.array([0, 1, 1]), n_valid=np.array([20003, 9001, 20003]))
    g = np.random.default_rng(8)
    nb = (20003 + 7) // 8
    blocks = np.stack([np.sort(g.choice(nb, 300, replace=False)) for _ in range(3)]).astype(np.int32)
    blocks[:, ::29] = -1
    gi, gsc = run_indexer(case, 512, cand_blocks=dev(blocks))
    for r in range(3):
        s = int(case["row_seq"][r])
        nv = int(case["n_valid"][r])
        pool = O.pool_positions(blocks[r], nv)
        sc = O.index_scores(case["q"][r], case["w"][r], case["keys"][s][pool])
        ref = O.indexer_topk_pool(case["q"][r], case["w"][r], case["keys"][s], pool, 512, nv)
        check_topk(gi[r], ref, pool, sc, 512, f"row {r}")


@pytest.mark.parametrize("fp4", [False, True])
def test_indexer_rows_outside_the_cache_all_modes(fp4):
    """Rows whose sequence is outside [0, n_seq) see no entry in every mode:
    candidate, block pool and hierarchical calls give all -1 for them (and
    read no key), while a valid row of the same call is selected normally."""
    say(f"indexer rows with row_seq -1 and n_seq, {'FP4' if fp4 else 'E4M3'} keys, every mode")
    S, N, k = 2, 5003, 64
    rs = np.array([-1, 0, S, 1], np.int64)
    case = idx_case(46, S, N, 4, row_seq=rs)
    kw = {}
    keys_o = [case["keys"][s] for s in range(S)]
    if fp4:
        _, codes, kscales = fp4_key_case(47, S, N)
        case["keys"] = codes
        kw["key_scales"] = dev(kscales)
        keys_o = [O.Fp4Keys(codes[s], kscales[s]) for s in range(S)]
    nb = (N + 7) // 8
    g = np.random.default_rng(48)
    cand = np.stack([g.permutation(N)[:900] for _ in range(4)]).astype(np.int32)
    cblk = np.stack([np.sort(g.choice(nb, 120, replace=False)) for _ in range(4)]).astype(np.int32)
    bk = np.stack([O.block_summary(keys_o[s]) for s in range(S)])
    blocks = torch.full((4, 100), 7, dtype=torch.int32, device="cuda")
    runs = {
        "candidate": dict(cand=dev(cand)),
        "block pool": dict(cand_blocks=dev(cblk)),
        "hierarchical": dict(block_keys=dev(bk), keep_blocks=100, out_blocks=blocks),
    }
    for mode, extra in runs.items():
        gi, gsc = run_indexer(case, k, **kw, **extra)
        for r in (0, 2):
            assert (gi[r] == -1).all() and (gsc[r] == 0).all(), f"{mode}: row {r} (row_seq {rs[r]})"
        q, w = case["q"][1], case["w"][1]
        if mode == "candidate":
            ids = cand[1]
        elif mode == "block pool":
            ids = O.pool_positions(cblk[1], N)
        else:
            gb = host(blocks)
            assert (gb[0] == -1).all() and (gb[2] == -1).all(), "hierarchical: kept blocks of invalid rows"
            ids = O.pool_positions(gb[1], N)
        sc = O.index_scores(q, w, keys_o[0][ids])
        check_topk(gi[1], O.topk_select(sc, ids, k), ids, sc, k, f"{mode}: row 1")


def test_indexer_wide_tie_bins():
    """Boundary bins far larger than the workgroup's staging buffer: every
    key equal (one bin holds the whole row) and three distinct keys (three
    bins of ~7000 entries); ties go to the lower entry id."""
    say("indexer flat, boundary bin of 20000 / ~7000 equal scores")
    g = np.random.default_rng(11)
    S, N = 2, 20000
    base = synth.to_e4m3(g.standard_normal((3, 128)).astype(np.float32))
    keys = np.empty((S, N, 128), np.uint8)
    keys[0] = base[0]
    keys[1] = base[g.integers(0, 3, N)]
    q = synth.to_e4m3(g.standard_normal((2, 32, 128)).astype(np.float32))
    case = dict(keys=keys, q=q, w=None, row_seq=None, n_valid=None)
    for k in (512, 2048):
        gi, gsc = run_indexer(case, k)
        check_flat_rows(case, gi, gsc, k)
    assert np.array_equal(gi[0], np.arange(2048))


def test_indexer_workspace_reuse():
    """One zeroed workspace serves many calls of the same shape and mode:
    the top-k kernel leaves its histograms and counters cleared, so a call
    repeated after calls on other data gives the same, correct result."""
    say("indexer workspace reuse: flat, hierarchical, candidates")
    caseA = idx_case(21, 2, 9000, 3, row_seq=np.array([0, 1, 1]), n_valid=np.array([9000, 4097, 0]))
    caseB = idx_case(22, 2, 9000, 3, row_seq=np.array([1, 0, 0]), n_valid=np.array([8000, 9000, 300]))
    cand = np.stack([np.random.default_rng(r).permutation(9000)[:5000] for r in range(3)]).astype(np.int32)
    bk = {id(c): np.stack([O.block_summary(c["keys"][s]) for s in range(2)]) for c in (caseA, caseB)}
    modes = {
        "flat": lambda c: {},
        "hier": lambda c: dict(block_keys=dev(bk[id(c)]), keep_blocks=200),
        "cand": lambda c: dict(cand=dev(cand)),
    }
    for name, extra in modes.items():
        ws = torch.zeros(C.indexer_topk_workspace(dev(caseA["q"]), dev(caseA["keys"]), 256, **{
            k: v for k, v in extra(caseA).items() if k in ("block_keys", "keep_blocks", "cand")}),
            dtype=torch.uint8, device="cuda")
        first = run_indexer(caseA, 256, workspace=ws, **extra(caseA))
        for _ in range(2):
            other = run_indexer(caseB, 256, workspace=ws, **extra(caseB))
        again = run_indexer(caseA, 256, workspace=ws, **extra(caseA))
        fresh = run_indexer(caseA, 256, **extra(caseA))
        fresh_b = run_indexer(caseB, 256, **extra(caseB))
        for got, ref in ((again, first), (first, fresh), (other, fresh_b)):
            assert np.array_equal(got[0], ref[0]), name
            assert np.array_equal(got[1][got[0] >= 0], ref[1][ref[0] >= 0]), name
        if name == "flat":
            check_flat_rows(caseA, *first, 256)
            check_flat_rows(caseB, *other, 256)


# ---------------------------------------------------------------------------
# FP4 index keys (128 E2M1 + one E4M3 scale per 32 channels)
# ---------------------------------------------------------------------------


def fp4_key_case(seed, S, N):
    """bf16 index keys with edge groups (zero, tiny, huge, mixed), their
    oracle FP4 encoding (the input both sides score from)."""
    g = np.random.default_rng(seed)
    k = (g.standard_normal((S, N, 128)) * np.exp(g.uniform(-2, 2, (S, N, 1)))).astype(np.float32)
    k[0, 0] = 0.0
    k[0, 1, :32] = 1e-30
    k[0, 2, 32:64] = 3.0e38
    k[0, 3, 96:] = [1e-38] * 16 + [-2e-38] * 16
    kb = synth.to_bf16_bits(k)
    enc = [O.index_key_quantize_fp4(kb[s]) for s in range(S)]
    codes = np.stack([e[0] for e in enc])
    scales = np.stack([e[1] for e in enc])
    return kb, codes, scales


def test_index_key_quantize():
    say("index_key_quantize: S=2 N=5003 bf16 keys -> FP4 (bit-exact)")
    kb, codes, scales = fp4_key_case(41, 2, 5003)
    gc, gs = C.index_key_quantize(dev(kb))
    torch.cuda.synchronize()
    assert np.array_equal(host(gc), codes) and np.array_equal(host(gs), scales)


def test_block_summary_word_aligned_buffers():
    # keys and summaries only 4-byte aligned take the 4-channel kernel; both
    # kernels must give the oracle's summaries
    say("index_block_summary on 4-byte aligned buffers, N=1003")
    N = 1003
    g = np.random.default_rng(7)
    keys = synth.to_e4m3(g.standard_normal((2, N, 128)).astype(np.float32) * 4)
    nb = (N + 7) // 8
    kbuf = torch.zeros(2 * N * 128 + 16, dtype=torch.uint8, device="cuda")
    kv = kbuf[4:4 + 2 * N * 128].view(2, N, 128)
    kv.copy_(dev(keys))
    sbuf = torch.zeros(2 * nb * 128 + 16, dtype=torch.uint8, device="cuda")
    sv = sbuf[4:4 + 2 * nb * 128].view(2, nb, 128)
    assert kv.data_ptr() % 16 == 4 and sv.data_ptr() % 16 == 4
    C.index_block_summary(kv, summ=sv)
    torch.cuda.synchronize()
    gsum = host(sv)
    for s in range(2):
        assert np.array_equal(gsum[s], O.block_summary(keys[s])), s


@pytest.mark.parametrize("N", [4096, 4093, 8, 5])
def test_block_summary_fp4(N):
    say(f"block_summary_fp4 N={N}")
    _, codes, scales = fp4_key_case(42 + N, 3, N)
    summ = C.index_block_summary_fp4(dev(codes), dev(scales))
    torch.cuda.synchronize()
    gs = host(summ)
    for s in range(3):
        assert np.array_equal(gs[s], O.block_summary_fp4(codes[s], scales[s])), s


def test_block_summary_fp4_word_aligned_buffers():
    # FP4 codes and summaries only 4-byte aligned take the 4-channel kernel
    say("block_summary_fp4 on 4-byte aligned buffers, N=1003")
    N = 1003
    _, codes, scales = fp4_key_case(77, 2, N)
    nb = (N + 7) // 8
    cbuf = torch.zeros(2 * N * 64 + 16, dtype=torch.uint8, device="cuda")
    cv = cbuf[4:4 + 2 * N * 64].view(2, N, 64)
    cv.copy_(dev(codes))
    sbuf = torch.zeros(2 * nb * 128 + 16, dtype=torch.uint8, device="cuda")
    sv = sbuf[4:4 + 2 * nb * 128].view(2, nb, 128)
    assert cv.data_ptr() % 8 == 4 and sv.data_ptr() % 16 == 4
    C.index_block_summary_fp4(cv, dev(scales), summ=sv)
    torch.cuda.synchronize()
    gs = host(sv)
    for s in range(2):
        assert np.array_equal(gs[s], O.block_summary_fp4(codes[s], scales[s])), s


def fp4_idx_case(seed, S, N, R, **kw):
    case = idx_case(seed, S, N, R, **kw)
    _, codes, scales = fp4_key_case(seed + 100, S, N)
    case["codes"], case["kscales"] = codes, scales
    case["keys"] = None
    return case


def check_fp4_rows(case, gi, gsc, k, pool_of=None):
    R = case["q"].shape[0]
    for r in range(R):
        s = r if case["row_seq"] is None else int(case["row_seq"][r])
        N = case["codes"].shape[1]
        nv = N if case["n_valid"] is None else int(case["n_valid"][r])
        keys = O.Fp4Keys(case["codes"][s], case["kscales"][s])
        ids = np.arange(nv) if pool_of is None else pool_of(r, nv)
        sc = O.index_scores(case["q"][r], case["w"][r], keys[ids])
        ref = O.topk_select(sc, ids, k)
        check_topk(gi[r], ref, ids, sc, k, f"row {r}")
        sel = gi[r][gi[r] >= 0]
        if len(sel):
            sfull = dict(zip(ids.tolist(), sc.tolist()))
            want = np.array([sfull[int(x)] for x in sel])
            err = np.abs(gsc[r][:len(sel)] - want)
            assert np.all(err <= 2e-6 * np.abs(want) + 1e-5), f"row {r} scores"


def run_fp4_indexer(case, k, **kw):
    R = case["q"].shape[0]
    out_score = torch.empty((R, k), dtype=torch.float32, device="cuda")
    args = dict(head_w=dev(case["w"]), key_scales=dev(case["kscales"]), out_score=out_score)
    if case.get("row_seq") is not None:
        args["row_seq"] = dev(case["row_seq"].astype(np.int32))
    if case.get("n_valid") is not None:
        args["n_valid"] = dev(case["n_valid"].astype(np.int32))
    args.update(kw)
    idx = C.indexer_topk(dev(case["q"]), dev(case["codes"]), k, **args)
    torch.cuda.synchronize()
    return host(idx), host(out_score)


def test_indexer_fp4_keys_flat():
    say("indexer with FP4 keys, flat: S=3 R=5 ragged, k=512")
    case = fp4_idx_case(43, 3, 7000, 5, row_seq=np.array([0, 1, 2, 0, 2]),
                        n_valid=np.array([7000, 300, 6999, 4097, 0]))
    gi, gsc = run_fp4_indexer(case, 512)
    check_fp4_rows(case, gi, gsc, 512)


def test_indexer_fp4_keys_hierarchical_and_block_pool():
    say("indexer with FP4 keys: hierarchical (summaries from FP4 keys) and block pool")
    case = fp4_idx_case(44, 2, 20003, 3, row_seq=np.array([0, 1, 1]), n_valid=np.array([20003, 20003, 9001]))
    summ = C.index_block_summary_fp4(dev(case["codes"]), dev(case["kscales"]))
    blocks = torch.empty((3, 300), dtype=torch.int32, device="cuda")
    gi, gsc = run_fp4_indexer(case, 512, block_keys=summ, keep_blocks=300, out_blocks=blocks)
    gb = host(blocks)
    for r in range(3):
        s, nv = int(case["row_seq"][r]), int(case["n_valid"][r])
        keys = O.Fp4Keys(case["codes"][s], case["kscales"][s])
        bk = O.block_summary(keys)
        ref_idx, ref_blocks = O.indexer_topk_hier(case["q"][r], case["w"][r], keys, bk, 512, nv, 300)
        nb = (nv + 7) // 8
        sb = O.index_scores(case["q"][r], case["w"][r], bk[:nb])
        check_topk(gb[r], ref_blocks, np.arange(nb), sb, 300, f"row {r} blocks")
        # the fine stage on the pool the GPU kept (equal to the oracle's
        # unless a coarse swap inside the tie band changed it)
        pool = O.pool_positions(gb[r], nv)
        sc = O.index_scores(case["q"][r], case["w"][r], keys[pool])
        check_topk(gi[r], O.topk_select(sc, pool, 512), pool, sc, 512, f"row {r} fine")
        if np.array_equal(gb[r], ref_blocks):
            assert np.array_equal(O.topk_select(sc, pool, 512), ref_idx)
    # the Full layer's pool, rescored by a new query over FP4 keys
    case2 = dict(case, q=idx_case(45, 2, 8, 3)["q"])
    gi2, gsc2 = run_fp4_indexer(case2, 256, cand_blocks=blocks)
    check_fp4_rows(case2, gi2, gsc2, 256, pool_of=lambda r, nv: O.pool_positions(gb[r], nv))


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------


def attn_case(seed, S, N, R, H, k, cap=128, dist="normal"):
    c = synth.make_decode_case(seed=seed, cfg=50, S=S, N=N, H=H, R=R, swa_cap=cap, swa_len=cap,
                               dist=dist, outliers=True)
    codes = np.empty((S, N, 256), np.uint8)
    scales = np.empty((S, N, 32), np.uint8)
    for s in range(S):
        codes[s], scales[s] = O.kv_compress_quantize(c.x_bits[s], None, 1)
    g = np.random.default_rng(seed)
    idx = np.stack([np.sort(g.choice(N, size=k, replace=False)) for _ in range(R)]).astype(np.int32)
    return c, codes, scales, idx


def run_attn(c, codes, scales, idx, swa_start, swa_len, sm_scale=0.0, row_seq=None, swa_max=0):
    if row_seq is None:
        row_seq = np.arange(c.q.shape[0]) % c.S
    out, lse = C.sparse_attn_decode(
        dev(c.q), dev(codes), dev(scales), dev(idx), swa=dev(c.swa),
        swa_start=dev(np.asarray(swa_start, np.int32)), swa_len=dev(np.asarray(swa_len, np.int32)),
        row_seq=None if row_seq is None else dev(np.asarray(row_seq, np.int32)), sm_scale=sm_scale,
        swa_max=swa_max)
    torch.cuda.synchronize()
    return host(out), host(lse)


def check_attn_rows(c, codes, scales, idx, swa_start, swa_len, out, lse, sm_scale=None, row_seq=None):
    worst = 0.0
    for r in range(c.q.shape[0]):
        s = r % c.S if row_seq is None else int(row_seq[r])
        slots = O.swa_slots(swa_start[r], swa_len[r], c.swa.shape[1])
        Ox, lx = O.sparse_attn(c.q[r], codes[s], scales[s], idx[r], c.swa[s], slots, sm_scale)
        worst = max(worst, check_close(out[r], Ox, f"row {r} out"), check_close(lse[r], lx, f"row {r} lse"))
    return worst


def test_attn_single_query_h16():
    say("sparse_attn H=16 N=4096 k=512 swa=128")
    c, codes, scales, idx = attn_case(1, 1, 4096, 1, 16, 512)
    out, lse = run_attn(c, codes, scales, idx, [0], [128])
    say(f"  worst/bound {check_attn_rows(c, codes, scales, idx, [0], [128], out, lse):.3f}")


@pytest.mark.parametrize("H", [16, 64])
def test_attn_window_bound_decode_rows(H):
    # few rows (the narrow kernel at H=16 and 64): windows longer than
    # swa_max are clamped to their first swa_max slots, wrapping the ring
    say(f"sparse_attn H={H}, 2 rows, swa_max=48 below the window lengths")
    c, codes, scales, idx = attn_case(6, 2, 2500, 2, H, 256)
    start, ln = [100, 120], [128, 90]
    out, lse = run_attn(c, codes, scales, idx, start, ln, swa_max=48)
    check_attn_rows(c, codes, scales, idx, start, [48, 48], out, lse)


@pytest.mark.parametrize("H", [32, 64, 128])
def test_attn_rows_masks_and_wrap(H):
    say(f"sparse_attn H={H} rows with -1 ids, short/wrapped windows")
    c, codes, scales, idx = attn_case(2, 2, 3000, 4, H, 512, dist="t3")
    idx[1, 100:300] = -1
    idx[2, :] = -1
    idx[3, 5] = 2999
    start, ln = [0, 100, 5, 127], [128, 37, 0, 128]
    out, lse = run_attn(c, codes, scales, idx, start, ln)
    check_attn_rows(c, codes, scales, idx, start, ln, out, lse)
    assert np.all(lse[2] == -np.inf) and np.all(out[2] == 0)


def test_attn_custom_scale_and_row_mapping():
    say("sparse_attn sm_scale=0.1 row_seq")
    c, codes, scales, idx = attn_case(3, 2, 2048, 3, 64, 300)
    rs = [1, 0, 1]
    out, lse = run_attn(c, codes, scales, idx, [0, 0, 64], [128, 128, 64], sm_scale=0.1, row_seq=rs)
    check_attn_rows(c, codes, scales, idx, [0, 0, 64], [128, 128, 64], out, lse, sm_scale=0.1, row_seq=rs)


def test_attn_sparse_covering_all_equals_dense():
    say("sparse_attn with k >= N: dense attention")
    c, codes, scales, _ = attn_case(4, 1, 700, 1, 64, 10)
    idx = np.arange(700, dtype=np.int32)[None]
    idx = np.concatenate([idx, -np.ones((1, 4), np.int32)], axis=1)
    out, lse = run_attn(c, codes, scales, idx, [0], [128])
    check_attn_rows(c, codes, scales, idx, [0], [128], out, lse)


def test_attn_no_keys():
    say("sparse_attn without keys")
    c, codes, scales, idx = attn_case(5, 1, 64, 2, 64, 16)
    idx[:] = -1
    out, lse = run_attn(c, codes, scales, idx, [0, 0], [0, 0])
    assert np.all(out == 0) and np.all(lse == -np.inf)


def test_empty_inputs():
    """Zero rows through every entry point and zero tokens through the cache
    write: each call succeeds, launches nothing and returns empty outputs
    (the host returns before validating pointers, which empty tensors leave
    NULL)."""
    say("zero rows: indexer flat/hierarchical/static, attention, append; zero tokens: cache write")
    N = 4096
    keys = torch.zeros((1, N, 128), dtype=torch.uint8, device="cuda")
    bkeys = torch.zeros((1, N // 8, 128), dtype=torch.uint8, device="cuda")
    q0 = torch.zeros((0, 32, 128), dtype=torch.uint8, device="cuda")
    assert tuple(C.indexer_topk(q0, keys, 512).shape) == (0, 512)
    assert tuple(C.indexer_topk(q0, keys, 512, block_keys=bkeys, keep_blocks=64).shape) == (0, 512)
    assert tuple(C.indexer_topk_static(q0, keys, 512).shape) == (0, 512)
    codes = torch.zeros((1, N, 256), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((1, N, 32), dtype=torch.uint8, device="cuda")
    qa = torch.zeros((0, 64, 512), dtype=torch.bfloat16, device="cuda")
    out, lse = C.sparse_attn_decode(qa, codes, scales, torch.zeros((0, 512), dtype=torch.int32, device="cuda"))
    assert tuple(out.shape) == (0, 64, 512) and tuple(lse.shape) == (0, 64)
    C.decode_append(torch.zeros((0, 512), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((0,), dtype=torch.int64, device="cuda"), codes, scales,
                    torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda"), keys)
    x0 = torch.zeros((1, 0, 512), dtype=torch.bfloat16, device="cuda")
    c0, s0 = C.kv_compress_quantize(x0, 2)
    assert tuple(c0.shape) == (1, 0, 256) and tuple(s0.shape) == (1, 0, 32)
    torch.cuda.synchronize()
    assert torch.all(codes == 0) and torch.all(keys == 0)   # nothing was written


# ---------------------------------------------------------------------------
# layer groups and prefill rows
# ---------------------------------------------------------------------------


def test_layer_group_full_reuse_reindex():
    say("layer group full/reuse x3/reindex/reuse x3, B=3 N=6000 H=64")
    modes = ["full", "reuse", "reuse", "reuse", "reindex", "reuse", "reuse", "reuse"]
    S, N, H, k = 3, 6000, 64, 512
    base = synth.make_decode_case(seed=9, cfg=4, S=S, N=N, H=H)
    codes = np.empty((S, N, 256), np.uint8)
    scales = np.empty((S, N, 32), np.uint8)
    for s in range(S):
        codes[s], scales[s] = O.kv_compress_quantize(base.x_bits[s], None, 1)
    layers = [synth.make_decode_case(seed=9, cfg=4, S=S, N=8, H=H, layer=L + 1) for L in range(len(modes))]
    d_codes, d_scales, d_keys = dev(codes), dev(scales), dev(base.keys)
    idx = None
    for L, mode in enumerate(modes):
        if mode in ("full", "reindex"):
            idx = C.indexer_topk(dev(layers[L].q_idx), d_keys, k, head_w=dev(layers[L].w_idx))
        out, lse = C.sparse_attn_decode(dev(layers[L].q), d_codes, d_scales, idx, swa=dev(layers[L].swa),
                                        swa_len=dev(np.full(S, 128, np.int32)))
        torch.cuda.synchronize()
        gi, go, gl = host(idx), host(out), host(lse)
        for r in range(S):
            ref = O.layer_group(modes[:L + 1], [l.q[r] for l in layers], [l.q_idx[r] for l in layers],
                                [l.w_idx[r] for l in layers], codes[r], scales[r], base.keys[r],
                                [l.swa[r] for l in layers], O.swa_slots(0, 128, 128), k)[-1]
            sc = O.index_scores(layers[L if mode != "reuse" else (0 if L < 4 else 4)].q_idx[r],
                                None, base.keys[r])
            check_topk(gi[r], ref[0], np.arange(N), sc, k, f"layer {L} row {r}")
            if np.array_equal(gi[r], ref[0]):
                check_close(go[r], ref[1], f"layer {L} row {r} out")
                check_close(gl[r], ref[2], f"layer {L} row {r} lse")


def test_prefill_rows_causal():
    say("prefill rows: T=1024 tokens at m=2, 48 rows, causal n_valid, SWA ranges")
    T, m, k, R = 1024, 2, 128, 48
    g = synth.rng(3, 5, synth.T_LATENT)
    xb = synth.to_bf16_bits(g.standard_normal((1, T, 512)).astype(np.float32))
    zb = synth.to_bf16_bits(synth.rng(3, 5, synth.T_GATE).standard_normal((1, T, 512)).astype(np.float32))
    codes, scales = O.kv_compress_quantize(xb[0], zb[0], m)      # the cache both sides read
    codes, scales = codes[None], scales[None]
    N = T // m
    keys = synth.to_e4m3(synth.rng(3, 5, synth.T_KEYS).standard_normal((1, N, 128)).astype(np.float32))
    swa = synth.to_e4m3(F.bf16_bits_to_f64(xb[0]).astype(np.float32))[None]   # window tokens, [1, T, 512]
    pos = np.arange(T - R, T)
    q_idx = synth.to_e4m3(synth.rng(3, 5, synth.T_QIDX).standard_normal((R, 32, 128)).astype(np.float32))
    q = synth.to_bf16_bits(synth.rng(3, 5, synth.T_QATTN).standard_normal((R, 64, 512)).astype(np.float32))
    views = [O.prefill_row_view(p, m) for p in pos]
    nv = np.array([v[0] for v in views], np.int32)
    lo = np.array([v[1] for v in views], np.int32)
    ln = np.array([v[2] for v in views], np.int32)
    row_seq = np.zeros(R, np.int32)
    idx = C.indexer_topk(dev(q_idx), dev(keys), k, row_seq=dev(row_seq), n_valid=dev(nv))
    out, lse = C.sparse_attn_decode(dev(q), dev(codes), dev(scales), idx, swa=dev(swa),
                                    swa_start=dev(lo), swa_len=dev(ln), row_seq=dev(row_seq))
    # the same rows with the window bound given (one key split per row instead
    # of splits planned for the whole window buffer), and with a bound below
    # the windows (each window clamped to its first 64 slots)
    out_b, lse_b = C.sparse_attn_decode(dev(q), dev(codes), dev(scales), idx, swa=dev(swa),
                                        swa_start=dev(lo), swa_len=dev(ln), row_seq=dev(row_seq),
                                        swa_max=128)
    out_c, lse_c = C.sparse_attn_decode(dev(q), dev(codes), dev(scales), idx, swa=dev(swa),
                                        swa_start=dev(lo), swa_len=dev(ln), row_seq=dev(row_seq),
                                        swa_max=64)
    torch.cuda.synchronize()
    gi, go, gl = host(idx), host(out), host(lse)
    gob, glb, goc, glc = host(out_b), host(lse_b), host(out_c), host(lse_c)
    assert ln.max() == 128
    differ = 0
    for r in range(R):
        sc = O.index_scores(q_idx[r], None, keys[0][:nv[r]])
        ref = O.topk_select(sc, np.arange(nv[r]), k)
        check_topk(gi[r], ref, np.arange(nv[r]), sc, k, f"row {r}")
        if not np.array_equal(gi[r], ref):
            differ += 1        # a tie swapped: the attention inputs differ legitimately
            continue
        Ox, lx = O.sparse_attn(q[r], codes[0], scales[0], ref, swa[0], range(lo[r], lo[r] + ln[r]))
        check_close(go[r], Ox, f"row {r} out")
        check_close(gl[r], lx, f"row {r} lse")
        check_close(gob[r], Ox, f"row {r} out (swa_max 128)")
        check_close(glb[r], lx, f"row {r} lse (swa_max 128)")
        Oc, lc = O.sparse_attn(q[r], codes[0], scales[0], ref, swa[0], range(lo[r], lo[r] + min(ln[r], 64)))
        check_close(goc[r], Oc, f"row {r} out (swa_max 64)")
        check_close(glc[r], lc, f"row {r} lse (swa_max 64)")
    assert differ <= 1
