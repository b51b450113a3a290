"""Comparison rules between the HIP path and the oracle.

* top-k sets: equal, except that an entry whose oracle score lies within
  1e-5 * |I_k| of the k-th oracle score may be swapped for another such
  entry (I_k = the k-th largest oracle score of the row); ids ascending,
  padded with -1 to the same count.
* attention: |gpu - ref| <= 2e-3 + 1e-2 * |ref| elementwise, for the output
  and the log-sum-exp (both -inf when a row has no key).
"""

import sys

import numpy as np
import torch

from oracle import formats as F

TOPK_REL = 1e-5
ATOL, RTOL = 2e-3, 1e-2
E2M1_THRESH = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)   # midpoints of the E2M1 magnitudes


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    """numpy -> GPU tensor (uint16 bf16 bits travel as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    return t.detach().cpu().numpy()


def check_topk(gpu_ids, ref_ids, ids, scores, k, what=""):
    """gpu_ids/ref_ids: [k] ascending, -1 padded.  ids/scores: the oracle's
    candidate ids and float64 scores (the set both sides chose from)."""
    gpu_ids = np.asarray(gpu_ids, dtype=np.int64)
    ref_ids = np.asarray(ref_ids, dtype=np.int64)
    g = gpu_ids[gpu_ids >= 0]
    r = ref_ids[ref_ids >= 0]
    assert len(g) == len(r), f"{what}: {len(g)} ids vs {len(r)}"
    assert np.all(np.diff(g) > 0), f"{what}: gpu ids not strictly ascending"
    assert np.all(gpu_ids[len(g):] == -1), f"{what}: padding"
    if len(r) == 0:
        return 0
    score_of = dict(zip(np.asarray(ids).tolist(), np.asarray(scores).tolist()))
    assert all(int(x) in score_of for x in g), f"{what}: gpu chose an id outside the candidates"
    ik = min(score_of[int(x)] for x in r)
    band = TOPK_REL * abs(ik)
    diff = set(g.tolist()) ^ set(r.tolist())
    bad = [x for x in diff if abs(score_of[int(x)] - ik) > band]
    assert not bad, f"{what}: {len(bad)} ids differ outside the tie band (I_k={ik}): {sorted(bad)[:8]}"
    return len(diff)


def check_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, what
    inf_r, inf_g = np.isneginf(ref), np.isneginf(gpu)
    assert np.array_equal(inf_r, inf_g), f"{what}: -inf pattern differs"
    fin = ~inf_r
    err = np.abs(gpu[fin] - ref[fin])
    lim = ATOL + RTOL * np.abs(ref[fin])
    worst = np.max(err / lim) if err.size else 0.0
    assert np.all(err <= lim), f"{what}: {np.sum(err > lim)} elements outside tolerance (worst {worst:.3g} of the bound)"
    return worst


def near_boundary(yg, rel=4e-7):
    """True if a float32 group of 16 pooled values sits within `rel` of a
    decision boundary of the quantiser: amax/6 near an E4M3 rounding
    midpoint, or a value near a midpoint t*s of the E2M1 grid.  Pooling with
    gates runs in float32 on the GPU and in float64 in the oracle, so only
    such groups may quantise differently."""
    amax = np.float32(np.abs(yg).max())
    q = float(amax / np.float32(6))
    mids = (F.E4M3_VALUES[0:0x7E] + F.E4M3_VALUES[1:0x7F]) / 2
    if np.any(np.abs(mids - q) <= rel * max(q, 1e-30)):
        return True
    s = float(F.e4m3_decode(F.e4m3_rne_sat(np.float64(q))))
    a = np.abs(yg)
    return bool(np.any(np.abs(a[:, None] - s * np.array(E2M1_THRESH)[None, :]) <= rel * a[:, None].clip(1e-30)))
