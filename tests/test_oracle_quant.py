"""Pins for the oracle's cache write: pooling, FP4 quantisation, block
summaries.  Each test checks the oracle against something other than itself:
an exact round trip, an independent threshold formulation of the rounding,
closed forms of the pooling, or PyTorch's float8 rounding."""

import numpy as np
import torch

from oracle import csa2 as O
from oracle import formats as F

# Decision thresholds of nearest-with-ties-to-even on the E2M1 grid, in units
# of the scale, and whether an exact tie rounds up (to the even code above).
THRESH = [(0.25, False), (0.75, True), (1.25, False), (1.75, True),
          (2.5, False), (3.5, True), (5.0, False)]


def threshold_codes(y, s):
    """Independent formulation: the magnitude code is the number of
    thresholds that |y| passes (strictly, or at equality when the tie rounds
    up)."""
    a = np.abs(y)
    mag = np.zeros(a.shape, dtype=np.int64)
    for t, up in THRESH:
        mag += (a >= t * s) if up else (a > t * s)
    if s == 0:
        mag[:] = 0
    return mag + 8 * ((y < 0) & (mag != 0))


def nibbles(codes):
    return O.unpack_fp4(codes)


def test_round_trip_canonical_groups():
    g = np.random.default_rng(2)
    E = 300
    nib = g.integers(0, 16, size=(E, 512))
    nib[:, ::16] = np.where(g.random((E, 32)) < 0.5, 7, 15)   # a +-6 in every group
    nib[nib == 8] = 0                                          # no -0 codes
    s_codes = g.integers(0x08, 0x7E, size=(E, 32)).astype(np.uint8)  # normal scales
    y = F.e2m1_decode(nib) * np.repeat(F.e4m3_decode(s_codes), 16, axis=1)
    codes, scales = O.quantize_fp4(y)
    assert np.array_equal(scales, s_codes)
    assert np.array_equal(nibbles(codes), nib)
    assert np.array_equal(O.dequantize_fp4(codes, scales), y)


def test_matches_threshold_rule_random_and_ties():
    g = np.random.default_rng(3)
    E = 400
    y = g.standard_normal((E, 512)).astype(np.float32).astype(np.float64)
    # plant exact ties at every threshold in some groups
    codes0, scales0 = O.quantize_fp4(y)
    s = np.repeat(F.e4m3_decode(scales0), 16, axis=1)
    for i, (t, _) in enumerate(THRESH):
        rows = slice(i * 40, i * 40 + 40)
        cols = np.arange(1, 512, 16)          # keep channel 0 (group max) intact
        sign = np.where(g.random((40, len(cols))) < 0.5, -1.0, 1.0)
        y[rows, cols] = sign * t * s[rows, cols]
    codes, scales = O.quantize_fp4(y)
    sc = F.e4m3_decode(scales)
    nib = nibbles(codes)
    for e in range(E):
        for gi in range(32):
            sl = slice(gi * 16, gi * 16 + 16)
            amax = np.float32(np.abs(y[e, sl]).max())
            expect_s = F.e4m3_rne_sat(np.float64(amax / np.float32(6)))
            assert scales[e, gi] == expect_s
            assert np.array_equal(nib[e, sl], threshold_codes(y[e, sl], sc[e, gi]))


def test_scale_edge_cases():
    y = np.zeros((4, 512))
    y[1, :16] = 2.0 ** -12                  # amax/6 below half the smallest subnormal scale
    y[2, :16] = np.linspace(-1e5, 1e5, 16)  # amax/6 above 448: scale saturates
    y[2, 16:32] = np.linspace(-3e38, 3e38, 16)   # far beyond the grid
    y[3, :16] = -0.0
    codes, scales = O.quantize_fp4(y)
    assert (scales[0] == 0).all() and (codes[0] == 0).all()
    assert scales[1, 0] == 0 and (codes[1, :8] == 0).all()
    assert scales[2, 0] == 0x7E
    nib = nibbles(codes)
    assert nib[2, 0] == 15 and nib[2, 15] == 7          # clipped to -+6 * 448
    assert nib[2, 16] == 15 and nib[2, 31] == 7 and scales[2, 1] == 0x7E
    assert (codes[3] == 0).all()                         # no negative zero


def test_subnormal_scale():
    y = np.zeros((1, 512))
    y[0, :16] = np.array([3 * 2.0 ** -9 * 6] + [0.0] * 15)  # amax/6 = 3 * 2^-9 (subnormal)
    codes, scales = O.quantize_fp4(y)
    assert scales[0, 0] == 0x03
    assert nibbles(codes)[0, 0] == 7


def test_pool_closed_forms():
    g = np.random.default_rng(4)
    x = g.standard_normal((64, 512)).astype(np.float32).astype(np.float64)
    # m = 1: identity
    assert np.array_equal(O.pool(x, None, 1), x)
    # no logits: the mean of each pair
    y = O.pool(x, None, 2)
    assert np.array_equal(y, ((x[0::2] + x[1::2]) / 2).astype(np.float32).astype(np.float64))
    # equal logits: the mean
    z = np.repeat(g.standard_normal((32, 1, 512)), 2, axis=1).reshape(64, 512)
    assert np.allclose(O.pool(x, z, 2), y, rtol=1e-7, atol=0)
    # a dominant logit selects its token
    z = np.zeros((64, 512))
    z[1::2] = 200.0
    assert np.array_equal(O.pool(x, z, 2), x[1::2])
    # two-token softmax closed form: sigmoid weights
    z = g.standard_normal((64, 512))
    p0 = 1.0 / (1.0 + np.exp(z[1::2] - z[0::2]))
    expect = (p0 * x[0::2] + (1 - p0) * x[1::2]).astype(np.float32).astype(np.float64)
    assert np.allclose(O.pool(x, z, 2), expect, rtol=2e-7, atol=1e-30)
    # convexity
    y4 = O.pool(x, g.standard_normal((64, 512)), 4)
    assert (np.abs(y4) <= np.abs(x).reshape(16, 4, 512).max(axis=1) * (1 + 1e-7)).all()


def test_pool_permutation_invariant_within_group():
    g = np.random.default_rng(5)
    x = g.standard_normal((8, 512))
    z = g.standard_normal((8, 512))
    perm = np.array([1, 0, 3, 2, 5, 4, 7, 6])
    assert np.allclose(O.pool(x, z, 2), O.pool(x[perm], z[perm], 2), rtol=1e-7, atol=0)


def test_kv_compress_quantize_drops_partial_group():
    g = np.random.default_rng(6)
    xb = torch.from_numpy(g.standard_normal((7, 512)).astype(np.float32)).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    codes, scales = O.kv_compress_quantize(bits, None, 2)
    assert codes.shape == (3, 256) and scales.shape == (3, 32)


def test_block_summary_vs_torch_mean():
    g = np.random.default_rng(7)
    for N in (64, 61, 8, 1, 13):
        keys = torch.from_numpy(g.standard_normal((N, 128)).astype(np.float32) * 3).to(
            torch.float8_e4m3fn)
        kf = keys.to(torch.float64)
        nb = (N + 7) // 8
        ref = torch.stack([kf[b * 8:(b + 1) * 8].mean(0) for b in range(nb)])
        ref = ref.to(torch.float8_e4m3fn).to(torch.float64).numpy()   # independent RNE
        mine = F.e4m3_decode(O.block_summary(keys.view(torch.uint8).numpy()))
        assert np.array_equal(mine, ref), N


def test_fp4_byte_layout_by_hand():
    # channel 2j in the low nibble of byte j; one scale per 16 channels
    y = np.zeros((1, 512))
    y[0, 0] = 3.0        # group 0 amax 3 -> scale 0.5 (0x30); 3.0 = 6 * 0.5 -> code 7
    y[0, 1] = -0.5       # -> -1 * 0.5 -> code 8 + 2 = 10
    y[0, 17] = 12.0      # group 1: amax 12 -> scale 2 (0x40); code 7 in the high nibble of byte 8
    y[0, 16] = 1.0       # 0.5 * 2 -> code 1 in the low nibble of byte 8
    codes, scales = O.quantize_fp4(y)
    assert scales[0, 0] == 0x30 and scales[0, 1] == 0x40 and (scales[0, 2:] == 0).all()
    assert codes[0, 0] == 0xA7
    assert codes[0, 8] == 0x71
    assert (np.delete(codes[0], [0, 8]) == 0).all()
    d = O.dequantize_fp4(codes, scales)[0]
    assert d[0] == 3.0 and d[1] == -0.5 and d[16] == 1.0 and d[17] == 12.0
