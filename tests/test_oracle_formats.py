"""Pins for the oracle's number formats: the definitions of E2M1 and E4M3FN,
checked exhaustively and against PyTorch's independent float8/bfloat16
implementations."""

import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e2m1_table_matches_definition():
    # E2M1: 2 exponent bits, 1 mantissa bit, bias 1, e=0 subnormal
    # (http://m.nxbn.cn/news/78290 §3.1; OCP MX element format).
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert F.E2M1_VALUES[:8].tolist() == pos
    assert F.E2M1_VALUES[8:].tolist() == [-v for v in pos]
    assert F.E2M1_MAGNITUDES.max() == 6.0


def test_e4m3_decode_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = F.E4M3_VALUES
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(mine))
    assert nan_ref.sum() == 2  # only S.1111.111
    assert np.array_equal(ref[~nan_ref], mine[~nan_ref])


def test_e4m3_anchors():
    assert F.e4m3_value(0x7E) == 448.0
    assert F.e4m3_value(0x38) == 1.0
    assert F.e4m3_value(0x08) == 2.0 ** -6       # smallest normal
    assert F.e4m3_value(0x01) == 2.0 ** -9       # smallest subnormal
    assert F.e4m3_value(0x07) == 7 * 2.0 ** -9   # largest subnormal
    assert np.isnan(F.e4m3_value(0x7F)) and np.isnan(F.e4m3_value(0xFF))


def test_e4m3_round_trip_all_codes():
    finite = [c for c in range(256) if not np.isnan(F.E4M3_VALUES[c])]
    vals = F.E4M3_VALUES[finite]
    back = F.e4m3_rne_sat(vals)
    for c, b in zip(finite, back):
        expect = 0 if c == 0x80 else c          # -0 encodes as +0
        assert b == expect, (hex(c), hex(b))


def test_e4m3_rne_vs_torch_random_and_midpoints():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(20000) * 10.0 ** g.uniform(-4, 2.6, 20000),
        # exact midpoints between consecutive finite values
        (F.E4M3_VALUES[1:0x7E] + F.E4M3_VALUES[2:0x7F]) / 2,
        -(F.E4M3_VALUES[1:0x7E] + F.E4M3_VALUES[2:0x7F]) / 2,
        [2.0 ** -10, 3 * 2.0 ** -11, 455.9, -455.9, 0.0],
    ])
    x = x[np.abs(x) < 464]           # torch saturates nothing; stay in range
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = F.e4m3_decode(F.e4m3_rne_sat(x))
    assert np.array_equal(ref, mine)


def test_e4m3_ties_go_to_even_code():
    # 1 + 1/16 lies halfway between 1 (0x38) and 1.125 (0x39): even wins
    assert F.e4m3_rne_sat(np.array([1.0625]))[0] == 0x38
    # 1.125 + 1/16 between 0x39 and 0x3A (1.25): even (0x3A) wins
    assert F.e4m3_rne_sat(np.array([1.1875]))[0] == 0x3A
    # half the smallest subnormal rounds to zero (+0)
    assert F.e4m3_rne_sat(np.array([-(2.0 ** -10)]))[0] == 0x00


def test_e4m3_saturates():
    assert (F.e4m3_rne_sat(np.array([448.0, 470.0, 1e6, 3e38])) == 0x7E).all()
    assert (F.e4m3_rne_sat(np.array([-470.0, -1e9])) == 0xFE).all()
    with pytest.raises(ValueError):
        F.e4m3_rne_sat(np.array([np.inf]))


def test_bf16_decode_vs_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = F.bf16_bits_to_f64(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(mine), ~ok)
    assert np.array_equal(ref[ok], mine[ok])


def test_fp4_times_scale_is_exact_in_bf16():
    # every E2M1 value times every finite E4M3 scale is exactly representable
    # in bfloat16, so dequantising to bf16 loses nothing
    s = F.E4M3_VALUES[~np.isnan(F.E4M3_VALUES)]
    prod = (F.E2M1_VALUES[:, None] * s[None, :]).ravel()
    back = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, prod)
