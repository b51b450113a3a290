"""Number formats of the CSA2 cache, written out from their definitions.

* FP4 E2M1 -- the main-KV element format named ``fp4_e2m1`` in the inference
  configuration [0539edu §3]; a sign bit, a 2-bit exponent with bias 1 and a
  1-bit mantissa [nxbn §3.1].  e = 0 is subnormal; there is no inf or NaN.
* FP8 E4M3 -- the per-16-channel scale (``e4m3_per_16_channel``) and the SWA
  cache (``swa_kv_dtype: fp8``) [0539edu §3].  Read as the OCP "FN" variant:
  bias 7, largest finite 448, no infinities, NaN = S.1111.111, subnormals down
  to 2**-9.
* bfloat16 -- the query and latent activation format; decoded exactly.

Rounding into E4M3 is round-to-nearest-even with saturation to +-448, and a
value that rounds to zero is encoded as +0 (code 0x00).

Test infrastructure only (see the package docstring).
"""

import numpy as np

# ---------------------------------------------------------------------------
# E2M1
# ---------------------------------------------------------------------------


def e2m1_value(code):
    """Value of a 4-bit E2M1 code from its bit fields [nxbn §3.1]."""
    code = int(code) & 0xF
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m * 0.5)
    return -mag if s else mag


E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
# The eight non-negative magnitudes in code order 0..7.
E2M1_MAGNITUDES = E2M1_VALUES[:8].copy()


def e2m1_decode(codes):
    """Decode an integer array of E2M1 codes (0..15) to float64."""
    return E2M1_VALUES[np.asarray(codes, dtype=np.int64) & 0xF]


# ---------------------------------------------------------------------------
# E4M3 (OCP FN)
# ---------------------------------------------------------------------------


def e4m3_value(code):
    """Value of an 8-bit E4M3FN code from its bit fields (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** (1 - 7) if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


E4M3_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_MAX = 448.0
# Non-negative finite codes 0x00..0x7E, whose values increase with the code.
_E4M3_POS = E4M3_VALUES[:0x7F].copy()


def e4m3_decode(codes):
    """Decode a uint8 array of E4M3FN codes to float64."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def e4m3_rne_sat(x):
    """Round float64 values to E4M3FN codes: nearest, ties to the even code,
    saturating at +-448; values that round to zero give +0.

    Written as a search over the sorted grid of finite non-negative values:
    the two neighbours of |x| are found and the nearer one kept; an exact tie
    keeps the neighbour whose code is even.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_rne_sat: non-finite input")
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first grid value >= a
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    vlo, vhi = _E4M3_POS[lo], _E4M3_POS[hi]
    exact = vhi == a
    dlo, dhi = a - vlo, vhi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    mag = np.where(exact, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    sign = ((x < 0) & (mag != 0)).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


# ---------------------------------------------------------------------------
# bfloat16 / float32 helpers
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits):
    """Decode bfloat16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
