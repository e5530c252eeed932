"""FP8 E4M3 ("e4m3fn") codec for the oracle.  Test infrastructure only.

The pages name the operand format only as "FP8" (ColossalAI PR #6419, "Fix:
Handle LowLevelZeroPlugin with use_fp8=True", "Forward pass"; pytorch/ao PR
#4390, "Add _grouped_mm dispatch handler to Float8Tensor", "Design").  The
format used here is the OCP 8-bit floating point E4M3 encoding with a maximum
finite magnitude of 448 and no infinities, which is the FP8 format gfx950's
matrix cores consume.  Encoding is round-to-nearest, ties-to-even, saturating
to +-448.

Decode (OCP OFP8 specification, E4M3 table):
  bit 7 = sign, bits 6..3 = exponent e (bias 7), bits 2..0 = mantissa m
  e == 0          : (-1)^s * m * 2^-9          (zero and subnormals)
  1 <= e <= 15    : (-1)^s * (1 + m/8) * 2^(e-7)
  e == 15, m == 7 : NaN (codes 0x7F and 0xFF); there is no infinity.

Parity pins live in ``tests/test_oracle_e4m3.py``: the OCP table points in
``tests/golden/e4m3_ocp_points.txt``, torch's CPU float8_e4m3fn view/cast,
brute force over every code midpoint, and the saturation rule.
"""

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def _decode_one(code):
    sign = -1.0 if (code & 0x80) else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def decode_table():
    """float64[256]: the value of every code (NaN for 0x7F / 0xFF)."""
    return np.array([_decode_one(c) for c in range(256)], dtype=np.float64)


_TABLE = decode_table()
# Magnitudes of the non-negative finite codes 0x00 .. 0x7E; strictly increasing,
# so the code index is the rank of the magnitude.
_MAGS = _TABLE[:0x7F].copy()
assert np.all(np.diff(_MAGS) > 0)


def decode(codes):
    """Decode uint8 codes to float64 values (exact)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(v):
    """Encode float32 values to E4M3 codes: round to nearest, ties to the code
    with an even mantissa, saturating to +-448; NaN -> 0x7F with v's sign; the
    sign bit is always v's sign bit (so -0.0 and tiny negatives give 0x80)."""
    v = np.asarray(v, dtype=np.float32)
    sign = np.signbit(v).astype(np.uint8) << 7
    nan = np.isnan(v)
    a = np.abs(v.astype(np.float64))
    a = np.where(nan, 0.0, np.minimum(a, MAX_FINITE))   # saturation (+inf too)
    hi = np.searchsorted(_MAGS, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    exact = _MAGS[hi] == a
    # The midpoint of two neighbouring codes is exact in float64, and so is a
    # (a float32 value), so these comparisons decide the rounding exactly.
    mid = (_MAGS[lo] + _MAGS[hi]) * 0.5
    even = np.where(lo % 2 == 0, lo, hi)
    mag = np.where(exact, hi,
                   np.where(a < mid, lo, np.where(a > mid, hi, even)))
    code = mag.astype(np.uint8) | sign
    code = np.where(nan, np.uint8(NAN_CODE) | sign, code)
    return code.astype(np.uint8)
