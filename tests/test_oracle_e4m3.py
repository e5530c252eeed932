"""Pins for the oracle's E4M3 codec (CPU only).

The codec is pinned to things other than itself: the OCP specification's
table points (tests/golden/e4m3_ocp_points.txt), torch's CPU float8_e4m3fn
view and cast (a library routine, independent of the oracle), and brute force
over every midpoint between neighbouring codes.
"""

import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_points.txt")


def _golden_points():
    pts = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code, val = line.split()
            try:
                v = float(val)                       # "nan", "-0", "448", ...
            except ValueError:
                v = float(eval(val, {}))             # "2**-9" style expressions
            pts.append((int(code, 16), v))
    return pts


def test_decode_matches_ocp_table_points():
    table = e4m3.decode_table()
    pts = _golden_points()
    assert len(pts) >= 15
    for code, val in pts:
        if np.isnan(val):
            assert np.isnan(table[code]), hex(code)
        else:
            assert table[code] == val, hex(code)
            assert np.signbit(table[code]) == np.signbit(val), hex(code)


def test_decode_matches_torch_float8_e4m3fn_for_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    table = e4m3.decode_table()
    assert np.array_equal(np.isnan(ref), np.isnan(table))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], table[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(table[ok]))


def test_table_shape_facts():
    t = e4m3.decode_table()
    finite = t[~np.isnan(t)]
    assert finite.size == 254
    assert finite.max() == 448.0 and finite.min() == -448.0
    assert np.min(np.abs(finite[finite != 0])) == 2.0 ** -9
    assert {c for c in range(256) if np.isnan(t[c])} == {0x7F, 0xFF}


def _torch_encode(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_every_inrange_bf16_value():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    assert v.size > 30000
    assert np.array_equal(e4m3.encode(v), _torch_encode(v))


def test_encode_matches_torch_on_random_fp32():
    rng = np.random.default_rng(12345)
    mag = np.exp2(rng.uniform(-16, np.log2(448.0), 1 << 20)).astype(np.float32)
    mag = np.minimum(mag, np.float32(448.0))
    v = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    assert np.array_equal(e4m3.encode(v), _torch_encode(v))


def test_every_midpoint_ties_to_even_and_neighbours_round_correctly():
    t = e4m3.decode_table()[:0x7F]
    for c in range(0x7E):
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2            # midpoints are fp32-exact
        even = c if c % 2 == 0 else c + 1
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(1e9))
        got = e4m3.encode(np.array([mid, below, above, -mid], np.float32))
        assert list(got) == [even, c, c + 1, even | 0x80], (c, got)


def test_saturation_nan_and_signed_zero():
    v = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, np.inf,
                  -449.0, -np.inf, np.nan, -np.nan, 0.0, -0.0, -1e-30, 1e-30,
                  2.0 ** -10, -(2.0 ** -10), 2.0 ** -10 * 1.0000001], np.float32)
    got = e4m3.encode(v)
    exp = [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E,
           0xFE, 0xFE, 0x7F, 0xFF, 0x00, 0x80, 0x80, 0x00,
           0x00, 0x80, 0x01]
    assert list(got) == exp


def test_round_trip_every_finite_code():
    t = e4m3.decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], np.uint8)
    assert np.array_equal(e4m3.encode(t[codes].astype(np.float32)), codes)
