"""Pins of the MXFP8 oracle (oracle/mx.py and the "mxfp8" recipe of
oracle/gemm.py) against what the format definition fixes: the shared
exponent in closed form, exact round trips of values the format represents,
the block-maximum band, saturation, and exact GEMMs by rational arithmetic."""

import math
from fractions import Fraction

import numpy as np

import workloads
from oracle import e4m3, gemm, mx, quant


def _bits(v32):
    return workloads.f32_to_bf16_bits(np.asarray(v32, np.float32))


def test_shared_exponent_closed_form():
    rng = np.random.default_rng(1)
    vals = np.concatenate([np.exp2(rng.uniform(-140, 127, 2000)), [2.0 ** -133, 1.0, 448.0, 511.9, 3.0e38],
                           np.exp2(np.arange(-126, 128, dtype=np.float64))])
    vals = quant.bf16_to_f32(_bits(vals)).astype(np.float64)
    vals = vals[vals > 0]
    got = mx.shared_exponent(vals)
    for v, e in zip(vals, got):
        m, ex = math.frexp(float(v))                  # v = m 2^ex, 0.5 <= m < 1
        assert e == max(-127, min(127, ex - 1 - 8)), (v, e)
    assert mx.shared_exponent(np.array([0.0]))[0] == -127


def test_exact_round_trip_of_representable_blocks():
    """A block of e4m3 values times 2^m whose largest magnitude is in [256,
    448] has E = m and comes back exactly."""
    rng = np.random.default_rng(2)
    mags = e4m3.decode(np.arange(0x7F, dtype=np.uint8))     # 0 .. 448
    rows = []
    for m in rng.integers(-100, 100, size=64):
        blk = rng.choice(mags, size=32) * rng.choice([-1.0, 1.0], size=32)
        blk[rng.integers(0, 32)] = rng.choice(mags[(mags >= 256) & (mags <= 448)])
        rows.append(blk * 2.0 ** float(m))
    x = np.array(rows)                                      # float64, exact in bf16? check
    xb = _bits(x)
    assert np.array_equal(quant.bf16_to_f32(xb).astype(np.float64), x)   # e4m3 values fit bf16
    q, s = mx.quantize_mx(xb)
    assert np.array_equal(mx.dequantize_mx(q, s), x)


def test_block_maximum_band_and_saturation():
    g = workloads.streams(3, 1)
    x = workloads.normal_bf16(g[0], (64, 256), 3.0)
    q, s = mx.quantize_mx(x)
    dec = np.abs(e4m3.decode(q)).reshape(64, 8, 32).max(axis=2)
    assert np.all((dec >= 256) & (dec <= 448)), dec.min()
    # a block whose maximum is 500 * 2^E saturates to the largest code
    blk = np.full((1, 32), 1.0)
    blk[0, 5] = 500.0 / 256.0            # amax = 1.953125: E = -8, quotient 500 -> 448
    q, s = mx.quantize_mx(_bits(blk))
    assert s[0, 0] == 127 - 8 and q[0, 5] == 0x7E and q[0, 0] == e4m3.encode(np.float32(256.0))


def test_zero_block_and_signs():
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = -1.0
    x[0, 3] = -0.0
    q, s = mx.quantize_mx(_bits(x))
    assert s[0, 0] == 0 and s[0, 1] == 0                 # E = -127
    assert q[0, 3] == 0x80 and q[0, 0] == 0x00
    assert s[1, 1] == 127 - 8 and np.all(q[1, 32:] == (0x80 | e4m3.encode(np.float32(256.0))))


def _exact(qa, sa, qb, sb):
    M, K = qa.shape
    N = qb.shape[0]
    da, db = e4m3.decode(qa), e4m3.decode(qb)
    out = np.zeros((M, N))
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(da[i, k]) * Fraction(2) ** (int(sa[i, k // 32]) - 127) *
                        Fraction(db[j, k]) * Fraction(2) ** (int(sb[j, k // 32]) - 127))
            out[i, j] = float(acc)
    return out


def test_mx_gemm_exact_by_fractions():
    g = workloads.streams(4, 2)
    a = workloads.normal_bf16(g[0], (5, 64))
    b = workloads.normal_bf16(g[1], (3, 64), 0.02)
    qa, sa = mx.quantize_mx(a)
    qb, sb = mx.quantize_mx(b)
    got = gemm.scaled_mm_exact(qa, qb, sa, "mxfp8", sb, "mxfp8")
    assert np.array_equal(got, _exact(qa, sa, qb, sb))


def test_mx_with_unit_scales_is_the_tensorwise_gemm():
    rng = np.random.default_rng(5)
    qa = rng.integers(0, 256, size=(7, 96)).astype(np.uint8)
    qb = rng.integers(0, 256, size=(4, 96)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0
    qb[(qb & 0x7F) == 0x7F] = 0
    ones_a = np.full((7, 3), 127, np.uint8)
    ones_b = np.full((4, 3), 127, np.uint8)
    one = np.ones(1, np.float32)
    assert np.array_equal(gemm.scaled_mm_exact(qa, qb, ones_a, "mxfp8", ones_b, "mxfp8"),
                          gemm.scaled_mm_exact(qa, qb, one, "tensorwise", one, "tensorwise"))
