"""Pins of the oracle's grouped (MoE) variants: the blockwise grouped GEMM in
both weight layouts, the per-expert 128x1 quantization in the padded token
layout, and the per-expert weight gradient.

Each is tied to something other than its own code: exact rational sums with
the expert and scale lookups written out element by element, the already
pinned dense functions on the cases where the grouped form reduces to them
(one expert; runs that are whole 128-token blocks), and the identity that
zero rows never raise a run's maximum (a short run quantizes like the run
zero-padded to 128 rows).
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, gemm, quant
from workloads import normal_bf16, streams

TABLE = e4m3.decode_table()
DEC = [Fraction(float(v)) if not np.isnan(v) else None for v in TABLE]


def _frac_round_bf16(fr):
    if fr == 0:
        return 0.0
    sgn = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = max(e - 7, -133)
    scaled = a / Fraction(2) ** q
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sgn * float(Fraction(n) * Fraction(2) ** q)


def _rand_codes(rng, shape):
    c = rng.integers(0, 0x7F, size=shape).astype(np.uint8)      # finite magnitudes
    return c | (rng.integers(0, 2, size=shape).astype(np.uint8) << 7)


def _expert_of(offs, i):
    """The expert that owns row i (scanning the end offsets), or None."""
    start = 0
    for e, end in enumerate(offs):
        if start <= i < end:
            return e
        start = max(start, int(end))
    return None


@pytest.mark.parametrize("layout", ["NK", "KN"])
def test_grouped_blockwise_matches_exact_rationals(layout):
    rng = np.random.default_rng(31)
    E, N, K = 3, 128, 256
    offs = np.array([3, 3, 5], np.int32)           # expert 1 empty, row 5 unowned
    M = 6
    A = _rand_codes(rng, (M, K))
    W = _rand_codes(rng, (E, N, K) if layout == "NK" else (E, K, N))
    sa = rng.uniform(0.001, 2.0, size=(K // 128, M)).astype(np.float32)
    grid = (N // 128, K // 128) if layout == "NK" else (K // 128, N // 128)
    sb = rng.uniform(0.001, 2.0, size=(E,) + grid).astype(np.float32)
    bias = rng.uniform(-1, 1, size=(E, N)).astype(np.float32)
    out, written = gemm.grouped_mm(A, W, offs, sa, sb, bias=bias, recipe_a="1x128",
                                   recipe_b="128x128", layout=layout)
    assert written.tolist() == [True] * 5 + [False]
    assert np.isnan(out[5]).all()
    cols = [0, 1, 77, 127]
    for i in range(5):
        e = _expert_of(offs, i)
        for j in cols:
            acc = Fraction(float(bias[e, j]))
            for k in range(K):
                w = W[e, j, k] if layout == "NK" else W[e, k, j]
                s_b = sb[e, j // 128, k // 128] if layout == "NK" else sb[e, k // 128, j // 128]
                acc += DEC[A[i, k]] * Fraction(float(sa[k // 128, i])) * DEC[w] * Fraction(float(s_b))
            assert out[i, j] == _frac_round_bf16(acc), (layout, i, j)


@pytest.mark.parametrize("layout", ["NK", "KN"])
def test_grouped_single_expert_is_the_dense_blockwise_gemm(layout):
    g = streams(32, 2)
    x = normal_bf16(g[0], (40, 256))
    w = normal_bf16(g[1], (256, 384) if layout == "KN" else (384, 256), 0.02)
    qa, sa = quant.quantize_blockwise(x, 1, 128)
    qw, sw = quant.quantize_blockwise(w, 128, 128)
    out, written = gemm.grouped_mm(qa, qw[None], np.array([40], np.int32), sa, sw[None],
                                   recipe_a="1x128", recipe_b="128x128", layout=layout)
    assert written.all()
    assert np.array_equal(out, gemm.scaled_mm(qa, qw, sa, "1x128", sw, "128x128", layout))


def test_grouped_rejects_other_recipes():
    z = np.zeros((2, 128), np.uint8)
    with pytest.raises(NotImplementedError):
        gemm.grouped_mm(z, np.zeros((1, 128, 128), np.uint8), np.array([2]), np.ones(1), np.ones(1),
                        recipe_a="tensorwise", recipe_b="tensorwise")


def test_grouped_128x1_whole_runs_are_the_dense_128x1_quantization():
    g = streams(33, 1)
    sizes = [256, 0, 128, 384]
    offs = np.cumsum(sizes).astype(np.int32)
    x = normal_bf16(g[0], (int(offs[-1]) + 5, 64))      # 5 trailing rows no expert owns
    qt, st, first = quant.quantize_grouped_128x1(x, offs)
    assert first.tolist() == [0, 2, 2, 3]
    assert qt.shape == (64, 128 * 6) and st.shape == (6, 64)
    start = 0
    for e, m in enumerate(sizes):
        if m:
            q_ref, s_ref = quant.quantize_blockwise(x[start:start + m], 128, 1, transpose_out=True)
            b = int(first[e])
            assert np.array_equal(qt[:, 128 * b:128 * b + m], q_ref)
            assert np.array_equal(st[b:b + m // 128], s_ref)
        start += m


def test_grouped_128x1_short_runs_equal_zero_padded_runs():
    """Zeros never raise a maximum: a short run quantizes exactly like the
    same run with zero rows appended up to 128, whose codes are 0."""
    g = streams(34, 1)
    sizes = [130, 5, 0, 257, 1]
    offs = np.cumsum(sizes).astype(np.int32)
    x = normal_bf16(g[0], (int(offs[-1]), 32))
    qt, st, first = quant.quantize_grouped_128x1(x, offs)
    assert first.tolist() == [0, 2, 3, 3, 6]
    assert qt.shape == (32, 128 * 7)
    start = 0
    for e, m in enumerate(sizes):
        if m:
            nb = (m + 127) // 128
            padded = np.zeros((128 * nb, 32), np.uint16)
            padded[:m] = x[start:start + m]
            q_ref, s_ref = quant.quantize_blockwise(padded, 128, 1, transpose_out=True)
            b = int(first[e])
            assert np.array_equal(qt[:, 128 * b:128 * (b + nb)], q_ref)
            assert not qt[:, 128 * b + m:128 * (b + nb)].any()
            assert np.array_equal(st[b:b + nb], s_ref)
        start += m


def test_grouped_128x1_amax_element_reaches_448():
    g = streams(35, 1)
    sizes = [70, 200, 3]
    offs = np.cumsum(sizes).astype(np.int32)
    x = normal_bf16(g[0], (273, 16), 3.0)
    qt, st, first = quant.quantize_grouped_128x1(x, offs)
    xv = quant.bf16_to_f32(x)
    start = 0
    for e, m in enumerate(sizes):
        for j in range((m + 127) // 128):
            r0, r1 = start + 128 * j, min(start + 128 * j + 128, start + m)
            b = int(first[e]) + j
            codes = qt[:, 128 * b:128 * b + (r1 - r0)]          # [C, rows]
            mag = TABLE[codes & 0x7F]
            assert (mag.max(axis=1) == 448.0).all()
            amax = np.abs(xv[r0:r1]).max(axis=0)
            assert np.array_equal(st[b], (amax / np.float32(448)).astype(np.float32))
        start += m


def test_grouped_grad_weight_matches_exact_rationals():
    """Expert 0: 130 tokens (a full run and a 2-token run), expert 1: none,
    expert 2: 10 tokens.  The pad columns carry nonzero codes here, which the
    definition (a sum over the expert's own tokens) must ignore."""
    rng = np.random.default_rng(36)
    sizes = [130, 0, 10]
    offs = np.cumsum(sizes).astype(np.int32)
    _, _, first, nb = quant.grouped_blocks(offs)
    NB = int(nb.sum())
    N_out, K_in = 2, 3
    gq = _rand_codes(rng, (N_out, 128 * NB))
    xq = _rand_codes(rng, (K_in, 128 * NB))
    gs = rng.uniform(0.001, 2.0, size=(NB, N_out)).astype(np.float32)
    xs = rng.uniform(0.001, 2.0, size=(NB, K_in)).astype(np.float32)
    out = gemm.grouped_grad_weight(gq, gs, xq, xs, offs)
    assert out.shape == (3, N_out, K_in)
    assert not out[1].any()
    for e, m in enumerate(sizes):
        for n in range(N_out):
            for k in range(K_in):
                acc = Fraction(0)
                for t in range(m):                 # the expert's t-th token
                    col = 128 * int(first[e]) + t
                    run = int(first[e]) + t // 128
                    acc += (DEC[gq[n, col]] * Fraction(float(gs[run, n]))
                            * DEC[xq[k, col]] * Fraction(float(xs[run, k])))
                assert out[e, n, k] == _frac_round_bf16(acc), (e, n, k)


def test_grouped_grad_weight_single_expert_is_the_dense_weight_gradient():
    g = streams(37, 2)
    go = normal_bf16(g[0], (256, 48), 1e-3)
    x = normal_bf16(g[1], (256, 80))
    offs = np.array([256], np.int32)
    gq, gs, _ = quant.quantize_grouped_128x1(go, offs)
    xq, xs, _ = quant.quantize_grouped_128x1(x, offs)
    out = gemm.grouped_grad_weight(gq, gs, xq, xs, offs, out_dtype="fp32")
    qg, sg = quant.quantize_blockwise(go, 128, 1, transpose_out=True)
    qx, sx = quant.quantize_blockwise(x, 128, 1, transpose_out=True)
    assert np.array_equal(out[0], gemm.linear_grad_weight(qg, sg, qx, sx, out_dtype="fp32"))


def test_grouped_grad_weight_splits_the_dense_sum_by_expert():
    """With experts whose token counts are multiples of 128, the experts'
    gradients add up (before rounding) to the dense weight gradient over all
    tokens with the same 128-token runs."""
    g = streams(38, 2)
    sizes = [128, 256, 0, 128]
    offs = np.cumsum(sizes).astype(np.int32)
    go = normal_bf16(g[0], (512, 32), 1e-3)
    x = normal_bf16(g[1], (512, 40))
    gq, gs, _ = quant.quantize_grouped_128x1(go, offs)
    xq, xs, _ = quant.quantize_grouped_128x1(x, offs)
    per = gemm.grouped_grad_weight(gq, gs, xq, xs, offs, out_dtype=None)
    qg, sg = quant.quantize_blockwise(go, 128, 1, transpose_out=True)
    qx, sx = quant.quantize_blockwise(x, 128, 1, transpose_out=True)
    dense = gemm.scaled_mm_exact(qg, qx, sg, "1x128", sx, "128x1")
    assert np.allclose(per.sum(axis=0), dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())
