"""Pins for the oracle's scaled GEMM (CPU only).

  * exact small-integer GEMMs (values exactly representable in E4M3, scale 1):
    the result is the exact integer matmul;
  * exact rational GEMMs (fractions.Fraction): every E4M3 value and float32
    scale is a dyadic rational, so the true value exists and is rounded to
    bf16 exactly once by an independent rational rounding;
  * the per-128-block scaled-sum invariant (blockwise scaled GEMM == GEMM of
    the dequantized operands);
  * transposition identities for the grad_input / grad_weight call forms;
  * grouped GEMM == concatenated per-expert rowwise GEMMs; E = 1 == rowwise;
  * bf16 output rounding against torch's CPU rounding;
  * the SQNR sanity floor of the MoE tests (pytorch/ao PR #4390, "Test plan").
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3, gemm, quant
from workloads import f32_to_bf16_bits, normal_bf16, streams

TABLE = e4m3.decode_table()
INT_CODES = {int(v): c for c, v in enumerate(TABLE[:0x7F]) if float(v).is_integer() and v <= 16}


def _int_codes(vals):
    mag = np.vectorize(lambda v: INT_CODES[abs(int(v))])(vals).astype(np.uint8)
    return (mag | ((vals < 0).astype(np.uint8) << 7)).astype(np.uint8)


def test_small_integer_gemm_is_exact():
    rng = np.random.default_rng(1)
    a = rng.integers(-16, 17, size=(24, 256))
    b = rng.integers(-16, 17, size=(40, 256))
    A, B = _int_codes(a), _int_codes(b)
    one = np.ones(1, np.float32)
    out = gemm.scaled_mm(A, B, one, "tensorwise", one, "tensorwise", out_dtype="fp32")
    assert np.array_equal(out, (a @ b.T).astype(np.float64))
    # layout KN reads the same logical operand
    out_kn = gemm.scaled_mm(A, np.ascontiguousarray(B.T), one, "tensorwise", one, "tensorwise",
                            layout="KN", out_dtype="fp32")
    assert np.array_equal(out_kn, out)
    # with an integer bias
    bias = rng.integers(-50, 50, size=40)
    out_b = gemm.scaled_mm(A, B, one, "tensorwise", one, "tensorwise", bias=bias, out_dtype="fp32")
    assert np.array_equal(out_b, (a @ b.T + bias).astype(np.float64))


def _frac_round_bf16(fr):
    """Round a Fraction to bf16 exactly (nearest, ties to even) -> float."""
    if fr == 0:
        return 0.0
    sgn = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = max(e - 7, -133)                    # ulp exponent: 8 significant bits
    scaled = a / Fraction(2) ** q
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sgn * float(Fraction(n) * Fraction(2) ** q)


def _exact_scaled(A, B, sa_fn, sb_fn, bias=None):
    M, K = A.shape
    N = B.shape[0]
    dec = [Fraction(float(v)) if not np.isnan(v) else None for v in TABLE]
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += dec[A[i, k]] * Fraction(float(sa_fn(i, k))) * dec[B[j, k]] * Fraction(float(sb_fn(j, k)))
            if bias is not None:
                acc += Fraction(float(bias[j]))
            out[i][j] = acc
    return out


@pytest.mark.parametrize("recipe_b", ["128x128", "128x1"])
def test_blockwise_gemm_matches_exact_rationals(recipe_b):
    rng = np.random.default_rng(2)
    M, N, K = 3, 130, 256
    N = 128 if recipe_b == "128x128" else 5
    A = rng.integers(0, 0x7F, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, size=(M, K)).astype(np.uint8) << 7)
    B = rng.integers(0, 0x7F, size=(N, K)).astype(np.uint8) | (rng.integers(0, 2, size=(N, K)).astype(np.uint8) << 7)
    sa = rng.uniform(0.001, 2.0, size=(K // 128, M)).astype(np.float32)
    sb = (rng.uniform(0.001, 2.0, size=(N // 128, K // 128)) if recipe_b == "128x128"
          else rng.uniform(0.001, 2.0, size=(K // 128, N))).astype(np.float32)
    if recipe_b == "128x128":
        sb_fn = lambda j, k: sb[j // 128, k // 128]
    else:
        sb_fn = lambda j, k: sb[k // 128, j]
    exact = _exact_scaled(A, B, lambda i, k: sa[k // 128, i], sb_fn)
    un = gemm.scaled_mm_exact(A, B, sa, "1x128", sb, recipe_b)
    rb = gemm.scaled_mm(A, B, sa, "1x128", sb, recipe_b)
    for i in range(M):
        for j in range(N):
            ex = exact[i][j]
            assert abs(Fraction(float(un[i, j])) - ex) <= abs(ex) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)
            assert rb[i, j] == _frac_round_bf16(ex)


def test_rowwise_with_bias_matches_exact_rationals():
    rng = np.random.default_rng(3)
    M, N, K = 4, 6, 96
    A = rng.integers(0, 0x7F, size=(M, K)).astype(np.uint8)
    B = rng.integers(0x80, 0xFF, size=(N, K)).astype(np.uint8)
    sa = rng.uniform(0.01, 1.0, size=M).astype(np.float32)
    sb = rng.uniform(0.01, 1.0, size=N).astype(np.float32)
    bias = quant.bf16_to_f32(normal_bf16(streams(5, 1)[0], (N,), 10.0))
    exact = _exact_scaled(A, B, lambda i, k: sa[i], lambda j, k: sb[j], bias)
    rb = gemm.scaled_mm(A, B, sa, "rowwise", sb, "rowwise", bias=bias)
    for i in range(M):
        for j in range(N):
            assert rb[i, j] == _frac_round_bf16(exact[i][j])


def test_tensorwise_scale_one_identity():
    rng = np.random.default_rng(4)
    A = rng.integers(0, 0x7F, size=(20, 64)).astype(np.uint8)
    B = rng.integers(0, 0x7F, size=(30, 64)).astype(np.uint8)
    one = np.ones(1, np.float32)
    un = gemm.scaled_mm_exact(A, B, one, "tensorwise", one, "tensorwise")
    assert np.allclose(un, TABLE[A] @ TABLE[B].T, rtol=1e-14, atol=0)


def test_blockwise_scaled_sum_equals_dequantized_gemm():
    g = streams(6, 2)
    x = normal_bf16(g[0], (64, 512))
    w = normal_bf16(g[1], (256, 512), 0.02)
    qa, sa = quant.quantize_blockwise(x, 1, 128)         # sa [K/128, M]
    qb, sb = quant.quantize_blockwise(w, 128, 128)       # sb [N/128, K/128]
    acc = np.zeros((64, 256))
    for kb in range(4):
        blk = TABLE[qa[:, kb * 128:(kb + 1) * 128]] @ TABLE[qb[:, kb * 128:(kb + 1) * 128]].T
        acc += blk * sa[kb][:, None].astype(np.float64) * np.repeat(sb[:, kb].astype(np.float64), 128)[None, :]
    un = gemm.scaled_mm_exact(qa, qb, sa, "1x128", sb, "128x128")
    assert np.allclose(un, acc, rtol=1e-12, atol=1e-12 * np.abs(acc).max())


def test_grad_input_form_is_forward_on_transposed_weight():
    g = streams(7, 2)
    go = normal_bf16(g[0], (64, 256))                    # grad_output [M, N_out]
    w = normal_bf16(g[1], (256, 384), 0.02)              # weight [N_out, K_in]
    qg, sg = quant.quantize_blockwise(go, 1, 128)
    qw, sw = quant.quantize_blockwise(w, 128, 128)       # sw [N_out/128, K_in/128]
    gi = gemm.linear_grad_input(qg, sg, "1x128", qw, sw, "128x128")
    # transposing a 128x128-blocked weight transposes codes and the scale grid
    alt = gemm.scaled_mm(qg, np.ascontiguousarray(qw.T), sg, "1x128",
                         np.ascontiguousarray(sw.T), "128x128", "NK")
    assert np.array_equal(gi, alt)
    ref = quant.dequantize(qg, sg, 1, 128) @ quant.dequantize(qw, sw, 128, 128)
    assert np.array_equal(gi, gemm.round_bf16(ref))


def test_grad_weight_form_contracts_over_tokens():
    g = streams(8, 2)
    go = normal_bf16(g[0], (256, 64), 1e-3)              # [T, N_out]
    x = normal_bf16(g[1], (256, 96))                     # [T, K_in]
    qg, sg = quant.quantize_blockwise(go, 128, 1, transpose_out=True)   # [N_out, T], [T/128, N_out]
    qx, sx = quant.quantize_blockwise(x, 128, 1, transpose_out=True)    # [K_in, T],  [T/128, K_in]
    gw = gemm.linear_grad_weight(qg, sg, qx, sx)
    ref = quant.dequantize(qg.T, sg, 128, 1).T @ quant.dequantize(qx.T, sx, 128, 1)
    assert gw.shape == (64, 96)
    assert np.allclose(gw, gemm.round_bf16(ref), rtol=0, atol=0)


def test_grouped_reduces_to_rowwise():
    g = streams(9, 2)
    E, N, K = 5, 48, 128
    act = normal_bf16(g[0], (40, K))
    W = normal_bf16(g[1], (E, N, K), 0.02)
    qa, sa = quant.quantize_rowwise(act)
    qw, sw = quant.quantize_rowwise(W.reshape(E * N, K))
    qw, sw = qw.reshape(E, N, K), sw.reshape(E, N)
    offs = np.array([7, 7, 20, 33, 38], np.int32)        # group 1 empty, rows 38.. unowned
    out, written = gemm.grouped_mm(qa, qw, offs, sa, sw)
    assert written.sum() == 38 and not written[38:].any()
    start = 0
    for e in range(E):
        end = offs[e]
        if end > start:
            ref = gemm.scaled_mm(qa[start:end], qw[e], sa[start:end], "rowwise", sw[e], "rowwise")
            assert np.array_equal(out[start:end], ref)
        start = end
    one, _ = gemm.grouped_mm(qa, qw[:1], np.array([40], np.int32), sa, sw[:1])
    assert np.array_equal(one, gemm.scaled_mm(qa, qw[0], sa, "rowwise", sw[0], "rowwise"))


def test_grouped_per_expert_bias():
    """Bias [E, N]: with all-zero activation codes every owned row of expert e
    is exactly bf16(bias[e]) (the product vanishes, one rounding of the bias);
    with real codes each expert equals its rowwise GEMM with bias row e."""
    g = streams(10, 3)
    E, N, K = 4, 32, 128
    W = normal_bf16(g[1], (E, N, K), 0.02)
    qw, sw = quant.quantize_rowwise(W.reshape(E * N, K))
    qw, sw = qw.reshape(E, N, K), sw.reshape(E, N)
    bias = quant.bf16_to_f32(normal_bf16(g[2], (E, N), 0.5))     # bf16 values
    offs = np.array([3, 10, 10, 17], np.int32)
    zero = np.zeros((17, K), np.uint8)
    out, written = gemm.grouped_mm(zero, qw, offs, np.ones(17, np.float32), sw, bias=bias)
    assert written.all()
    rows_e = np.searchsorted(offs, np.arange(17), side="right")
    assert np.array_equal(out, bias[rows_e].astype(np.float64))
    act = normal_bf16(g[0], (17, K))
    qa, sa = quant.quantize_rowwise(act)
    out, _ = gemm.grouped_mm(qa, qw, offs, sa, sw, bias=bias)
    start = 0
    for e in range(E):
        end = offs[e]
        if end > start:
            ref = gemm.scaled_mm(qa[start:end], qw[e], sa[start:end], "rowwise", sw[e], "rowwise",
                                 bias=bias[e])
            assert np.array_equal(out[start:end], ref)
        start = end


def test_unsupported_pairs_raise():
    z = np.zeros((2, 128), np.uint8)
    with pytest.raises(NotImplementedError):
        gemm.scaled_mm(z, z, np.ones(2), "rowwise", np.ones(1), "tensorwise")


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(13)
    v = (rng.standard_normal(1 << 18) * np.exp2(rng.integers(-140, 120, 1 << 18))).astype(np.float32)
    ties = (np.arange(1, 4096, dtype=np.uint32) << 15 | 0x3F800000).view(np.float32)   # exact halfway cases
    v = np.concatenate([v, ties, -ties])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(gemm.round_bf16(v.astype(np.float64)), ref)


@pytest.mark.parametrize("recipe", ["tensorwise", "rowwise", "blockwise"])
def test_sqnr_floor(recipe):
    g = streams(10, 2)
    x = normal_bf16(g[0], (128, 1024))
    w = normal_bf16(g[1], (256, 1024), 0.02)
    if recipe == "tensorwise":
        qa, sa = quant.quantize_tensorwise(x); qb, sb = quant.quantize_tensorwise(w); ra, rb = "tensorwise", "tensorwise"
    elif recipe == "rowwise":
        qa, sa = quant.quantize_rowwise(x); qb, sb = quant.quantize_rowwise(w); ra, rb = "rowwise", "rowwise"
    else:
        qa, sa = quant.quantize_blockwise(x, 1, 128); qb, sb = quant.quantize_blockwise(w, 128, 128); ra, rb = "1x128", "128x128"
    out = gemm.scaled_mm(qa, qb, sa, ra, sb, rb)
    hp = quant.bf16_to_f32(x).astype(np.float64) @ quant.bf16_to_f32(w).astype(np.float64).T
    assert gemm.sqnr_db(hp, out) >= 20.0
    # weight SQNR floor of the MoE tests
    assert gemm.sqnr_db(quant.bf16_to_f32(w), quant.dequantize(qb, sb, *({"tensorwise": (256, 1024), "rowwise": (1, 1024), "blockwise": (128, 128)}[recipe]))) >= 25.0


def test_entries_evaluator_matches_full():
    g = streams(11, 2)
    x = normal_bf16(g[0], (64, 256))
    w = normal_bf16(g[1], (384, 256), 0.02)
    qa, sa = quant.quantize_blockwise(x, 1, 128)
    qb, sb = quant.quantize_blockwise(np.ascontiguousarray(w.reshape(384, 256).T), 128, 128)   # stored [K, N]
    full = gemm.scaled_mm(qa, qb, sa, "1x128", sb, "128x128", layout="KN")
    rng = np.random.default_rng(0)
    r = rng.integers(0, 64, 500); c = rng.integers(0, 384, 500)
    ent = gemm.scaled_mm_entries(qa, qb, sa, "1x128", sb, "128x128", r, c, layout="KN")
    assert np.array_equal(ent, full[r, c])


def test_parity_bars_accept_a_correct_bf16_kernel_and_reject_plausible_bugs():
    """A result computed exactly, perturbed like fp32 accumulation and rounded
    once to bf16 meets both bars; a dropped K block, a wrong scale and a
    transposed operand do not."""
    g = streams(12, 2)
    x = normal_bf16(g[0], (256, 1024))
    w = normal_bf16(g[1], (384, 1024), 0.02)
    qa, sa = quant.quantize_blockwise(x, 1, 128)
    qb, sb = quant.quantize_blockwise(w, 128, 128)
    exact = gemm.scaled_mm_exact(qa, qb, sa, "1x128", sb, "128x128")
    rng = np.random.default_rng(0)
    fp32ish = exact * (1 + rng.standard_normal(exact.shape) * 2e-6)
    good = gemm.round_bf16(fp32ish)
    rel_f, rel_m = gemm.parity(good, exact)
    assert rel_f <= 1e-3 and rel_m <= 4e-3
    # against the once-rounded oracle a single last-place flip can exceed 4e-3
    flips = (good != gemm.round_bf16(exact))
    assert flips.any()
    assert np.max(np.abs(good - gemm.round_bf16(exact)) / np.abs(exact).max()) <= 2.0 ** -7
    sa_bad = sa.copy(); sa_bad[3] *= 1.01
    dropped = gemm.scaled_mm(qa, qb, sa, "1x128", sb * np.array([1, 1, 1, 1, 1, 1, 1, 0], np.float32)[None, :], "128x128")
    wrong_scale = gemm.scaled_mm(qa, qb, sa_bad, "1x128", sb, "128x128")
    transposed_blk = gemm.scaled_mm(qa, qb, sa, "1x128", np.ascontiguousarray(sb[::-1]), "128x128")
    for bad in (dropped, wrong_scale, transposed_blk):
        rel_f, rel_m = gemm.parity(bad, exact)
        assert rel_f > 1e-3 or rel_m > 4e-3
