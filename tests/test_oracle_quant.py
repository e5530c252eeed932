"""Pins for the oracle's dynamic quantizers (CPU only).

Pinned by closed forms rather than by retyping the formula:
  * power-of-two round trips: a group built from E4M3 values times 2^k whose
    largest element is 448 * 2^k has scale exactly 2^k and quantizes back to
    the very codes it was built from (pins the divisor, the direction of the
    division, the encoder and every scale layout, since k differs per group);
  * the amax element of every non-zero group encodes to +-448;
  * all-zero groups (scale 1.0, codes +-0 with the sign kept);
  * the rowwise epsilon only shows when amax < 448 * 2^-15.
"""

import numpy as np
import pytest
import torch

from oracle import e4m3, quant
from workloads import f32_to_bf16_bits

TABLE = e4m3.decode_table()
FINITE_POS = np.array([c for c in range(0x7F)], np.uint8)          # 0x00..0x7E


def _codes(rng, shape):
    mag = rng.choice(FINITE_POS, size=shape)
    sgn = (rng.random(shape) < 0.5).astype(np.uint8) << 7
    return (mag | sgn).astype(np.uint8)


def _build(codes, k_grid, block_rows, block_cols):
    """bf16 matrix = dec(codes) * 2^k(group); every group gets one 0x7E."""
    rows, cols = codes.shape
    codes = codes.copy()
    gr, gc = rows // block_rows, cols // block_cols
    for a in range(gr):
        for b in range(gc):
            codes[a * block_rows, b * block_cols] = 0x7E
    k_elem = np.repeat(np.repeat(k_grid, block_rows, 0), block_cols, 1)
    vals = TABLE[codes] * np.exp2(k_elem)
    bits = f32_to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(quant.bf16_to_f32(bits).astype(np.float64), vals)   # exact in bf16
    return codes, bits


@pytest.mark.parametrize("rows,cols,br,bc", [
    (256, 384, 1, 128), (256, 384, 128, 128), (384, 256, 128, 1)])
def test_blockwise_power_of_two_round_trip(rows, cols, br, bc):
    rng = np.random.default_rng(7)
    gr, gc = rows // br, cols // bc
    k_grid = rng.integers(-20, 20, size=(gr, gc))
    codes, bits = _build(_codes(rng, (rows, cols)), k_grid, br, bc)
    q, s = quant.quantize_blockwise(bits, br, bc)
    assert np.array_equal(q, codes)
    exp = np.exp2(k_grid).astype(np.float32)
    if (br, bc) == (1, 128):
        exp = exp.T
    assert s.dtype == np.float32 and np.array_equal(s, exp)
    # dequantize inverts exactly
    assert np.array_equal(quant.dequantize(q, s, br, bc), quant.bf16_to_f32(bits).astype(np.float64))


def test_blockwise_128x1_transposed_output():
    rng = np.random.default_rng(8)
    k_grid = rng.integers(-10, 10, size=(3, 256))
    codes, bits = _build(_codes(rng, (384, 256)), k_grid, 128, 1)
    q, s = quant.quantize_blockwise(bits, 128, 1, transpose_out=True)
    assert q.shape == (256, 384) and np.array_equal(q, codes.T)
    assert np.array_equal(s, np.exp2(k_grid).astype(np.float32))


def test_rowwise_power_of_two_round_trip():
    rng = np.random.default_rng(9)
    k_grid = rng.integers(-15, 20, size=(64, 1))        # eps invisible for k >= -15
    codes, bits = _build(_codes(rng, (64, 300)), k_grid, 1, 300)
    q, s = quant.quantize_rowwise(bits)
    assert np.array_equal(q, codes)
    assert np.array_equal(s, np.exp2(k_grid[:, 0]).astype(np.float32))


def test_tensorwise_power_of_two_round_trip():
    rng = np.random.default_rng(10)
    codes, bits = _build(_codes(rng, (96, 160)), np.array([[-3]]), 96, 160)
    q, s = quant.quantize_tensorwise(bits)
    assert np.array_equal(q, codes) and s.shape == (1,) and s[0] == np.float32(0.125)


@pytest.mark.parametrize("kind", ["tensor", "row", "1x128", "128x128", "128x1"])
def test_amax_element_encodes_to_448(kind):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((256, 512)).astype(np.float32) * np.exp2(rng.integers(-30, 30, size=(256, 1)))
    bits = f32_to_bf16_bits(x.astype(np.float32))
    xf = np.abs(quant.bf16_to_f32(bits))
    if kind == "tensor":
        q, _ = quant.quantize_tensorwise(bits); br, bc = 256, 512
    elif kind == "row":
        q, _ = quant.quantize_rowwise(bits); br, bc = 1, 512
    else:
        br, bc = {"1x128": (1, 128), "128x128": (128, 128), "128x1": (128, 1)}[kind]
        q, _ = quant.quantize_blockwise(bits, br, bc)
    gr, gc = 256 // br, 512 // bc
    qb = (q & 0x7F).reshape(gr, br, gc, bc)
    xb = xf.reshape(gr, br, gc, bc)
    amax = xb.max(axis=(1, 3))
    at_max = np.where(xb == amax[:, None, :, None], qb, 0).max(axis=(1, 3))
    if kind == "row":       # the epsilon shifts the scale of rows below 448*2^-15
        big = amax >= np.float32(448.0 * 2.0 ** -15)
        assert big.sum() > 100 and (~big).sum() > 10
        # the amax element leaves code 448 once amax/s < 432 (the midpoint
        # below 448), i.e. once amax < about 28 * 448 * eps = 1.25e-8
        tiny = amax < np.float32(1e-8)
        assert np.all(at_max[big] == 0x7E) and tiny.sum() > 10 and np.all(at_max[tiny] < 0x7E)
    else:
        assert np.all(at_max == 0x7E)
    assert np.all(qb <= 0x7E)


def test_zero_groups_get_scale_one_and_keep_sign():
    x = np.zeros((128, 256), np.float32)
    x[:, 128:] = -0.0
    x[5, 200] = 3.0
    bits = f32_to_bf16_bits(x)
    q, s = quant.quantize_blockwise(bits, 1, 128)
    assert s[0].tolist() == [1.0] * 128                  # k-block 0 all zero
    assert s[1, 5] == np.float32(3.0) / np.float32(448.0)
    assert np.all(q[:, :128] == 0x00)
    assert np.all(np.delete(q[:, 128:], 5, axis=0) == 0x80)
    q, s = quant.quantize_tensorwise(f32_to_bf16_bits(np.zeros((4, 8), np.float32)))
    assert s[0] == 1.0 and np.all(q == 0)


def test_rowwise_epsilon_only_matters_for_tiny_rows():
    rows = np.array([0.0, 448.0 * 2.0 ** -15, 448.0 * 2.0 ** -16, 1e-30, 448.0], np.float32)
    x = np.zeros((5, 128), np.float32)
    x[:, 3] = rows
    bits = f32_to_bf16_bits(x)
    _, s = quant.quantize_rowwise(bits)
    _, s_noeps = quant.quantize_rowwise(bits, eps=0.0)
    # zero row: s = fl32(1e-12); rows with amax >= 448*2^-15: epsilon invisible
    assert s[0] == np.float32(1e-12) and s_noeps[0] == 1.0
    assert s[1] == s_noeps[1] == np.float32(2.0 ** -15)
    assert s[4] == 1.0
    # below the threshold the epsilon shifts the scale upward
    assert s[2] > s_noeps[2] and s[3] > s_noeps[3]


def test_quantizer_agrees_with_torch_cast_on_random_rows():
    """Cross-check against torch's CPU fp32 division and float8_e4m3fn cast."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((64, 1024)) * 3).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    q, s = quant.quantize_rowwise(bits)
    xt = torch.from_numpy(quant.bf16_to_f32(bits).copy())
    st = xt.abs().amax(dim=1, keepdim=True) / 448.0 + torch.tensor(1e-12, dtype=torch.float32)
    qt = (xt / st).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s, st[:, 0].numpy())
    assert np.array_equal(q, qt)
