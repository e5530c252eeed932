"""MXFP8 quantization for the oracle.  Test infrastructure only.

pytorch PR #164141 ("Add _scaled_mm_v2 API") names "mxfp8" as a recipe of the
scaled matrix multiply (the dispatch table of its review, where the recipe
string stands for both operands) but does not spell the format out.  The
reading taken is the OCP Microscaling (MX) format, version 1.0, with FP8 E4M3
elements: every run of 32 consecutive elements along a row (the contraction
dimension of a GEMM operand) shares one power-of-two scale stored as an E8M0
byte (the exponent plus 127), and

  amax  = max over the block of |x|                  (exact in float32)
  E     = floor(log2(amax)) - 8                       (8: exponent of E4M3's
                                                       largest normal, 448)
          clamped to [-127, 127]; an all-zero block takes E = -127
  code  = enc(x / 2^E)                                (x / 2^E is exact; enc
                                                       is the E4M3 encoder:
                                                       nearest even, saturating
                                                       to +-448)
  value = dec(code) * 2^E

so the block's largest element lands in [256, 512) before the cast (values
from 448 up saturate).  Scale layout: uint8 [rows, cols / 32], row-major.

Pins: ``tests/test_oracle_mx.py``.
"""

import numpy as np

from . import e4m3
from .quant import bf16_to_f32

MX_BLOCK = 32
E4M3_EMAX = 8
E8M0_BIAS = 127


def shared_exponent(amax):
    """E = floor(log2(amax)) - 8, clamped to [-127, 127]; 0 -> -127."""
    amax = np.asarray(amax, np.float64)
    _, ex = np.frexp(amax)                  # amax = m * 2^ex, 0.5 <= m < 1
    e = ex.astype(np.int64) - 1 - E4M3_EMAX  # floor(log2(amax)) = ex - 1
    e = np.where(amax > 0, e, -E8M0_BIAS)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS)


def quantize_mx(x_bits):
    """bf16 bits [rows, cols] (cols % 32 == 0) -> (codes uint8 [rows, cols],
    scale bytes uint8 [rows, cols / 32])."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    rows, cols = x.shape
    assert cols % MX_BLOCK == 0
    blocks = x.reshape(rows, cols // MX_BLOCK, MX_BLOCK)
    e = shared_exponent(np.abs(blocks).max(axis=2))              # [rows, cols/32]
    y = blocks / np.exp2(e)[:, :, None].astype(np.float64)       # exact
    codes = e4m3.encode(y.astype(np.float32)).reshape(rows, cols)
    return codes, (e + E8M0_BIAS).astype(np.uint8)


def scale_values(scale_bytes):
    """2^(byte - 127) as float64."""
    return np.exp2(np.asarray(scale_bytes, np.float64) - E8M0_BIAS)


def dequantize_mx(q, scale_bytes):
    """float64 dec(q) * 2^E per 32-element block."""
    q = np.asarray(q, np.uint8)
    return e4m3.decode(q) * np.repeat(scale_values(scale_bytes), MX_BLOCK, axis=1)
