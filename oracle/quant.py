"""Dynamic FP8 quantization for the oracle.  Test infrastructure only.

Inputs are bfloat16 matrices given as numpy ``uint16`` bit patterns (row-major
``[rows, cols]``); widening bf16 to float32 is exact.

What is computed, per scaling group G (the whole tensor, one row, a 1x128 run
along a row, a 128x128 block, or a 128x1 run down a column):

  amax_G  = max over G of |x|                            (exact in float32)
  s_G     = fl32(amax_G / 448)
            rowwise:  fl32( fl32(amax_G / 448) + fl32(eps) ), eps = 1e-12
            a group whose scale comes out as 0 (an all-zero group) gets 1.0
  code    = enc( fl32(x / s_G) )      IEEE float32 division, then the E4M3
                                      round-to-nearest-even saturating encode
  value   = dec(code) * s_G           (the scale is a dequantization multiplier)

Sources: per-token (per-row) scale from the row's maximum absolute value,
input divided by the scale plus a small epsilon before the FP8 cast
(DiffSynth-Engine PR #160, "per-token scaling for fp8 linear", "Highlights");
the scale handed to the GEMM is the inverse of the quantization factor, i.e.
a dequantization multiplier (ColossalAI PR #6419, "Forward pass"); tensorwise,
rowwise, 1x128 and 128x128 groupings (pytorch PR #164141, "Add _scaled_mm_v2
API", recipe names in the dispatch review); 1x128 x 128x1 for the weight
gradient (pytorch/ao PR #2784, "improve fp8 blockwise gemm perf", second
table).  The 448 divisor, the 1e-12 value and "divide, then round" are the
readings the method fixes where the pages only say "max abs value" and "small
epsilon".

Scale layouts (float32, C order):
  tensorwise          [1]
  rowwise             [rows]
  block (1, 128)      [cols/128, rows]       k-block major
  block (128, 128)    [rows/128, cols/128]
  block (128, 1)      [rows/128, cols]       (codes optionally written
                                              transposed as [cols, rows])

Pins: ``tests/test_oracle_quant.py`` (power-of-two round trips, the
"amax element encodes to +-448" invariant, designed-amax layout checks, the
epsilon closed form, zero groups).
"""

import numpy as np

from . import e4m3

FP8_MAX = np.float32(448.0)
ROWWISE_EPS = np.float32(1e-12)


def bf16_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def scale_from_amax(amax, eps=None):
    """s = fl32(amax/448) [+ eps, rowwise]; a zero scale becomes 1.0."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / FP8_MAX).astype(np.float32)
    if eps is not None:
        s = (s + np.float32(eps)).astype(np.float32)
    return np.where(s == 0, np.float32(1.0), s).astype(np.float32)


def cast(x32, s32):
    """code = enc(fl32(x / s)) elementwise (s broadcast to x)."""
    y = (np.asarray(x32, np.float32) / np.asarray(s32, np.float32)).astype(np.float32)
    return e4m3.encode(y)


def quantize_tensorwise(x_bits):
    x = bf16_to_f32(x_bits)
    amax = np.max(np.abs(x)) if x.size else np.float32(0)
    s = scale_from_amax(amax).reshape(1)
    return cast(x, s[0]), s


def quantize_rowwise(x_bits, eps=ROWWISE_EPS):
    x = bf16_to_f32(x_bits)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = scale_from_amax(amax, eps)
    return cast(x, s[:, None]), s


def quantize_blockwise(x_bits, block_rows, block_cols, transpose_out=False):
    """Blockwise quantization with groups of block_rows x block_cols; the block
    shapes of the method are (1,128), (128,128) and (128,1)."""
    x = bf16_to_f32(x_bits)
    rows, cols = x.shape
    assert rows % block_rows == 0 and cols % block_cols == 0
    gr, gc = rows // block_rows, cols // block_cols
    blocks = np.abs(x).reshape(gr, block_rows, gc, block_cols)
    amax = blocks.max(axis=(1, 3))                       # [gr, gc]
    s_grid = scale_from_amax(amax)                       # [gr, gc]
    s_elem = np.repeat(np.repeat(s_grid, block_rows, 0), block_cols, 1)
    q = cast(x, s_elem)
    if (block_rows, block_cols) == (1, 128):
        scale = np.ascontiguousarray(s_grid.T)          # [cols/128, rows]
    elif (block_rows, block_cols) == (128, 1):
        scale = s_grid                                   # [rows/128, cols]
    else:
        scale = s_grid                                   # [rows/128, cols/128]
    if transpose_out:
        q = np.ascontiguousarray(q.T)
    return q, np.ascontiguousarray(scale, dtype=np.float32)


def dequantize(q, scale, block_rows, block_cols):
    """float64 values dec(q) * s for a [rows, cols] code matrix whose scale
    array has the layout of ``quantize_blockwise`` / ``quantize_rowwise`` /
    ``quantize_tensorwise``.  block_rows/block_cols: (rows, cols) for the whole
    tensor, (1, cols) for rowwise."""
    q = np.asarray(q, np.uint8)
    rows, cols = q.shape
    vals = e4m3.decode(q)
    scale = np.asarray(scale, np.float64)
    if block_rows == rows and block_cols == cols:        # tensorwise
        return vals * scale.reshape(-1)[0]
    if block_rows == 1 and block_cols == cols:           # rowwise
        return vals * scale.reshape(rows, 1)
    if (block_rows, block_cols) == (1, 128):
        grid = scale.T                                   # [rows, cols/128]
    else:
        grid = scale
    s_elem = np.repeat(np.repeat(grid, block_rows, 0), block_cols, 1)
    return vals * s_elem
