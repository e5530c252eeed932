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
  grouped (128, 1)    [runs, cols]           runs of 128 tokens restarted at
                                              each expert (see
                                              ``quantize_grouped_128x1``)

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


# ---------------------------------------------------------------------------
# Grouped (MoE) weight-gradient operands: 128x1 runs that restart at each
# expert's first token.
#
# The pages give the grouped GEMM only for the forward, rowwise, with expert e
# owning activation rows [offs[e-1], offs[e]) (pytorch/ao PR #4390, "Add
# _grouped_mm dispatch handler to Float8Tensor", "Design"), and the 128x1
# token runs only for the dense weight gradient (pytorch/ao PR #2784, "improve
# fp8 blockwise gemm perf", second table).  Reading for the grouped weight
# gradient: each expert's tokens are cut into runs of 128 from the expert's
# first token (the last run may be shorter), so no scaling group mixes two
# experts; each run x column is one group.  The codes are stored transposed,
# each expert starting at a multiple of 128 columns of a padded token axis:
# run j of expert e is block first_block[e] + j, first_block being the
# exclusive prefix sum of the experts' run counts ceil(m_e / 128); columns of
# a short run past the expert's last token hold zero codes.
# ---------------------------------------------------------------------------

def group_ranges(offs):
    """Row range [start, end) of every expert: [offs[e-1], offs[e]) with
    offs[-1] = 0.  Offsets must be non-decreasing and non-negative."""
    offs = np.asarray(offs, np.int64)
    assert offs.ndim == 1 and (offs >= 0).all() and (np.diff(offs) >= 0).all()
    start = np.concatenate([[0], offs[:-1]]).astype(np.int64)
    return start, offs.copy()


def grouped_blocks(offs):
    """(start, end, first_block, n_blocks) per expert for the padded token
    layout: n_blocks = ceil((end - start) / 128), first_block its exclusive
    prefix sum."""
    start, end = group_ranges(offs)
    n_blocks = (end - start + 127) // 128
    first = np.concatenate([[0], np.cumsum(n_blocks)[:-1]]).astype(np.int64)
    return start, end, first, n_blocks


def quantize_grouped_128x1(x_bits, offs):
    """x bf16 bits [T, C], offs int [E] (end offsets, offs[E-1] <= T).
    Returns (qt uint8 [C, 128 * NB], scale float32 [NB, C], first_block [E])
    with NB the total run count; rows at or past offs[E-1] belong to no run."""
    x = bf16_to_f32(x_bits)
    T, C = x.shape
    start, end, first, n_blocks = grouped_blocks(offs)
    assert end.size == 0 or end[-1] <= T
    NB = int(n_blocks.sum())
    qt = np.zeros((C, 128 * NB), np.uint8)
    scale = np.zeros((NB, C), np.float32)
    for e in range(end.size):
        for j in range(int(n_blocks[e])):
            r0 = int(start[e]) + 128 * j
            r1 = min(r0 + 128, int(end[e]))
            run = x[r0:r1]                                   # [rows, C]
            s = scale_from_amax(np.max(np.abs(run), axis=0))  # [C]
            b = int(first[e]) + j
            scale[b] = s
            qt[:, 128 * b:128 * b + (r1 - r0)] = cast(run, s[None, :]).T
    return qt, scale, first
