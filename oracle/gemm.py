"""Scaled FP8 GEMM for the oracle.  Test infrastructure only.

The method's GEMM is

    out[i, j] = sum_k  dec(A[i,k]) * sA(i,k)  *  dec(B[j,k]) * sB(j,k)  (+ bias[j])

where sA(i,k) / sB(j,k) is the scale of the quantization group that holds the
element.  This is exactly the "dequantize both operands, then one ordinary
matmul" formulation that ColossalAI PR #6419 ("Fix: Handle LowLevelZeroPlugin
with use_fp8=True", "Forward pass" and "Backward pass") shows to be equivalent
to the fused scaled-mm call; the oracle evaluates it that way in float64 and
rounds ONCE to the output dtype (bf16 round-to-nearest-even, or fp32).  Bias
is added in float64 before that single rounding (the scaled-mm call takes the
bias as an argument rather than adding it after a rounded matmul).

Operand conventions (all row-major numpy arrays):
  A        uint8 [M, K]                    K contiguous
  B        uint8 [N, K] (layout "NK")  or  [K, N] (layout "KN", N contiguous)
  recipes  A: "tensorwise" [1] | "rowwise" [M] | "1x128" [K/128, M]
           B: "tensorwise" [1] | "rowwise" [N] | "128x128" ([N/128, K/128] for
              NK, [K/128, N/128] for KN: the quantizer's grid of B as stored)
              | "128x1" [K/128, N]  (128 along the contraction x 1 along N,
              named in the [K, N] orientation of the weight-gradient table of
              pytorch/ao PR #2784, "improve fp8 blockwise gemm perf")
           A and B: "mxfp8" uint8 E8M0 bytes [M, K/32] / [N, K/32] (B as [N, K];
              see ``mx``)
Accepted pairs (pytorch PR #164141, "Add _scaled_mm_v2 API": one explicit
recipe per operand, checked against a table):
  (tensorwise, tensorwise) (rowwise, rowwise) (1x128, 128x128) (1x128, 128x1)
  (mxfp8, mxfp8)

Grouped (MoE) GEMM (pytorch/ao PR #4390, "Add _grouped_mm dispatch handler to
Float8Tensor", "Design" and review): expert e owns activation rows
[offs[e-1], offs[e]) (offs[-1] = 0), weights are [E, N, K] and are used in the
form grouped_mm(act, weight.transpose(-2, -1)); the pages give rowwise scales.
Readings beyond the pages: the blockwise recipe applied per expert in the same
grouped form (1x128 activations, 128x128 expert weights), the input gradient
as the grouped GEMM reading each expert's weight as [K, N], and the weight
gradient per expert over the expert's own tokens (``grouped_grad_weight``).

Linear call forms (ColossalAI PR #6419 "Forward pass" / "Backward pass";
pytorch/ao PR #2784 tables):
  forward      out         = input @ weight.t()
  grad_input   grad_input  = grad_output @ weight
  grad_weight  grad_weight = grad_output.t() @ input

Pins: ``tests/test_oracle_gemm.py`` (exact Fraction GEMMs on small-integer and
dyadic inputs, tensorwise scale-1 identity, the per-128-block scaled-sum
invariant, transposition identities, grouped reductions, SQNR sanity floor).
"""

import numpy as np

from . import e4m3, mx, quant

PAIRS = {("tensorwise", "tensorwise"), ("rowwise", "rowwise"),
         ("1x128", "128x128"), ("1x128", "128x1"), ("mxfp8", "mxfp8")}


def _scale_grid_A(scale, recipe, M, K):
    s = np.asarray(scale, np.float64)
    if recipe == "tensorwise":
        return np.full((M, K), s.reshape(-1)[0])
    if recipe == "rowwise":
        return np.repeat(s.reshape(M, 1), K, 1)
    if recipe == "1x128":
        return np.repeat(s.reshape(K // 128, M).T, 128, 1)
    if recipe == "mxfp8":
        return np.repeat(mx.scale_values(scale).reshape(M, K // mx.MX_BLOCK), mx.MX_BLOCK, 1)
    raise ValueError(recipe)


def _scale_grid_B_nk(scale, recipe, N, K, layout):
    """Per-element scale of B in its logical [N, K] orientation."""
    s = np.asarray(scale, np.float64)
    if recipe == "tensorwise":
        return np.full((N, K), s.reshape(-1)[0])
    if recipe == "rowwise":
        return np.repeat(s.reshape(N, 1), K, 1)
    if recipe == "128x128":
        if layout == "NK":
            g = s.reshape(N // 128, K // 128)
        else:                       # stored [K, N]: grid [K/128, N/128]
            g = s.reshape(K // 128, N // 128).T
        return np.repeat(np.repeat(g, 128, 0), 128, 1)
    if recipe == "128x1":
        return np.repeat(s.reshape(K // 128, N).T, 128, 1)
    if recipe == "mxfp8":
        if layout != "NK":
            raise NotImplementedError("mxfp8 B is read as [N, K]")
        return np.repeat(mx.scale_values(scale).reshape(N, K // mx.MX_BLOCK), mx.MX_BLOCK, 1)
    raise ValueError(recipe)


def dequant_A(A, scale, recipe):
    A = np.asarray(A, np.uint8)
    M, K = A.shape
    return e4m3.decode(A) * _scale_grid_A(scale, recipe, M, K)


def dequant_B(B, scale, recipe, layout="NK"):
    """Dequantized B in the logical [N, K] orientation (float64)."""
    B = np.asarray(B, np.uint8)
    Bnk = B if layout == "NK" else B.T
    N, K = Bnk.shape
    return e4m3.decode(Bnk) * _scale_grid_B_nk(scale, recipe, N, K, layout)


def round_bf16(x):
    """Round float64 values once to bfloat16 (round to nearest, ties to even);
    returns the rounded values as float64."""
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)                      # x = m * 2^e with 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)             # exponent of one bf16 ulp at x
    r = np.ldexp(np.round(np.ldexp(x, -q)), q)   # np.round: ties to even
    return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)


def round_out(x, out_dtype):
    """Round once to out_dtype; out_dtype None keeps the float64 value."""
    if out_dtype is None:
        return np.asarray(x, np.float64)
    if out_dtype == "bf16":
        return round_bf16(x)
    if out_dtype == "fp32":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(out_dtype)


def scaled_mm_exact(A, B, scale_a, recipe_a, scale_b, recipe_b, layout="NK",
                    bias=None):
    """Unrounded float64 result of the scaled GEMM."""
    if (recipe_a, recipe_b) not in PAIRS:
        raise NotImplementedError((recipe_a, recipe_b))
    a = dequant_A(A, scale_a, recipe_a)
    b = dequant_B(B, scale_b, recipe_b, layout)
    out = a @ b.T
    if bias is not None:
        out = out + np.asarray(bias, np.float64)[None, :]
    return out


def scaled_mm(A, B, scale_a, recipe_a, scale_b, recipe_b, layout="NK",
              bias=None, out_dtype="bf16"):
    """Scaled GEMM rounded once to out_dtype (float64 array of the values)."""
    return round_out(scaled_mm_exact(A, B, scale_a, recipe_a, scale_b, recipe_b,
                                     layout, bias), out_dtype)


def scaled_mm_entries(A, B, scale_a, recipe_a, scale_b, recipe_b, rows, cols,
                      layout="NK", bias=None, out_dtype="bf16"):
    """The same definition evaluated only at output entries (rows[t], cols[t]);
    used where the full product is too large for the CPU."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    A = np.asarray(A, np.uint8)
    M, K = A.shape
    urows, rinv = np.unique(rows, return_inverse=True)
    ucols, cinv = np.unique(cols, return_inverse=True)
    a = e4m3.decode(A[urows]) * _scale_grid_A(scale_a, recipe_a, M, K)[urows]
    Bnk = np.asarray(B, np.uint8) if layout == "NK" else np.asarray(B, np.uint8).T
    N = Bnk.shape[0]
    b = (e4m3.decode(Bnk[ucols])
         * _scale_grid_B_nk(scale_b, recipe_b, N, K, layout)[ucols])
    vals = np.einsum("tk,tk->t", a[rinv], b[cinv])
    if bias is not None:
        vals = vals + np.asarray(bias, np.float64)[cols]
    return round_out(vals, out_dtype)


GROUPED_PAIRS = {("rowwise", "rowwise"), ("1x128", "128x128")}


def grouped_mm(A, W, offs, scale_a, scale_b, bias=None, out_dtype="bf16",
               recipe_a="rowwise", recipe_b="rowwise", layout="NK"):
    """MoE grouped GEMM: rows [offs[e-1], offs[e]) of A times expert e's B.
    A [M_total, K]; W [E, N, K] (layout "NK", the forward's
    grouped_mm(act, weight.transpose(-2, -1))) or [E, K, N] (layout "KN", e.g.
    the stored [E, N_out, K_in] weights read by the input gradient, which
    contracts over N_out); offs int32 [E] cumulative END offsets.
    Recipes: rowwise x rowwise (scale_a [M_total], scale_b [E, N]) or
    1x128 x 128x128 (scale_a [K/128, M_total], scale_b [E] x the 128x128 grid
    of expert e's B as stored).  bias None, values [N] (every expert) or
    [E, N] (row e for expert e).
    Returns (out [M_total, N] float64 with NaN in rows no group owns,
    rows_written bool [M_total])."""
    if (recipe_a, recipe_b) not in GROUPED_PAIRS:
        raise NotImplementedError((recipe_a, recipe_b))
    A = np.asarray(A, np.uint8)
    W = np.asarray(W, np.uint8)
    M_total, K = A.shape
    E = W.shape[0]
    N = W.shape[1] if layout == "NK" else W.shape[2]
    scale_a = np.asarray(scale_a)
    out = np.full((M_total, N), np.nan)
    written = np.zeros(M_total, bool)
    start = 0
    for e in range(E):
        end = int(offs[e])
        if end > start:
            b = None if bias is None else (np.asarray(bias)[e] if np.ndim(bias) == 2 else bias)
            sa = scale_a[start:end] if recipe_a == "rowwise" else scale_a[:, start:end]
            out[start:end] = scaled_mm(A[start:end], W[e], sa, recipe_a,
                                       np.asarray(scale_b)[e], recipe_b, layout,
                                       b, out_dtype)
            written[start:end] = True
        start = max(start, end)
    return out, written


def grouped_grad_weight(gt_q, gt_scale, xt_q, xt_scale, offs, out_dtype="bf16"):
    """Per-expert weight gradient grad_weight[e] = grad_output[rows_e].T @
    input[rows_e] (the dense weight-gradient call form applied to expert e's
    tokens), both operands in the grouped 128x1 layout of
    ``quant.quantize_grouped_128x1``: gt_q [N_out, P] with gt_scale [NB, N_out],
    xt_q [K_in, P] with xt_scale [NB, K_in].  The sum runs over the expert's
    own tokens only; an expert without tokens gets zeros.
    Returns [E, N_out, K_in] float64, rounded once to out_dtype."""
    gt_q = np.asarray(gt_q, np.uint8)
    xt_q = np.asarray(xt_q, np.uint8)
    gt_scale = np.asarray(gt_scale, np.float64)
    xt_scale = np.asarray(xt_scale, np.float64)
    start, end, first, _ = quant.grouped_blocks(offs)
    E = end.size
    N_out, K_in = gt_q.shape[0], xt_q.shape[0]
    out = np.zeros((E, N_out, K_in))
    for e in range(E):
        m = int(end[e] - start[e])
        if m == 0:
            continue
        j = np.arange(m)
        cols = 128 * int(first[e]) + j                   # the expert's tokens
        blocks = int(first[e]) + j // 128                # their scaling runs
        a = e4m3.decode(gt_q[:, cols]) * gt_scale[blocks].T     # [N_out, m]
        b = e4m3.decode(xt_q[:, cols]) * xt_scale[blocks].T     # [K_in, m]
        out[e] = a @ b.T
    return round_out(out, out_dtype)


def linear_forward(x_q, x_scale, x_recipe, w_q, w_scale, w_recipe, bias=None,
                   out_dtype="bf16"):
    """out = input @ weight.t(): A = input [M, K], B = weight [N, K] (NK)."""
    return scaled_mm(x_q, w_q, x_scale, x_recipe, w_scale, w_recipe, "NK",
                     bias, out_dtype)


def linear_grad_input(g_q, g_scale, g_recipe, w_q, w_scale, w_recipe,
                      out_dtype="bf16"):
    """grad_input = grad_output @ weight: A = grad_output [M, N_out],
    B = weight [N_out, K_in] read as [K, N] (KN)."""
    return scaled_mm(g_q, w_q, g_scale, g_recipe, w_scale, w_recipe, "KN",
                     None, out_dtype)


def linear_grad_weight(gt_q, gt_scale, xt_q, xt_scale, out_dtype="bf16"):
    """grad_weight = grad_output.t() @ input, both operands quantized in runs
    of 128 tokens and stored transposed: A = grad_output^T [N_out, T] (1x128
    along T, scale [T/128, N_out]), B = input^T [K_in, T] (128x1 in the [K, N]
    orientation, scale [T/128, K_in]), layout NK."""
    return scaled_mm(gt_q, xt_q, gt_scale, "1x128", xt_scale, "128x1", "NK",
                     None, out_dtype)


def parity(out, ref_exact, out_dtype="bf16"):
    """The GEMM parity figures of a result against the float64 oracle:
      rel_fro = ||out - R|| / ||R||, R = ref_exact rounded once to out_dtype
      rel_max = max|out - ref_exact| / max|ref_exact|
    The Frobenius figure uses the rounded reference because bf16 rounding
    alone is about 1.6e-3 relative in Frobenius norm; the elementwise figure
    uses the unrounded reference because one correct bf16 rounding moves an
    element by at most 2^-8 of its own magnitude, while against the rounded
    reference a single last-place flip can reach 2^-7."""
    out = np.asarray(out, np.float64)
    ref_exact = np.asarray(ref_exact, np.float64)
    rel_f, _ = compare(out, round_out(ref_exact, out_dtype))
    _, rel_m = compare(out, ref_exact)
    return rel_f, rel_m


def compare(out, ref):
    """(relative Frobenius error, max |err| / max |ref|) of out against ref."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    err = out - ref
    nref = np.linalg.norm(ref)
    mref = np.max(np.abs(ref)) if ref.size else 0.0
    rel_f = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    rel_m = np.max(np.abs(err)) / mref if mref > 0 else (np.max(np.abs(err)) if err.size else 0.0)
    return float(rel_f), float(rel_m)


def sqnr_db(ref, approx):
    ref = np.asarray(ref, np.float64)
    noise = ref - np.asarray(approx, np.float64)
    return 10.0 * np.log10(np.sum(ref * ref) / np.sum(noise * noise))
