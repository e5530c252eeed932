"""FP8 scaled matrix multiply for AMD MI355X (gfx950).

Python binding over the C ABI of ``libfp8mm.so`` (include/fp8mm.h).  The
functions carry the C names; they only check and marshal arguments, allocate
outputs with torch and pass device pointers plus the current HIP stream.
Every step of the computation runs in the library's HIP kernels.

Recipes are named "tensorwise", "rowwise", "1x128", "128x128" and "128x1";
scales are always returned as 2-D float32 tensors:
  tensorwise [1, 1]     rowwise [rows, 1]     1x128 [cols/128, rows]
  128x128 [rows/128, cols/128]                128x1 [rows/128, cols]
Errors map to ValueError (bad arguments), NotImplementedError (valid but not
supported) and RuntimeError (HIP failures).
"""

import torch

from . import _lib

__all__ = [
    "fp8_quantize_tensorwise", "fp8_quantize_rowwise", "fp8_quantize_blockwise", "fp8_quantize_blockwise_dual", "fp8_quantize_mx",
    "fp8_scaled_mm", "fp8_scaled_grouped_mm", "fp8_scaled_grouped_mm_v2", "grouped_runs_capacity",
    "fp8_quantize_grouped_128x1", "fp8_quantize_grouped_dual", "fp8_grouped_linear_grad_weight",
    "fp8_linear_forward",
    "fp8_linear_grad_input", "fp8_linear_grad_weight", "recipe_pair_supported",
    "FP8BlockwiseLinear", "fp8_blockwise_linear", "FP8GroupedLinear", "fp8_grouped_linear",
]

ROWWISE_EPS = 1e-12


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _ld(t, name):
    """Leading dimension of a row-major 2-D tensor (unit column stride)."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D row-major tensor")
    if t.shape[0] > 1 and t.shape[1] > 0:
        return t.stride(0)
    return _ld16(t.shape[1])     # one row or no columns: any padded width will do


def _ptr(t):
    return None if t is None else t.data_ptr()


def _recipe(r):
    if isinstance(r, str):
        if r not in _lib.RECIPES:
            raise ValueError(f"unknown recipe {r!r}")
        return _lib.RECIPES[r]
    return int(r)


def _out_code(dtype):
    if dtype == torch.bfloat16:
        return _lib.OUT_BF16
    if dtype == torch.float32:
        return _lib.OUT_FP32
    raise ValueError(f"out_dtype must be torch.bfloat16 or torch.float32, got {dtype}")


def _ld16(n):
    return max(16, (n + 15) // 16 * 16)


def _check_scale(scale, recipe, operand, M, N, K, device):
    """The C ABI takes bare pointers, so each scale array is checked here:
    a tensor on the operands' device, its dtype and its element count against
    the recipe (see fp8mm_recipe)."""
    if not isinstance(scale, torch.Tensor):
        raise ValueError(f"scale_{operand} must be a torch.Tensor")
    if scale.device != device:
        raise ValueError(f"scale_{operand} must be on {device}, got {scale.device}")
    r = _recipe(recipe)
    rows = M if operand == "a" else N
    want = {0: 1, 1: rows}
    if operand == "a":
        want[2] = (K // 128) * M
    else:
        want[3] = (N // 128) * (K // 128)
        want[4] = (K // 128) * N
    want[5] = rows * (K // 32)
    if r in want and scale.numel() != want[r]:
        raise ValueError(f"scale_{operand} has {scale.numel()} elements, recipe needs {want[r]}")
    want_dtype = torch.uint8 if r == 5 else torch.float32     # MXFP8: E8M0 bytes
    if scale.dtype != want_dtype:
        raise ValueError(f"scale_{operand} must be {want_dtype} for recipe {recipe!r}, got {scale.dtype}")


def fp8_quantize_tensorwise(x):
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((1, 1), dtype=torch.float32, device=x.device)
    st = _lib.load().fp8_quantize_tensorwise(x.data_ptr(), rows, cols, _ld(x, "x"), q.data_ptr(),
                                             _ld(q, "q"), s.data_ptr(), _stream(x))
    _lib.check(st, "fp8_quantize_tensorwise")
    return q, s


def fp8_quantize_rowwise(x, eps=ROWWISE_EPS):
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, 1), dtype=torch.float32, device=x.device)
    st = _lib.load().fp8_quantize_rowwise(x.data_ptr(), rows, cols, _ld(x, "x"), float(eps), q.data_ptr(),
                                          _ld(q, "q"), s.data_ptr(), _stream(x))
    _lib.check(st, "fp8_quantize_rowwise")
    return q, s


def fp8_quantize_blockwise(x, block=(1, 128), transpose_out=False):
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    br, bc = int(block[0]), int(block[1])
    if br <= 0 or bc <= 0 or rows % br or cols % bc:
        raise ValueError(f"shape {tuple(x.shape)} is not a multiple of block {(br, bc)}")
    qshape = (cols, rows) if transpose_out else (rows, cols)
    q = torch.empty(qshape, dtype=torch.uint8, device=x.device)
    if (br, bc) == (1, 128):
        sshape = (cols // 128, rows)
    elif (br, bc) == (128, 1):
        sshape = (rows // 128, cols)
    else:
        sshape = (rows // br, cols // bc)
    s = torch.empty(sshape, dtype=torch.float32, device=x.device)
    st = _lib.load().fp8_quantize_blockwise(x.data_ptr(), rows, cols, _ld(x, "x"), br, bc, int(bool(transpose_out)),
                                            q.data_ptr(), _ld(q, "q"), s.data_ptr(), _stream(x))
    _lib.check(st, "fp8_quantize_blockwise")
    return q, s


def fp8_quantize_mx(x):
    """MXFP8: (codes uint8 [rows, cols], E8M0 scale bytes uint8 [rows,
    cols/32]); cols % 32 == 0."""
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    if cols % 32:
        raise ValueError(f"cols ({cols}) must be a multiple of 32")
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    st = _lib.load().fp8_quantize_mx(x.data_ptr(), rows, cols, _ld(x, "x"), q.data_ptr(), _ld(q, "q"),
                                     s.data_ptr(), _stream(x))
    _lib.check(st, "fp8_quantize_mx")
    return q, s


def fp8_quantize_blockwise_dual(x):
    """grad_output of a linear layer, quantized once for both backward GEMMs:
    (q_row [rows, cols], scale_row [cols/128, rows]) with 1x128 groups and
    (q_col_t [cols, rows], scale_col [rows/128, cols]) with 128x1 groups,
    written transposed.  rows and cols multiples of 128."""
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    if rows % 128 or cols % 128:
        raise ValueError(f"shape {tuple(x.shape)} is not a multiple of 128")
    q_row = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s_row = torch.empty((cols // 128, rows), dtype=torch.float32, device=x.device)
    q_col = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    s_col = torch.empty((rows // 128, cols), dtype=torch.float32, device=x.device)
    st = _lib.load().fp8_quantize_blockwise_dual(x.data_ptr(), rows, cols, _ld(x, "x"), q_row.data_ptr(),
                                                 _ld(q_row, "q_row"), s_row.data_ptr(), q_col.data_ptr(),
                                                 _ld(q_col, "q_col_t"), s_col.data_ptr(), _stream(x))
    _lib.check(st, "fp8_quantize_blockwise_dual")
    return q_row, s_row, q_col, s_col


def fp8_scaled_mm(A, B, scale_a, recipe_a, scale_b, recipe_b, b_layout="NK", bias=None,
                  out_dtype=torch.bfloat16, out=None):
    """out = (A * s_a) @ (B * s_b)^T (+ bias).  A uint8 [M, K]; B uint8
    [N, K] (b_layout "NK") or [K, N] ("KN")."""
    _need(A, torch.uint8, "A")
    _need(B, torch.uint8, "B")
    if b_layout not in _lib.B_LAYOUTS:
        raise ValueError(f"b_layout must be 'NK' or 'KN', got {b_layout!r}")
    if B.device != A.device:
        raise ValueError(f"B must be on {A.device}, got {B.device}")
    M, K = A.shape
    N = B.shape[0] if b_layout == "NK" else B.shape[1]
    kb = B.shape[1] if b_layout == "NK" else B.shape[0]
    if kb != K:
        raise ValueError(f"contraction mismatch: A has K={K}, B has {kb}")
    _check_scale(scale_a, recipe_a, "a", M, N, K, A.device)
    _check_scale(scale_b, recipe_b, "b", M, N, K, A.device)
    if not (scale_a.is_contiguous() and scale_b.is_contiguous()):
        raise ValueError("scales must be contiguous")
    if bias is not None:
        _need(bias, torch.bfloat16, "bias")
        if bias.numel() != N or not bias.is_contiguous() or bias.device != A.device:
            raise ValueError("bias must be a contiguous bf16 tensor of N elements on the operands' device")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (M, N) or out.device != A.device:
        raise ValueError("out has the wrong dtype, shape or device")
    st = _lib.load().fp8_scaled_mm(A.data_ptr(), M, K, _ld(A, "A"), B.data_ptr(), N, _ld(B, "B"),
                                   _lib.B_LAYOUTS[b_layout], scale_a.data_ptr(), _recipe(recipe_a),
                                   scale_b.data_ptr(), _recipe(recipe_b), _ptr(bias), _out_code(out_dtype),
                                   out.data_ptr(), _ld(out, "out"), _stream(A))
    _lib.check(st, "fp8_scaled_mm")
    return out


def fp8_scaled_grouped_mm(A, B_EnK, offsets, scale_a, scale_b, bias=None, out_dtype=torch.bfloat16, out=None):
    """Grouped (MoE) GEMM in the form grouped_mm(act, weight.transpose(-2, -1),
    offs): A uint8 [M_total, K], B_EnK uint8 [E, N, K], offsets int32 [E]
    (cumulative end rows), rowwise scales scale_a [M_total] and scale_b [E, N],
    bias bf16 [N] added to every expert's rows.  Rows at or past offsets[-1]
    are left as they are in `out` (zeros when the output is allocated here)."""
    if offsets is None:
        raise ValueError("offsets are required for the grouped GEMM")
    _need(A, torch.uint8, "A")
    _need(B_EnK, torch.uint8, "B_EnK")
    _need(offsets, torch.int32, "offsets")
    _need(scale_a, torch.float32, "scale_a")
    _need(scale_b, torch.float32, "scale_b")
    if B_EnK.dim() != 3 or not B_EnK.is_contiguous() or not A.is_contiguous():
        raise ValueError("A must be contiguous [M_total, K] and B_EnK contiguous [E, N, K]")
    M, K = A.shape
    E, N, K2 = B_EnK.shape
    if K2 != K:
        raise ValueError(f"contraction mismatch: A has K={K}, B_EnK has {K2}")
    if offsets.numel() != E or not offsets.is_contiguous():
        raise ValueError("offsets must be a contiguous int32 tensor of E elements")
    if scale_a.numel() != M or scale_b.numel() != E * N:
        raise ValueError("rowwise scales must have M_total and E*N elements")
    if bias is not None:
        _need(bias, torch.bfloat16, "bias")
        if bias.numel() != N or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous bf16 tensor of N elements (shared by every expert)")
    if out is None:
        out = torch.zeros((M, N), dtype=out_dtype, device=A.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (M, N) or out.device != A.device:
        raise ValueError("out has the wrong dtype, shape or device")
    st = _lib.load().fp8_scaled_grouped_mm(A.data_ptr(), M, K, B_EnK.data_ptr(), E, N, offsets.data_ptr(),
                                           scale_a.data_ptr(), scale_b.data_ptr(), _ptr(bias),
                                           _out_code(out_dtype), out.data_ptr(), _ld(out, "out"), _stream(A))
    _lib.check(st, "fp8_scaled_grouped_mm")
    return out


def fp8_scaled_grouped_mm_v2(A, B_E, offsets, scale_a, recipe_a, scale_b, recipe_b, b_layout="NK", bias=None,
                             bias_per_expert=False, out_dtype=torch.bfloat16, out=None):
    """Grouped (MoE) GEMM with explicit recipes: rows [offsets[e-1],
    offsets[e]) of A [M_total, K] times expert e's B, B_E uint8 [E, N, K]
    (b_layout "NK") or [E, K, N] ("KN").  Pairs: rowwise x rowwise (scale_a
    [M_total], scale_b [E, N]) and 1x128 x 128x128 (scale_a [K/128, M_total],
    scale_b [E] x expert e's 128x128 grid of B as stored).  bias: bf16 [N]
    shared by every expert, or [E, N] (row e for expert e) with
    bias_per_expert=True.  Rows at or past offsets[-1] are left as they are in
    `out` (zeros when allocated here)."""
    if offsets is None:
        raise ValueError("offsets are required for the grouped GEMM")
    if b_layout not in _lib.B_LAYOUTS:
        raise ValueError(f"b_layout must be 'NK' or 'KN', got {b_layout!r}")
    _need(A, torch.uint8, "A")
    _need(B_E, torch.uint8, "B_E")
    _need(offsets, torch.int32, "offsets")
    if B_E.dim() != 3 or not B_E.is_contiguous() or A.dim() != 2 or not A.is_contiguous():
        raise ValueError("A must be contiguous [M_total, K] and B_E contiguous 3-D")
    M, K = A.shape
    if b_layout == "NK":
        E, N, K2 = B_E.shape
    else:
        E, K2, N = B_E.shape
    if K2 != K:
        raise ValueError(f"contraction mismatch: A has K={K}, B_E has {K2}")
    if offsets.numel() != E or not offsets.is_contiguous():
        raise ValueError("offsets must be a contiguous int32 tensor of E elements")
    ra, rb = _recipe(recipe_a), _recipe(recipe_b)
    for t, n in ((scale_a, "scale_a"), (scale_b, "scale_b")):
        _need(t, torch.float32, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if (ra, rb) == (_lib.RECIPES["1x128"], _lib.RECIPES["128x128"]):
        want_a, want_b = (K // 128) * M, E * (N // 128) * (K // 128)
    else:
        want_a, want_b = M, E * N
    if scale_a.numel() != want_a or scale_b.numel() != want_b:
        raise ValueError(f"scales have {scale_a.numel()} and {scale_b.numel()} elements, "
                         f"the recipes need {want_a} and {want_b}")
    if bias is not None:
        _need(bias, torch.bfloat16, "bias")
        want = E * N if bias_per_expert else N
        if bias.numel() != want or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous bf16 tensor of " +
                             ("[E, N] elements (bias_per_expert)" if bias_per_expert else "N elements"))
    if out is None:
        out = torch.zeros((M, N), dtype=out_dtype, device=A.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (M, N) or out.device != A.device:
        raise ValueError("out has the wrong dtype, shape or device")
    st = _lib.load().fp8_scaled_grouped_mm_v2(A.data_ptr(), M, K, B_E.data_ptr(), E, N, _lib.B_LAYOUTS[b_layout],
                                              offsets.data_ptr(), scale_a.data_ptr(), ra, scale_b.data_ptr(), rb,
                                              _ptr(bias), int(bool(bias_per_expert)), _out_code(out_dtype),
                                              out.data_ptr(), _ld(out, "out"), _stream(A))
    _lib.check(st, "fp8_scaled_grouped_mm_v2")
    return out


def grouped_runs_capacity(T, E):
    """Runs of 128 tokens that T tokens over E experts can need: T // 128 + E."""
    return int(_lib.load().fp8mm_grouped_runs_capacity(int(T), int(E)))


def fp8_quantize_grouped_128x1(x, offsets):
    """x bf16 [T, C] -> (q_t uint8 [C, ld], scale float32 [ld / 128, C]) with
    ld = 128 * grouped_runs_capacity(T, E): runs of 128 tokens restarted at
    each expert's first token (offsets int32 [E], cumulative end rows), run r
    at columns [128 r, 128 r + 128).  Columns and scale rows past the last run
    are left unwritten."""
    _need(x, torch.bfloat16, "x")
    _need(offsets, torch.int32, "offsets")
    if not offsets.is_contiguous() or offsets.dim() != 1:
        raise ValueError("offsets must be a contiguous 1-D int32 tensor")
    T, C = x.shape
    E = offsets.numel()
    ld = 128 * grouped_runs_capacity(T, E)
    q = torch.empty((C, max(ld, 16)), dtype=torch.uint8, device=x.device)
    scale = torch.empty((ld // 128, C), dtype=torch.float32, device=x.device)
    st = _lib.load().fp8_quantize_grouped_128x1(x.data_ptr(), T, C, _ld(x, "x"), offsets.data_ptr(), E,
                                                q.data_ptr(), q.stride(0), scale.data_ptr(), _stream(x))
    _lib.check(st, "fp8_quantize_grouped_128x1")
    return q, scale


def fp8_quantize_grouped_dual(x, offsets):
    """x bf16 [T, C] (C % 128 == 0) -> (q_row uint8 [T, C], scale_row float32
    [C/128, T], q_t uint8 [C, ld], scale_t float32 [ld/128, C]) from one read:
    the 1x128 codes of every row an expert owns (rows at or past
    offsets[-1] are left unwritten) and the per-expert runs of
    fp8_quantize_grouped_128x1."""
    _need(x, torch.bfloat16, "x")
    _need(offsets, torch.int32, "offsets")
    if not offsets.is_contiguous() or offsets.dim() != 1:
        raise ValueError("offsets must be a contiguous 1-D int32 tensor")
    T, C = x.shape
    E = offsets.numel()
    ld = 128 * grouped_runs_capacity(T, E)
    q_row = torch.empty((T, C), dtype=torch.uint8, device=x.device)
    s_row = torch.empty((C // 128, T), dtype=torch.float32, device=x.device)
    q_t = torch.empty((C, max(ld, 16)), dtype=torch.uint8, device=x.device)
    s_t = torch.empty((ld // 128, C), dtype=torch.float32, device=x.device)
    st = _lib.load().fp8_quantize_grouped_dual(x.data_ptr(), T, C, _ld(x, "x"), offsets.data_ptr(), E,
                                               q_row.data_ptr(), _ld16(C), s_row.data_ptr(), q_t.data_ptr(),
                                               q_t.stride(0), s_t.data_ptr(), _stream(x))
    _lib.check(st, "fp8_quantize_grouped_dual")
    return q_row, s_row, q_t, s_t


def fp8_grouped_linear_grad_weight(gt_q, gt_scale, xt_q, xt_scale, offsets, T, out_dtype=torch.bfloat16):
    """grad_w [E, N_out, K_in]: expert e's grad_output[rows_e].t() @
    input[rows_e] from the two outputs of fp8_quantize_grouped_128x1 with the
    same offsets and token count T."""
    for t, n in ((gt_q, "gt_q"), (xt_q, "xt_q")):
        _need(t, torch.uint8, n)
    for t, n in ((gt_scale, "gt_scale"), (xt_scale, "xt_scale")):
        _need(t, torch.float32, n)
    _need(offsets, torch.int32, "offsets")
    N_out, ld = gt_q.shape
    K_in = xt_q.shape[0]
    E = offsets.numel()
    if xt_q.shape[1] != ld or not (gt_q.is_contiguous() and xt_q.is_contiguous()):
        raise ValueError("gt_q [N_out, ld] and xt_q [K_in, ld] must be contiguous with the same ld")
    if gt_scale.shape != (ld // 128, N_out) or xt_scale.shape != (ld // 128, K_in):
        raise ValueError("scales must be [ld/128, N_out] and [ld/128, K_in]")
    out = torch.empty((E, N_out, K_in), dtype=out_dtype, device=gt_q.device)
    st = _lib.load().fp8_grouped_linear_grad_weight(gt_q.data_ptr(), N_out, gt_scale.data_ptr(), xt_q.data_ptr(),
                                                    K_in, xt_scale.data_ptr(), ld, int(T), offsets.data_ptr(), E,
                                                    _out_code(out_dtype), out.data_ptr(), _stream(gt_q))
    _lib.check(st, "fp8_grouped_linear_grad_weight")
    return out


def fp8_linear_forward(x_q, x_scale, x_recipe, w_q, w_scale, w_recipe, bias=None, out_dtype=torch.bfloat16):
    """out = input @ weight.t(): x_q [M, K], w_q [N, K]."""
    for t, n in ((x_q, "x_q"), (w_q, "w_q")):
        _need(t, torch.uint8, n)
    M, K = x_q.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K or not (x_q.is_contiguous() and w_q.is_contiguous()):
        raise ValueError("x_q [M, K] and w_q [N, K] must be contiguous with equal K")
    if bias is not None:
        _need(bias, torch.bfloat16, "bias")
        if bias.numel() != N or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous bf16 tensor of N elements")
    for t, n in ((x_scale, "x_scale"), (w_scale, "w_scale")):
        _need(t, torch.float32, n)
    _check_scale(x_scale, x_recipe, "a", M, N, K, x_q.device)
    _check_scale(w_scale, w_recipe, "b", M, N, K, x_q.device)
    out = torch.empty((M, N), dtype=out_dtype, device=x_q.device)
    st = _lib.load().fp8_linear_forward(x_q.data_ptr(), M, K, x_scale.data_ptr(), _recipe(x_recipe), w_q.data_ptr(),
                                        N, w_scale.data_ptr(), _recipe(w_recipe), _ptr(bias),
                                        _out_code(out_dtype), out.data_ptr(), _stream(x_q))
    _lib.check(st, "fp8_linear_forward")
    return out


def fp8_linear_grad_input(g_q, g_scale, g_recipe, w_q, w_scale, w_recipe, out_dtype=torch.bfloat16):
    """grad_input = grad_output @ weight: g_q [M, N_out], w_q [N_out, K_in]."""
    for t, n in ((g_q, "g_q"), (w_q, "w_q")):
        _need(t, torch.uint8, n)
    M, N_out = g_q.shape
    if w_q.shape[0] != N_out or not (g_q.is_contiguous() and w_q.is_contiguous()):
        raise ValueError("g_q [M, N_out] and w_q [N_out, K_in] must be contiguous")
    K_in = w_q.shape[1]
    for t, n in ((g_scale, "g_scale"), (w_scale, "w_scale")):
        _need(t, torch.float32, n)
    _check_scale(g_scale, g_recipe, "a", M, K_in, N_out, g_q.device)
    _check_scale(w_scale, w_recipe, "b", M, K_in, N_out, g_q.device)
    out = torch.empty((M, K_in), dtype=out_dtype, device=g_q.device)
    st = _lib.load().fp8_linear_grad_input(g_q.data_ptr(), M, N_out, g_scale.data_ptr(), _recipe(g_recipe),
                                           w_q.data_ptr(), K_in, w_scale.data_ptr(), _recipe(w_recipe),
                                           _out_code(out_dtype), out.data_ptr(), _stream(g_q))
    _lib.check(st, "fp8_linear_grad_input")
    return out


def fp8_linear_grad_weight(gt_q, gt_scale, xt_q, xt_scale, out_dtype=torch.bfloat16):
    """grad_weight = grad_output.t() @ input from (128, 1)-quantized,
    transposed operands: gt_q [N_out, T], xt_q [K_in, T]."""
    for t, n in ((gt_q, "gt_q"), (xt_q, "xt_q")):
        _need(t, torch.uint8, n)
    N_out, T = gt_q.shape
    if xt_q.shape[1] != T or not (gt_q.is_contiguous() and xt_q.is_contiguous()):
        raise ValueError("gt_q [N_out, T] and xt_q [K_in, T] must be contiguous with equal T")
    K_in = xt_q.shape[0]
    for t, n in ((gt_scale, "gt_scale"), (xt_scale, "xt_scale")):
        _need(t, torch.float32, n)
    _check_scale(gt_scale, "1x128", "a", N_out, K_in, T, gt_q.device)
    _check_scale(xt_scale, "128x1", "b", N_out, K_in, T, gt_q.device)
    out = torch.empty((N_out, K_in), dtype=out_dtype, device=gt_q.device)
    st = _lib.load().fp8_linear_grad_weight(gt_q.data_ptr(), N_out, T, gt_scale.data_ptr(), xt_q.data_ptr(), K_in,
                                            xt_scale.data_ptr(), _out_code(out_dtype), out.data_ptr(), _stream(gt_q))
    _lib.check(st, "fp8_linear_grad_weight")
    return out


def recipe_pair_supported(recipe_a, recipe_b, b_layout="NK"):
    return bool(_lib.load().fp8mm_recipe_pair_supported(_recipe(recipe_a), _recipe(recipe_b),
                                                        _lib.B_LAYOUTS[b_layout]))


from .linear import (FP8BlockwiseLinear, FP8GroupedLinear, fp8_blockwise_linear,  # noqa: E402  (uses the functions above)
                     fp8_grouped_linear)
