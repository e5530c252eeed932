"""FP8 blockwise linear layer as one autograd op: the forward GEMM, both
backward GEMMs and every quantization pass, each a call of the C ABI.

The data flow follows the FP8 linear of ColossalAI PR #6419 ("Fix: Handle
LowLevelZeroPlugin with use_fp8=True", Forward pass and Backward pass) with
the blockwise recipes of pytorch/ao PR #2784 ("improve fp8 blockwise gemm
perf"): input 1x128 x weight 128x128 for the forward and for grad_input,
grad_output 1x128 over tokens x input 128x1 over tokens for grad_weight.

  forward:  input  -> dual-layout quantize (1x128 rows for the forward GEMM,
                      128x1 transposed, kept for grad_weight)
            weight -> 128x128 quantize (kept for grad_input)
            out = input @ weight.t()
  backward: grad_out -> dual-layout quantize
            grad_input  = grad_out @ weight          (weight read as [K, N])
            grad_weight = grad_out.t() @ input       (both over tokens)

Python only orders the calls and allocates outputs; every step runs in the
library's kernels.  No bias: its gradient is a plain reduction outside the
FP8 path.
"""

import torch

from . import (fp8_grouped_linear_grad_weight, fp8_linear_forward, fp8_linear_grad_input, fp8_linear_grad_weight,
               fp8_quantize_blockwise, fp8_quantize_blockwise_dual, fp8_quantize_grouped_128x1,
               fp8_quantize_grouped_dual, fp8_scaled_grouped_mm_v2)


class FP8BlockwiseLinear(torch.autograd.Function):
    """y = x @ w.t() with x [T, K_in] and w [N_out, K_in] bf16 on the GPU;
    T, K_in, N_out multiples of 128.  Outputs and gradients are bf16."""

    @staticmethod
    def forward(ctx, x, w):
        if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
            raise ValueError("x and w must be bf16")
        x = x.contiguous()
        w = w.contiguous()
        qx, sx, qxt, sxt = fp8_quantize_blockwise_dual(x)
        qw, sw = fp8_quantize_blockwise(w, (128, 128))
        ctx.save_for_backward(qxt, sxt, qw, sw)
        return fp8_linear_forward(qx, sx, "1x128", qw, sw, "128x128")

    @staticmethod
    def backward(ctx, grad_out):
        qxt, sxt, qw, sw = ctx.saved_tensors
        g = grad_out.to(torch.bfloat16).contiguous()
        qg, sg, qgt, sgt = fp8_quantize_blockwise_dual(g)
        grad_x = grad_w = None
        if ctx.needs_input_grad[0]:
            grad_x = fp8_linear_grad_input(qg, sg, "1x128", qw, sw, "128x128")
        if ctx.needs_input_grad[1]:
            grad_w = fp8_linear_grad_weight(qgt, sgt, qxt, sxt)
        return grad_x, grad_w


def fp8_blockwise_linear(x, w):
    """x @ w.t() through FP8BlockwiseLinear (differentiable in x and w)."""
    return FP8BlockwiseLinear.apply(x, w)


class FP8GroupedLinear(torch.autograd.Function):
    """MoE expert layer y[rows_e] = x[rows_e] @ w[e].t() for every expert e,
    expert e owning token rows [offs[e-1], offs[e]) (the grouped form of
    pytorch/ao PR #4390), in the blockwise recipe applied per expert:

      forward:  x -> one read: 1x128 codes (forward GEMM) and per-expert
                     128-token runs written transposed (kept for grad_weight)
                w [E, N_out, K_in] -> 128x128 codes per expert (kept)
                y = grouped GEMM, expert weights read [N, K]
      backward: grad_out -> one read: 1x128 codes and per-expert runs
                grad_x    = grouped GEMM, the same weight codes read [K, N]
                grad_w[e] = grad_out[rows_e].t() @ x[rows_e]

    x [T, K_in], w [E, N_out, K_in] bf16, offs int32 [E] on the GPU; K_in and
    N_out multiples of 128.  Rows of y and grad_x at or past offs[E-1] are 0."""

    @staticmethod
    def forward(ctx, x, w, offs):
        if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
            raise ValueError("x and w must be bf16")
        x = x.contiguous()
        w = w.contiguous()
        E, N_out, K_in = w.shape
        qx, sx, qxt, sxt = fp8_quantize_grouped_dual(x, offs)
        qw, sw = fp8_quantize_blockwise(w.view(E * N_out, K_in), (128, 128))
        qw = qw.view(E, N_out, K_in)
        sw = sw.view(E, N_out // 128, K_in // 128)
        ctx.save_for_backward(qxt, sxt, qw, sw, offs)
        ctx.tokens = x.shape[0]
        return fp8_scaled_grouped_mm_v2(qx, qw, offs, sx, "1x128", sw, "128x128")

    @staticmethod
    def backward(ctx, grad_out):
        qxt, sxt, qw, sw, offs = ctx.saved_tensors
        g = grad_out.to(torch.bfloat16).contiguous()
        grad_x = grad_w = None
        need_x, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if need_x and need_w:
            qg, sg, qgt, sgt = fp8_quantize_grouped_dual(g, offs)
        elif need_x:
            qg, sg = fp8_quantize_blockwise(g, (1, 128))
        elif need_w:
            qgt, sgt = fp8_quantize_grouped_128x1(g, offs)
        if need_x:
            grad_x = fp8_scaled_grouped_mm_v2(qg, qw, offs, sg, "1x128", sw, "128x128", b_layout="KN")
        if need_w:
            grad_w = fp8_grouped_linear_grad_weight(qgt, sgt, qxt, sxt, offs, ctx.tokens)
        return grad_x, grad_w, None


def fp8_grouped_linear(x, w, offs):
    """The MoE expert layer through FP8GroupedLinear (differentiable in x and w)."""
    return FP8GroupedLinear.apply(x, w, offs)
