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

from . import (fp8_linear_forward, fp8_linear_grad_input, fp8_linear_grad_weight, fp8_quantize_blockwise,
               fp8_quantize_blockwise_dual)


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
