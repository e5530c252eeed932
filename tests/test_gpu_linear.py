"""The FP8 blockwise linear layer as one autograd op: forward output and both
gradients against the oracle's call forms on the same bf16 inputs (each side
quantizes independently; codes are bit-exact, so the GEMM bar applies)."""

import numpy as np
import pytest
import torch

import precision_matmul_amd as fp8mm
import workloads
from oracle import gemm, quant
from tests.gpu_util import bf16_dev, out_f64, say
from tests.test_gpu_gemm import _assert_close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,K_in,N_out", [(256, 384, 128), (640, 256, 512), (384, 1024, 384)])
def test_linear_forward_and_backward(T, K_in, N_out):
    say(f"linear T={T} K_in={K_in} N_out={N_out}")
    g = workloads.streams(T + K_in + N_out, 3)
    x = workloads.normal_bf16(g[0], (T, K_in))
    w = workloads.normal_bf16(g[1], (N_out, K_in), 0.02)
    go = workloads.normal_bf16(g[2], (T, N_out), 1e-3)
    xd = bf16_dev(x).requires_grad_(True)
    wd = bf16_dev(w).requires_grad_(True)
    y = fp8mm.fp8_blockwise_linear(xd, wd)
    y.backward(bf16_dev(go))
    # oracle: the same recipes through the call forms
    qx, sx = quant.quantize_blockwise(x, 1, 128)
    qw, sw = quant.quantize_blockwise(w, 128, 128)
    _assert_close(out_f64(y.detach()), gemm.linear_forward(qx, sx, "1x128", qw, sw, "128x128", out_dtype=None),
                  "linear forward")
    qg, sg = quant.quantize_blockwise(go, 1, 128)
    _assert_close(out_f64(xd.grad), gemm.linear_grad_input(qg, sg, "1x128", qw, sw, "128x128", out_dtype=None),
                  "linear grad_input")
    qgt, sgt = quant.quantize_blockwise(go, 128, 1, transpose_out=True)
    qxt, sxt = quant.quantize_blockwise(x, 128, 1, transpose_out=True)
    _assert_close(out_f64(wd.grad), gemm.linear_grad_weight(qgt, sgt, qxt, sxt, out_dtype=None),
                  "linear grad_weight")


def test_linear_gradient_only_for_what_requires_it():
    g = workloads.streams(5, 2)
    x = bf16_dev(workloads.normal_bf16(g[0], (128, 128)))
    w = bf16_dev(workloads.normal_bf16(g[1], (128, 128), 0.02)).requires_grad_(True)
    fp8mm.fp8_blockwise_linear(x, w).sum().backward()
    assert x.grad is None and w.grad is not None and w.grad.shape == (128, 128)
    assert bool(torch.isfinite(w.grad.float()).all())


@pytest.mark.parametrize("sizes,K_in,N_out", [([100, 0, 300, 129], 256, 384), ([40, 90, 7], 384, 128)])
def test_grouped_linear_forward_and_backward(sizes, K_in, N_out):
    """The MoE expert layer: output and both gradients against the oracle's
    grouped forms on the same bf16 inputs; 3 trailing rows no expert owns."""
    E = len(sizes)
    offs = np.cumsum(sizes).astype(np.int32)
    T = int(offs[-1]) + 3
    say(f"grouped linear sizes={sizes} K_in={K_in} N_out={N_out}")
    g = workloads.streams(T + K_in + N_out, 3)
    x = workloads.normal_bf16(g[0], (T, K_in))
    w = workloads.normal_bf16(g[1], (E, N_out, K_in), 0.02)
    go = workloads.normal_bf16(g[2], (T, N_out), 1e-3)
    xd = bf16_dev(x).requires_grad_(True)
    wd = bf16_dev(w).requires_grad_(True)
    od = torch.from_numpy(offs).cuda()
    y = fp8mm.fp8_grouped_linear(xd, wd, od)
    y.backward(bf16_dev(go))
    owned = np.zeros(T, bool)
    owned[:offs[-1]] = True
    qx, sx = quant.quantize_blockwise(x, 1, 128)
    qw, sw = quant.quantize_blockwise(w.reshape(E * N_out, K_in), 128, 128)
    qw, sw = qw.reshape(E, N_out, K_in), sw.reshape(E, N_out // 128, K_in // 128)
    ref, written = gemm.grouped_mm(qx, qw, offs, sx, sw, out_dtype=None, recipe_a="1x128", recipe_b="128x128")
    yv = out_f64(y.detach())
    assert np.array_equal(written, owned) and not yv[~owned].any()
    _assert_close(yv[owned], ref[owned], "grouped linear forward")
    qg, sg = quant.quantize_blockwise(go, 1, 128)
    ref_gx, _ = gemm.grouped_mm(qg, qw, offs, sg, sw, out_dtype=None, recipe_a="1x128", recipe_b="128x128",
                                layout="KN")
    gx = out_f64(xd.grad)
    assert not gx[~owned].any()
    _assert_close(gx[owned], ref_gx[owned], "grouped linear grad_input")
    qgt, sgt, _ = quant.quantize_grouped_128x1(go, offs)
    qxt, sxt, _ = quant.quantize_grouped_128x1(x, offs)
    ref_gw = gemm.grouped_grad_weight(qgt, sgt, qxt, sxt, offs, out_dtype=None)
    assert wd.grad.shape == (E, N_out, K_in)
    _assert_close(out_f64(wd.grad), ref_gw, "grouped linear grad_weight")
