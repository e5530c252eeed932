"""GPU parity of the scaled GEMM kernels against the CPU oracle.

Inputs are seeded bf16 tensors from ``workloads``; the GPU quantizes them
with the library and the oracle quantizes them itself (the quantizers are
bit-exact, checked in test_gpu_quant.py, so both sides multiply the same
codes).  The GEMM bar: relative Frobenius error <= 1e-3 and elementwise
|err| <= 4e-3 * max|ref| against the float64 oracle rounded once to the
output dtype.  Small cases compare every element; the benchmark shapes are
compared on sampled output entries that the oracle evaluates one by one.
"""

import numpy as np
import pytest
import torch

import precision_matmul_amd as fp8mm
import workloads
from oracle import gemm, mx, quant
from tests.gpu_util import TOL_FRO, TOL_MAX, bf16_dev, host, out_f64, say

pytestmark = pytest.mark.gpu

BLOCKS = {"1x128": (1, 128), "128x128": (128, 128), "128x1": (128, 1)}


def _assert_close(got, ref_exact, what, out_dtype="bf16"):
    """ref_exact: the unrounded float64 oracle (gemm.parity rounds it once to
    out_dtype for the Frobenius figure)."""
    rel_f, rel_m = gemm.parity(got, ref_exact, out_dtype)
    say(f"{what}: rel_fro={rel_f:.3e} rel_max={rel_m:.3e}")
    assert np.all(np.isfinite(got)), what
    assert rel_f <= TOL_FRO and rel_m <= TOL_MAX, (what, rel_f, rel_m)


def _quant_both(bits, recipe, transpose_out=False):
    """(gpu codes, gpu scales, oracle codes, oracle scales)."""
    d = bf16_dev(bits)
    if recipe == "tensorwise":
        q, s = fp8mm.fp8_quantize_tensorwise(d)
        rq, rs = quant.quantize_tensorwise(bits)
    elif recipe == "rowwise":
        q, s = fp8mm.fp8_quantize_rowwise(d)
        rq, rs = quant.quantize_rowwise(bits)
    else:
        q, s = fp8mm.fp8_quantize_blockwise(d, BLOCKS[recipe], transpose_out=transpose_out)
        rq, rs = quant.quantize_blockwise(bits, *BLOCKS[recipe], transpose_out=transpose_out)
    return q, s, rq, rs


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_tensorwise_256(out_dtype):
    inp = workloads.tensorwise()
    qa, sa, ra, rsa = _quant_both(inp["A"], "tensorwise")
    qb, sb, rb, rsb = _quant_both(inp["B"], "tensorwise")
    out = fp8mm.fp8_scaled_mm(qa, qb, sa, "tensorwise", sb, "tensorwise", out_dtype=out_dtype)
    od = "bf16" if out_dtype == torch.bfloat16 else "fp32"
    _assert_close(out_f64(out), gemm.scaled_mm(ra, rb, rsa, "tensorwise", rsb, "tensorwise", out_dtype=None),
                  f"tensorwise 256^3 {od}", out_dtype=od)


def test_exact_small_integer_gemm():
    """Codes of small integers with unit scales: the GEMM is exact in fp32."""
    rng = np.random.default_rng(5)
    from tests.test_oracle_gemm import _int_codes
    a = rng.integers(-16, 17, size=(70, 256))
    b = rng.integers(-16, 17, size=(50, 256))
    A, B = _int_codes(a), _int_codes(b)
    one = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    out = fp8mm.fp8_scaled_mm(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), one, "tensorwise",
                              one, "tensorwise", out_dtype=torch.float32)
    assert np.array_equal(out_f64(out), (a @ b.T).astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 200, 4096), (17, 33, 144), (512, 640, 1040)])
@pytest.mark.parametrize("layout", ["NK", "KN"])
def test_tensorwise_shapes(M, N, K, layout):
    inp = workloads.tensorwise(n=N, m=M, k=K, seed=M * 31 + N)
    qa, sa, ra, rsa = _quant_both(inp["A"], "tensorwise")
    if layout == "NK":
        qb, sb, rb, rsb = _quant_both(inp["B"], "tensorwise")
    else:
        # B stored [K, N] with rows padded to a multiple of 16 bytes; zero
        # padding leaves the tensorwise amax, hence the codes, unchanged.
        bits_b = np.ascontiguousarray(inp["B"].T)
        ldb = (N + 15) // 16 * 16
        padded = np.zeros((K, ldb), np.uint16)
        padded[:, :N] = bits_b
        qpad, sb, _, _ = _quant_both(padded, "tensorwise")
        qb = qpad[:, :N]
        rb, rsb = quant.quantize_tensorwise(bits_b)
        assert np.array_equal(host(qb), rb)
    out = fp8mm.fp8_scaled_mm(qa, qb, sa, "tensorwise", sb, "tensorwise", b_layout=layout)
    _assert_close(out_f64(out), gemm.scaled_mm(ra, rb, rsa, "tensorwise", rsb, "tensorwise", layout, out_dtype=None),
                  f"tensorwise {M}x{N}x{K} {layout}")


@pytest.mark.parametrize("M,N,K", [(300, 200, 4096), (256, 512, 1024), (1, 16, 16), (129, 257, 528)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_rowwise_linear(M, N, K, with_bias):
    inp = workloads.rowwise(M=M, N=N, K=K, seed=M + N + K)
    qa, sa, ra, rsa = _quant_both(inp["x"], "rowwise")
    qb, sb, rb, rsb = _quant_both(inp["w"], "rowwise")
    bias = bf16_dev(inp["bias"]) if with_bias else None
    rbias = quant.bf16_to_f32(inp["bias"]) if with_bias else None
    out = fp8mm.fp8_scaled_mm(qa, qb, sa, "rowwise", sb, "rowwise", bias=bias)
    _assert_close(out_f64(out), gemm.scaled_mm(ra, rb, rsa, "rowwise", rsb, "rowwise", bias=rbias, out_dtype=None),
                  f"rowwise {M}x{N}x{K} bias={with_bias}")
    fwd = fp8mm.fp8_linear_forward(qa, sa, "rowwise", qb, sb, "rowwise", bias=bias)
    assert torch.equal(fwd, out)


@pytest.mark.parametrize("M,N,K", [(320, 384, 1024), (256, 256, 128), (1000, 128, 512), (64, 640, 2048)])
def test_blockwise_forward(M, N, K):
    inp = workloads.blockwise(M=M, N=N, K=K, seed=M + 3 * N + K)
    qa, sa, ra, rsa = _quant_both(inp["input"], "1x128")
    qb, sb, rb, rsb = _quant_both(inp["weight"], "128x128")
    out = fp8mm.fp8_linear_forward(qa, sa, "1x128", qb, sb, "128x128")
    _assert_close(out_f64(out), gemm.linear_forward(ra, rsa, "1x128", rb, rsb, "128x128", out_dtype=None),
                  f"blockwise fwd {M}x{N}x{K}")


@pytest.mark.parametrize("M,N_out,K_in", [(320, 512, 384), (256, 128, 256), (130, 256, 640)])
def test_blockwise_grad_input(M, N_out, K_in):
    inp = workloads.blockwise(M=M, N=N_out, K=K_in, seed=M + N_out + 5 * K_in)
    qg, sg, rg, rsg = _quant_both(inp["grad_output"], "1x128")      # [M, N_out]
    qw, sw, rw, rsw = _quant_both(inp["weight"], "128x128")          # [N_out, K_in]
    out = fp8mm.fp8_linear_grad_input(qg, sg, "1x128", qw, sw, "128x128")
    _assert_close(out_f64(out), gemm.linear_grad_input(rg, rsg, "1x128", rw, rsw, "128x128", out_dtype=None),
                  f"blockwise grad_input {M}x{K_in}x{N_out}")


@pytest.mark.parametrize("T,N_out,K_in", [(512, 256, 384), (256, 128, 128), (384, 80, 176)])
def test_blockwise_grad_weight(T, N_out, K_in):
    inp = workloads.grad_weight(T=T, N_out=N_out, K_in=K_in, seed=T + N_out + K_in)
    qg, sg, rg, rsg = _quant_both(inp["grad_output"], "128x1", transpose_out=True)   # [N_out, T]
    qx, sx, rx, rsx = _quant_both(inp["input"], "128x1", transpose_out=True)         # [K_in, T]
    out = fp8mm.fp8_linear_grad_weight(qg, sg, qx, sx)
    _assert_close(out_f64(out), gemm.linear_grad_weight(rg, rsg, rx, rsx, out_dtype=None),
                  f"blockwise grad_weight {N_out}x{K_in}x{T}")


# More 256 x 256 output tiles than compute units, with a short last round:
# the streaming kernel takes the tile rows that fill whole rounds and the
# remaining (ragged) rows run on smaller tiles.  On a 256-CU device M = 4400
# gives 18 x 16 tiles and a 32-tile tail (128 x 128 tail tiles), M = 5008
# gives 20 x 16 tiles and a 64-tile tail (256 x 128 tail tiles); elsewhere
# the same shapes still check the full result.
@pytest.mark.parametrize("M,K", [(4400, 256), (5008, 256), (4400, 2048)])
@pytest.mark.parametrize("recipe", ["tensorwise", "rowwise", "blockwise", "grad_weight", "grad_input",
                                    "tensorwise_kn"])
def test_split_tail_rows(recipe, M, K):
    """K = 2048 also splits the 32-tile tail of M = 4400 along K (two ranges
    of 8 steps, fp32 partials summed by a second kernel, bias added there)."""
    N = 4096
    if recipe == "grad_input":
        # B stored [K, N]: grad_output [M, 256] @ weight [256, 4096]
        inp = workloads.blockwise(M=M, N=K, K=N, seed=81)
        qg, sg, rg, rsg = _quant_both(inp["grad_output"], "1x128")
        qw, sw, rw, rsw = _quant_both(inp["weight"], "128x128")
        out = fp8mm.fp8_linear_grad_input(qg, sg, "1x128", qw, sw, "128x128")
        ref = gemm.linear_grad_input(rg, rsg, "1x128", rw, rsw, "128x128", out_dtype=None)
    elif recipe == "tensorwise_kn":
        inp = workloads.tensorwise(n=N, m=M, k=K, seed=82)
        qa, sa, ra, rsa = _quant_both(inp["A"], "tensorwise")
        qb, sb, rb, rsb = _quant_both(np.ascontiguousarray(inp["B"].T), "tensorwise")   # [K, N]
        out = fp8mm.fp8_scaled_mm(qa, qb, sa, "tensorwise", sb, "tensorwise", b_layout="KN")
        ref = gemm.scaled_mm(ra, rb, rsa, "tensorwise", rsb, "tensorwise", layout="KN", out_dtype=None)
    elif recipe == "grad_weight":
        inp = workloads.grad_weight(T=K, N_out=M, K_in=N, seed=77)
        qg, sg, rg, rsg = _quant_both(inp["grad_output"], "128x1", transpose_out=True)
        qx, sx, rx, rsx = _quant_both(inp["input"], "128x1", transpose_out=True)
        out = fp8mm.fp8_linear_grad_weight(qg, sg, qx, sx)
        ref = gemm.linear_grad_weight(rg, rsg, rx, rsx, out_dtype=None)
    elif recipe == "blockwise":
        inp = workloads.blockwise(M=M, N=N, K=K, seed=78)
        qa, sa, ra, rsa = _quant_both(inp["input"], "1x128")
        qb, sb, rb, rsb = _quant_both(inp["weight"], "128x128")
        out = fp8mm.fp8_linear_forward(qa, sa, "1x128", qb, sb, "128x128")
        ref = gemm.linear_forward(ra, rsa, "1x128", rb, rsb, "128x128", out_dtype=None)
    elif recipe == "rowwise":
        inp = workloads.rowwise(M=M, N=N, K=K, seed=79)
        qa, sa, ra, rsa = _quant_both(inp["x"], "rowwise")
        qb, sb, rb, rsb = _quant_both(inp["w"], "rowwise")
        bias = bf16_dev(inp["bias"])
        out = fp8mm.fp8_scaled_mm(qa, qb, sa, "rowwise", sb, "rowwise", bias=bias)
        ref = gemm.scaled_mm(ra, rb, rsa, "rowwise", rsb, "rowwise", bias=quant.bf16_to_f32(inp["bias"]),
                             out_dtype=None)
    else:
        inp = workloads.tensorwise(n=N, m=M, k=K, seed=80)
        qa, sa, ra, rsa = _quant_both(inp["A"], "tensorwise")
        qb, sb, rb, rsb = _quant_both(inp["B"], "tensorwise")
        out = fp8mm.fp8_scaled_mm(qa, qb, sa, "tensorwise", sb, "tensorwise")
        ref = gemm.scaled_mm(ra, rb, rsa, "tensorwise", rsb, "tensorwise", out_dtype=None)
    _assert_close(out_f64(out), ref, f"split tail {recipe} {M}x{N}x{K}")


@pytest.mark.parametrize("recipe", ["blockwise", "grad_input", "rowwise", "mxfp8"])
def test_split_tail_three_uneven_k_ranges(recipe):
    """A row tail split along K into three uneven ranges.  M = 3300, 5120
    output columns: 13 x 20 = 260 tiles of 256 x 256, so on a 256-CU device
    the streaming kernel takes the 12 tile rows that fill whole rounds (240
    tiles, rows 0 .. 3071) and the 228 remaining rows (20 tiles of 256 x 256,
    80 of 128 x 128) are split into min(256 / 80, 25 / 8, 8) = 3 K ranges of
    8, 8 and 9 steps over the contraction of 3200 (25 steps of 128); with B
    stored [K, N] (grad_input) the tail runs 40 tiles of 256 x 128 in
    min(256 / 40, 25 / 8, 8) = 3 ranges.  The same split happens at 16640 x
    5120 x 8192 (21 / 21 / 22 of 64 steps).  Every element is compared; the
    rowwise case adds the bias in the reduction."""
    M, N, K = 3300, 5120, 3200
    if recipe == "grad_input":
        # grad_input [M, 5120] = grad_output [M, 3200] @ weight [3200, 5120] (B stored [K, N])
        inp = workloads.blockwise(M=M, N=K, K=N, seed=91)
        qg, sg, rg, rsg = _quant_both(inp["grad_output"], "1x128")
        qw, sw, rw, rsw = _quant_both(inp["weight"], "128x128")
        out = fp8mm.fp8_linear_grad_input(qg, sg, "1x128", qw, sw, "128x128")
        ref = gemm.linear_grad_input(rg, rsg, "1x128", rw, rsw, "128x128", out_dtype=None)
    elif recipe == "blockwise":
        inp = workloads.blockwise(M=M, N=N, K=K, seed=92)
        qa, sa, ra, rsa = _quant_both(inp["input"], "1x128")
        qb, sb, rb, rsb = _quant_both(inp["weight"], "128x128")
        out = fp8mm.fp8_linear_forward(qa, sa, "1x128", qb, sb, "128x128")
        ref = gemm.linear_forward(ra, rsa, "1x128", rb, rsb, "128x128", out_dtype=None)
    elif recipe == "rowwise":
        inp = workloads.rowwise(M=M, N=N, K=K, seed=93)
        qa, sa, ra, rsa = _quant_both(inp["x"], "rowwise")
        qb, sb, rb, rsb = _quant_both(inp["w"], "rowwise")
        out = fp8mm.fp8_scaled_mm(qa, qb, sa, "rowwise", sb, "rowwise", bias=bf16_dev(inp["bias"]))
        ref = gemm.scaled_mm(ra, rb, rsa, "rowwise", rsb, "rowwise", bias=quant.bf16_to_f32(inp["bias"]),
                             out_dtype=None)
    else:
        g = workloads.streams(94, 2)
        x = workloads.normal_bf16(g[0], (M, K))
        w = workloads.normal_bf16(g[1], (N, K), 0.02)
        qa, sa = fp8mm.fp8_quantize_mx(bf16_dev(x))
        qb, sb = fp8mm.fp8_quantize_mx(bf16_dev(w))
        ra, rsa = mx.quantize_mx(x)
        rb, rsb = mx.quantize_mx(w)
        out = fp8mm.fp8_scaled_mm(qa, qb, sa, "mxfp8", sb, "mxfp8")
        ref = gemm.scaled_mm(ra, rb, rsa, "mxfp8", rsb, "mxfp8", out_dtype=None)
    got = out_f64(out)
    _assert_close(got, ref, f"three-way split tail {recipe} {M}x{N}x{K}")
    _assert_close(got[3072:], ref[3072:], f"three-way split tail {recipe}: the tail rows alone")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("pad", [0, 64])
def test_output_rows_contiguous_or_padded(out_dtype, pad):
    """M = 4400 has a short tail on a 256-CU device.  pad = 0: the split
    tail's fp32 partials are staged in the output's head rows, which are then
    overwritten.  pad = 64 (ldo > N): the rows are not contiguous, the tail
    runs unsplit, and every padding column keeps its sentinel."""
    M, N, K = 4400, 4096, 2048
    inp = workloads.blockwise(M=M, N=N, K=K, seed=83)
    qa, sa, ra, rsa = _quant_both(inp["input"], "1x128")
    qb, sb, rb, rsb = _quant_both(inp["weight"], "128x128")
    full = torch.full((M, N + pad), -7.0, dtype=out_dtype, device="cuda")
    out = full[:, :N]
    fp8mm.fp8_scaled_mm(qa, qb, sa, "1x128", sb, "128x128", out_dtype=out_dtype, out=out)
    pad = full[:, N:]
    assert bool((pad == -7.0).all()), "padding columns of the output were written"
    ref = gemm.linear_forward(ra, rsa, "1x128", rb, rsb, "128x128", out_dtype=None)
    _assert_close(out_f64(out), ref, f"padded output {out_dtype}",
                  out_dtype="bf16" if out_dtype == torch.bfloat16 else "fp32")


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (300, 200, 1024), (17, 528, 256), (640, 896, 2048),
                                   (4400, 4096, 512), (4400, 4096, 2048)])
@pytest.mark.parametrize("with_bias,out_dtype", [(False, torch.bfloat16), (True, torch.float32)])
def test_mxfp8_scaled_mm(M, N, K, with_bias, out_dtype):
    """MXFP8 x MXFP8 (E8M0 per 32 along K, applied by the block-scaled MFMA)
    against the oracle's dequantize-then-matmul on the same bf16 inputs.
    The shapes reach every launch path: small problems on 128 x 128 tiles
    only, the streaming kernel with a 128 x 128 tail (4400 x 4096 x 512) and
    with a tail split along K (4400 x 4096 x 2048)."""
    g = workloads.streams(M + N + K, 3)
    x = workloads.normal_bf16(g[0], (M, K))
    w = workloads.normal_bf16(g[1], (N, K), 0.02)
    bias = workloads.normal_bf16(g[2], (N,), 0.01) if with_bias else None
    qa, sa = fp8mm.fp8_quantize_mx(bf16_dev(x))
    qb, sb = fp8mm.fp8_quantize_mx(bf16_dev(w))
    ra, rsa = mx.quantize_mx(x)
    rb, rsb = mx.quantize_mx(w)
    assert np.array_equal(host(qa), ra) and np.array_equal(host(sa), rsa)
    out = fp8mm.fp8_scaled_mm(qa, qb, sa, "mxfp8", sb, "mxfp8", out_dtype=out_dtype,
                              bias=None if bias is None else bf16_dev(bias))
    ref = gemm.scaled_mm(ra, rb, rsa, "mxfp8", rsb, "mxfp8",
                         bias=None if bias is None else quant.bf16_to_f32(bias), out_dtype=None)
    _assert_close(out_f64(out), ref, f"mxfp8 {M}x{N}x{K} bias={with_bias}",
                  out_dtype="bf16" if out_dtype == torch.bfloat16 else "fp32")


def test_full_mxfp8_sampled():
    """The blockwise forward shape 16640x5120x8192 in MXFP8, sampled entries."""
    M, N, K = 16640, 5120, 8192
    inp = workloads.blockwise(M=M, N=N, K=K)
    x, w = inp["input"], inp["weight"]
    qa, sa = fp8mm.fp8_quantize_mx(bf16_dev(x))
    qb, sb = fp8mm.fp8_quantize_mx(bf16_dev(w))
    out = out_f64(fp8mm.fp8_scaled_mm(qa, qb, sa, "mxfp8", sb, "mxfp8"))
    I = _rows_with_tail(M, 48, 16, 11)
    J = _sample(N, 64, 12)
    ra, rsa = mx.quantize_mx(x[I])
    rb, rsb = mx.quantize_mx(w[J])
    ref = gemm.scaled_mm(ra, rb, rsa, "mxfp8", rsb, "mxfp8", out_dtype=None)
    _assert_close(out[np.ix_(I, J)], ref, "mxfp8 16640x5120x8192 sampled")


def _grouped_case(E, N, K, sizes, seed, bias_form=None):
    """bias_form: None, "shared" (bf16 [N] through fp8_scaled_grouped_mm) or
    "per_expert" (bf16 [E, N] through fp8_scaled_grouped_mm_v2)."""
    g = workloads.streams(seed, 3)
    M = int(np.sum(sizes))
    act = workloads.normal_bf16(g[0], (M + 7, K))          # 7 trailing rows no expert owns
    W = workloads.normal_bf16(g[1], (E, N, K), 0.02)
    bias = None
    if bias_form is not None:
        bias = workloads.normal_bf16(g[2], (E, N) if bias_form == "per_expert" else (N,), 0.5)
    offs = np.cumsum(sizes).astype(np.int32)
    qa, sa, ra, rsa = _quant_both(act, "rowwise")
    qw, sw, rw, rsw = _quant_both(W.reshape(E * N, K), "rowwise")
    if bias_form == "per_expert":
        out = fp8mm.fp8_scaled_grouped_mm_v2(qa, qw.reshape(E, N, K), torch.from_numpy(offs).cuda(), sa.reshape(-1),
                                             "rowwise", sw.reshape(-1), "rowwise", bias=bf16_dev(bias),
                                             bias_per_expert=True)
    else:
        out = fp8mm.fp8_scaled_grouped_mm(qa, qw.reshape(E, N, K), torch.from_numpy(offs).cuda(), sa,
                                          sw.reshape(E, N), bias=None if bias is None else bf16_dev(bias))
    ref, written = gemm.grouped_mm(ra, rw.reshape(E, N, K), offs, rsa, rsw.reshape(E, N),
                                   bias=None if bias is None else quant.bf16_to_f32(bias), out_dtype=None)
    got = out_f64(out)
    assert np.all(got[~written] == 0), "rows no expert owns must not be written"
    return got[written], ref[written]


@pytest.mark.parametrize("E,N,K,sizes", [
    (8, 256, 512, [100, 0, 300, 1, 129, 0, 0, 256]),
    (3, 136, 272, [5, 260, 64]),
    (1, 128, 256, [333]),
    (70, 64, 128, [3] * 70),
    (4, 128, 64, [10, 50, 0, 70]),                       # K below 128 bytes: 128 x 128 tiles
    (16, 384, 1024, [300, 257, 256, 255, 1, 0, 512, 40, 290, 310, 222, 260, 275, 233, 249, 301]),
    # experts of 800 rows on average: the 256 x 256 streaming tiles (the
    # cases above have at most 384 rows per expert on average and take the
    # 320-row weight-streaming kernel)
    (2, 256, 512, [700, 900]),
    (3, 400, 384, [1000, 0, 700])])
@pytest.mark.parametrize("bias_form", [None, "shared", "per_expert"])
def test_grouped_rowwise(E, N, K, sizes, bias_form):
    got, ref = _grouped_case(E, N, K, np.array(sizes), seed=E + N + K, bias_form=bias_form)
    _assert_close(got, ref, f"grouped E={E} N={N} K={K} bias={bias_form}")


def test_grouped_single_expert_equals_rowwise_gemm():
    inp = workloads.rowwise(M=200, N=128, K=256, seed=77)
    qa, sa, _, _ = _quant_both(inp["x"], "rowwise")
    qb, sb, _, _ = _quant_both(inp["w"], "rowwise")
    grouped = fp8mm.fp8_scaled_grouped_mm(qa, qb.reshape(1, 128, 256), torch.tensor([200], dtype=torch.int32,
                                          device="cuda"), sa, sb)
    plain = fp8mm.fp8_scaled_mm(qa, qb, sa, "rowwise", sb, "rowwise")
    ra, rsa = quant.quantize_rowwise(inp["x"])
    rb, rsb = quant.quantize_rowwise(inp["w"])
    ref = gemm.scaled_mm(ra, rb, rsa, "rowwise", rsb, "rowwise", out_dtype=None)
    _assert_close(out_f64(grouped), ref, "grouped E=1")
    _assert_close(out_f64(plain), ref, "rowwise (same operands)")
    say(f"grouped E=1 and rowwise outputs bit-identical: {torch.equal(grouped, plain)}")


def test_zero_sized_problems():
    dev = "cuda"
    z = torch.empty((0, 128), dtype=torch.uint8, device=dev)
    b = torch.zeros((64, 128), dtype=torch.uint8, device=dev)
    one = torch.ones((1, 1), dtype=torch.float32, device=dev)
    out = fp8mm.fp8_scaled_mm(z, b, one, "tensorwise", one, "tensorwise")
    assert out.shape == (0, 64)
    a = torch.zeros((8, 0), dtype=torch.uint8, device=dev)
    bb = torch.zeros((4, 0), dtype=torch.uint8, device=dev)
    out = fp8mm.fp8_scaled_mm(a, bb, one, "tensorwise", one, "tensorwise", out_dtype=torch.float32)
    assert torch.count_nonzero(out).item() == 0


def test_host_scale_tensors_are_rejected():
    """The ABI takes bare device pointers: a scale (or bias) in host memory
    must be refused with ValueError before anything is launched."""
    a = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    dev_one = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    host_one = torch.ones((1, 1), dtype=torch.float32)
    with pytest.raises(ValueError, match="scale_a"):
        fp8mm.fp8_scaled_mm(a, a, host_one, "tensorwise", dev_one, "tensorwise")
    with pytest.raises(ValueError, match="scale_b"):
        fp8mm.fp8_scaled_mm(a, a, dev_one, "tensorwise", host_one, "tensorwise")
    with pytest.raises(ValueError, match="x_scale"):
        fp8mm.fp8_linear_forward(a, host_one, "tensorwise", a, dev_one, "tensorwise")
    with pytest.raises(ValueError, match="bias"):
        fp8mm.fp8_scaled_mm(a, a, dev_one, "tensorwise", dev_one, "tensorwise",
                            bias=torch.zeros(256, dtype=torch.bfloat16))
    torch.cuda.synchronize()


def test_unsupported_pair_raises_not_implemented():
    a = torch.zeros((128, 128), dtype=torch.uint8, device="cuda")
    s = torch.ones((128, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(NotImplementedError):
        fp8mm.fp8_scaled_mm(a, a, s, "rowwise", torch.ones((1, 1), device="cuda"), "tensorwise")


# ---- benchmark shapes: full-size launches, sampled outputs ----

def _sample(n, count, seed):
    return np.sort(np.random.default_rng(seed).choice(n, count, replace=False))


def test_full_rowwise_linear_sampled():
    inp = workloads.rowwise()
    x, w, bias = inp["x"], inp["w"], inp["bias"]
    qa, sa = fp8mm.fp8_quantize_rowwise(bf16_dev(x))
    qb, sb = fp8mm.fp8_quantize_rowwise(bf16_dev(w))
    out = fp8mm.fp8_scaled_mm(qa, qb, sa, "rowwise", sb, "rowwise", bias=bf16_dev(bias))
    got = out_f64(out)
    I, J = _sample(x.shape[0], 64, 1), _sample(w.shape[0], 64, 2)
    ra, rsa = quant.quantize_rowwise(x[I])
    rb, rsb = quant.quantize_rowwise(w[J])
    ref = gemm.scaled_mm(ra, rb, rsa, "rowwise", rsb, "rowwise", bias=quant.bf16_to_f32(bias[J]), out_dtype=None)
    _assert_close(got[np.ix_(I, J)], ref, "rowwise 8192x4096x4096 sampled")


def _rows_with_tail(M, count, tail_count, seed):
    """Sampled output rows: `count` from the rows the 256 x 256 streaming
    tiles cover and `tail_count` from the row tail.  At M = 16640 with N of
    5120 or 8192 on a 256-CU device the tiles fill exactly 5 or 8 rounds with
    rows 0 .. 16383, and rows 16384 .. 16639 run on the 128 x 128 tail tiles,
    split along K (3 uneven ranges of 21 / 21 / 22 K steps when the output
    has 20 tile columns and K = 8192, 2 even ones otherwise) and summed by the
    reduction kernel."""
    assert M == 16640
    head = 16384
    return np.concatenate([_sample(head, count, seed), head + _sample(M - head, tail_count, seed + 100)])


@pytest.mark.parametrize("M,N,K", [(16640, 5120, 8192), (16640, 8192, 5120)])
def test_full_blockwise_forward_and_grad_input_sampled(M, N, K):
    inp = workloads.blockwise(M=M, N=N, K=K)
    x, w, go = inp["input"], inp["weight"], inp["grad_output"]
    qx, sx = fp8mm.fp8_quantize_blockwise(bf16_dev(x), (1, 128))
    qw, sw = fp8mm.fp8_quantize_blockwise(bf16_dev(w), (128, 128))
    fwd = out_f64(fp8mm.fp8_linear_forward(qx, sx, "1x128", qw, sw, "128x128"))
    I = _rows_with_tail(M, 40, 16, 3)
    assert np.sum(I >= 16384) == 16
    slabs = _sample(N // 128, 3, 4)
    J = np.concatenate([s * 128 + _sample(128, 16, 5 + s) for s in slabs])
    rqx, rsx = quant.quantize_blockwise(x[I], 1, 128)
    # evaluate per slab with the slab's scale row (columns of a slab share one 128-row block)
    ref = np.zeros((len(I), len(J)))
    for t, s in enumerate(slabs):
        q, sc = quant.quantize_blockwise(w[s * 128:(s + 1) * 128], 128, 128)
        cols = J[t * 16:(t + 1) * 16] - s * 128
        full = gemm.scaled_mm(rqx, q, rsx, "1x128", sc, "128x128", out_dtype=None)   # [len(I), 128]
        ref[:, t * 16:(t + 1) * 16] = full[:, cols]
    _assert_close(fwd[np.ix_(I, J)], ref, f"blockwise fwd {M}x{N}x{K} sampled")
    # grad_input = grad_output @ weight, with grad_output [M, N] and weight [N, K]
    qg, sg = fp8mm.fp8_quantize_blockwise(bf16_dev(go), (1, 128))
    gi = out_f64(fp8mm.fp8_linear_grad_input(qg, sg, "1x128", qw, sw, "128x128"))
    Jk = _sample(K, 48, 6)
    rqg, rsg = quant.quantize_blockwise(go[I], 1, 128)
    rqw_full, rsw_full = quant.quantize_blockwise(w, 128, 128)
    ref_gi = gemm.scaled_mm_entries(rqg, rqw_full, rsg, "1x128", rsw_full, "128x128",
                                    np.repeat(np.arange(len(I)), len(Jk)), np.tile(Jk, len(I)), layout="KN",
                                    out_dtype=None)
    _assert_close(gi[np.ix_(I, Jk)].reshape(-1), ref_gi, f"blockwise grad_input {M}x{K}x{N} sampled")


def test_full_blockwise_grad_weight_sampled():
    inp = workloads.grad_weight()
    go, x = inp["grad_output"], inp["input"]                # [T, N_out], [T, K_in]
    qg, sg = fp8mm.fp8_quantize_blockwise(bf16_dev(go), (128, 1), transpose_out=True)
    qx, sx = fp8mm.fp8_quantize_blockwise(bf16_dev(x), (128, 1), transpose_out=True)
    gw = out_f64(fp8mm.fp8_linear_grad_weight(qg, sg, qx, sx))
    I, J = _sample(go.shape[1], 48, 7), _sample(x.shape[1], 48, 8)
    rqg, rsg = quant.quantize_blockwise(np.ascontiguousarray(go[:, I]), 128, 1, transpose_out=True)
    rqx, rsx = quant.quantize_blockwise(np.ascontiguousarray(x[:, J]), 128, 1, transpose_out=True)
    ref = gemm.linear_grad_weight(rqg, rsg, rqx, rsx, out_dtype=None)
    _assert_close(gw[np.ix_(I, J)], ref, "blockwise grad_weight 5120x8192x16640 sampled")


def test_full_grouped_moe_sampled():
    inp = workloads.grouped()
    act, W, offs = inp["act"], inp["W"], inp["offs"]
    E, N, K = W.shape
    qa, sa = fp8mm.fp8_quantize_rowwise(bf16_dev(act))
    qw, sw = fp8mm.fp8_quantize_rowwise(bf16_dev(W.reshape(E * N, K)))
    out = out_f64(fp8mm.fp8_scaled_grouped_mm(qa, qw.reshape(E, N, K), torch.from_numpy(offs).cuda(), sa,
                                              sw.reshape(E, N)))
    assert offs[-1] == act.shape[0]
    rows = _sample(act.shape[0], 96, 9)
    cols = _sample(N, 64, 10)
    expert = np.searchsorted(offs, rows, side="right")
    ra, rsa = quant.quantize_rowwise(act[rows])
    got, ref = [], []
    for t, (r, e) in enumerate(zip(rows, expert)):
        rw, rsw = quant.quantize_rowwise(W[e][cols])
        ref.append(gemm.scaled_mm(ra[t:t + 1], rw, rsa[t:t + 1], "rowwise", rsw, "rowwise", out_dtype=None)[0])
        got.append(out[r, cols])
    _assert_close(np.array(got), np.array(ref), "grouped E=64 16384x1408x2048 sampled")


def _random_case(rng):
    """One seeded random GEMM: recipe pair, B layout, ragged sizes within the
    ABI's rules, output dtype and bias."""
    recipe = rng.choice(["tensorwise", "rowwise", "1x128_128x128", "1x128_128x1", "mxfp8"])
    layout = "NK" if recipe in ("mxfp8", "1x128_128x1") or rng.random() < 0.5 else "KN"
    blocked = recipe in ("1x128_128x128", "1x128_128x1", "mxfp8")
    M = int(rng.integers(1, 1500))
    K = int(rng.integers(1, 9)) * 128 if blocked else int(rng.integers(1, 64)) * 16
    if recipe == "1x128_128x128":
        N = int(rng.integers(1, 10)) * 128
    elif layout == "KN" or recipe == "1x128_128x1":
        N = int(rng.integers(1, 80)) * 16
    else:
        N = int(rng.integers(1, 1300))
    out_dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    with_bias = recipe in ("tensorwise", "rowwise") and rng.random() < 0.5
    return recipe, layout, M, N, K, out_dtype, with_bias


def test_random_shapes_sweep():
    """40 seeded random problems through every dispatch path the sizes reach
    (small problems, the streaming kernel with or without a row tail), each
    against the oracle on the same bf16 inputs."""
    rng = np.random.default_rng(20260101)
    for case in range(40):
        recipe, layout, M, N, K, out_dtype, with_bias = _random_case(rng)
        say(f"sweep {case}: {recipe} {layout} M={M} N={N} K={K} {out_dtype} bias={with_bias}")
        g = workloads.streams(1000 + case, 3)
        x = workloads.normal_bf16(g[0], (M, K))
        w = workloads.normal_bf16(g[1], (N, K), 0.02)            # logical [N, K]
        bias = workloads.normal_bf16(g[2], (N,), 0.5) if with_bias else None
        if recipe in ("tensorwise", "rowwise"):
            qa, sa, ra, rsa = _quant_both(x, recipe)
            qb, sb, rb, rsb = _quant_both(w, recipe)
            rec_a = rec_b = recipe
            if layout == "KN":                                   # codes stored [K, N], same scales
                qb, rb = qb.t().contiguous(), np.ascontiguousarray(rb.T)
            if recipe == "rowwise":
                sa, sb = sa.reshape(-1), sb.reshape(-1)
        elif recipe == "1x128_128x128":
            qa, sa, ra, rsa = _quant_both(x, "1x128")
            stored = w if layout == "NK" else np.ascontiguousarray(w.T)
            qb, sb, rb, rsb = _quant_both(stored, "128x128")
            rec_a, rec_b = "1x128", "128x128"
        elif recipe == "1x128_128x1":
            qa, sa, ra, rsa = _quant_both(x, "1x128")
            qb, sb, rb, rsb = _quant_both(np.ascontiguousarray(w.T), "128x1", transpose_out=True)
            rec_a, rec_b = "1x128", "128x1"
        else:
            qa, sa = fp8mm.fp8_quantize_mx(bf16_dev(x))
            qb, sb = fp8mm.fp8_quantize_mx(bf16_dev(w))
            ra, rsa = mx.quantize_mx(x)
            rb, rsb = mx.quantize_mx(w)
            rec_a = rec_b = "mxfp8"
        out = fp8mm.fp8_scaled_mm(qa, qb, sa, rec_a, sb, rec_b, b_layout=layout, out_dtype=out_dtype,
                                  bias=None if bias is None else bf16_dev(bias))
        ref = gemm.scaled_mm(ra, rb, rsa, rec_a, rsb, rec_b, layout,
                             bias=None if bias is None else quant.bf16_to_f32(bias), out_dtype=None)
        _assert_close(out_f64(out), ref, f"sweep {case} {recipe} {layout} {M}x{N}x{K}",
                      out_dtype="bf16" if out_dtype == torch.bfloat16 else "fp32")
