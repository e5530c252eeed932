"""GPU parity of the grouped (MoE) variants against the CPU oracle: the
grouped GEMM with explicit recipes (rowwise and 1x128 x 128x128, expert
weights read [N, K] or [K, N]), the per-expert 128x1 quantizer (bit-exact)
and the per-expert weight gradient.

The GPU and the oracle quantize the same seeded bf16 inputs independently.
GEMM bar as for the dense GEMMs: relative Frobenius error <= 1e-3 and
elementwise |err| <= 4e-3 * max|ref| against the float64 oracle rounded once
to the output dtype.
"""

import numpy as np
import pytest
import torch

import precision_matmul_amd as fp8mm
import workloads
from oracle import gemm, quant
from tests.gpu_util import TOL_FRO, TOL_MAX, bf16_dev, host, out_f64, say

pytestmark = pytest.mark.gpu


def _assert_close(got, ref_exact, what, out_dtype="bf16"):
    rel_f, rel_m = gemm.parity(got, ref_exact, out_dtype)
    say(f"{what}: rel_fro={rel_f:.3e} rel_max={rel_m:.3e}")
    assert np.all(np.isfinite(got)), what
    assert rel_f <= TOL_FRO and rel_m <= TOL_MAX, (what, rel_f, rel_m)


def _offs_dev(offs):
    return torch.from_numpy(np.asarray(offs, np.int32)).cuda()


def _quant_block(bits, block):
    q, s = fp8mm.fp8_quantize_blockwise(bf16_dev(bits), block)
    rq, rs = quant.quantize_blockwise(bits, *block)
    return q, s, rq, rs


def _grouped_blockwise_case(E, N, K, sizes, layout, seed, bias_form=None, out_dtype=torch.bfloat16):
    """bias_form: None, "shared" (bf16 [N], every expert) or "per_expert"
    (bf16 [E, N], row e for expert e)."""
    g = workloads.streams(seed, 3)
    M = int(np.sum(sizes))
    act = workloads.normal_bf16(g[0], (M + 5, K))                 # 5 trailing rows no expert owns
    shape = (E, N, K) if layout == "NK" else (E, K, N)
    W = workloads.normal_bf16(g[1], shape, 0.02)
    bias = None
    if bias_form is not None:
        bias = workloads.normal_bf16(g[2], (E, N) if bias_form == "per_expert" else (N,), 0.5)
    offs = np.cumsum(sizes).astype(np.int32)
    qa, sa, ra, rsa = _quant_block(act, (1, 128))
    qw, sw, rw, rsw = _quant_block(W.reshape(E * shape[1], shape[2]), (128, 128))
    grid = sw.shape[0] // E, sw.shape[1]
    say(f"grouped blockwise E={E} N={N} K={K} {layout} bias={bias_form} {out_dtype}")
    out = fp8mm.fp8_scaled_grouped_mm_v2(qa, qw.reshape(shape), _offs_dev(offs), sa, "1x128",
                                         sw.reshape((E,) + grid), "128x128", b_layout=layout,
                                         bias=None if bias is None else bf16_dev(bias),
                                         bias_per_expert=bias_form == "per_expert", out_dtype=out_dtype)
    ref, written = gemm.grouped_mm(ra, rw.reshape(shape), offs, rsa, rsw.reshape((E,) + grid),
                                   bias=None if bias is None else quant.bf16_to_f32(bias), out_dtype=None,
                                   recipe_a="1x128", recipe_b="128x128", layout=layout)
    got = out_f64(out)
    assert np.all(got[~written] == 0), "rows no expert owns must not be written"
    return got[written], ref[written]


@pytest.mark.parametrize("layout", ["NK", "KN"])
@pytest.mark.parametrize("E,N,K,sizes", [
    (8, 256, 512, [100, 0, 300, 1, 129, 0, 0, 256]),
    (3, 128, 256, [5, 260, 64]),                 # N = 128: B stored [K, N] takes 128 x 128 tiles
    (1, 384, 384, [333]),
    (16, 384, 1024, [300, 257, 256, 255, 1, 0, 512, 40, 290, 310, 222, 260, 275, 233, 249, 301]),
    (2, 512, 512, [700, 900]),                  # experts of 800 rows: the 256 x 256 streaming tiles
    (6, 1408, 512, [320, 321, 0, 640, 1, 319])])   # N = 1408: eight 176-column n-blocks; m-block edges
def test_grouped_blockwise(E, N, K, sizes, layout):
    got, ref = _grouped_blockwise_case(E, N, K, np.array(sizes), layout, seed=E + N + K)
    _assert_close(got, ref, f"grouped 1x128 x 128x128 E={E} N={N} K={K} {layout}")


def _many_experts_sizes():
    """150 experts (three 64-expert chunks of the offset scan): empty experts
    on both sides of the first chunk boundary, one of 700 rows (three
    320-row m-blocks) just before the second and a single row just after."""
    sizes = workloads.streams(150, 1)[0].integers(0, 300, size=150)
    sizes[[63, 64]] = 0
    sizes[127], sizes[128] = 700, 1
    return sizes


@pytest.mark.parametrize("layout", ["NK", "KN"])
def test_grouped_blockwise_more_than_64_experts(layout):
    """The offset scans carry from one chunk of 64 experts to the next: E =
    150 on the weight-streaming kernel (weights read [N, K]) and on the
    streaming kernel (read [K, N]), and E = 70 experts of 400-900 rows on the
    streaming kernel's long-tiles-first order."""
    got, ref = _grouped_blockwise_case(150, 256, 256, _many_experts_sizes(), layout, seed=151)
    _assert_close(got, ref, f"grouped blockwise E=150 {layout}")
    sizes = workloads.streams(70, 1)[0].integers(400, 900, size=70)
    got, ref = _grouped_blockwise_case(70, 256, 256, sizes, layout, seed=71)
    _assert_close(got, ref, f"grouped blockwise E=70, long experts, {layout}")


@pytest.mark.parametrize("K", [128, 32])
def test_grouped_rowwise_at_the_expert_limit(K):
    """E = 2^16, the most experts a grouped call accepts: every workgroup's
    offset scan runs over 1024 chunks of 64 experts.  About 300 random
    experts own 1-40 rows each, expert 0 five, expert 2^15 seven hundred (three
    m-blocks) and the last expert 33; the rest are empty.  K = 128 runs on the
    weight-streaming kernel, K = 32 (rows below its 128-byte loads) on the
    128 x 128 grouped tiles.  Only the owning experts' weights are read, so
    the others are zero; the oracle quantizes the owning experts' weight rows
    (rowwise scaling is per row)."""
    E, N = 1 << 16, 16
    g = workloads.streams(65536 + K, 4)
    sizes = np.zeros(E, np.int64)
    picked = g[0].choice(np.arange(1, E - 1), 300, replace=False)
    sizes[picked] = g[0].integers(1, 41, size=300)
    sizes[0], sizes[E // 2], sizes[E - 1] = 5, 700, 33
    owners = np.flatnonzero(sizes)
    M = int(sizes.sum())
    act = workloads.normal_bf16(g[1], (M, K))
    w_own = workloads.normal_bf16(g[2], (owners.size, N, K), 0.02)
    W = np.zeros((E, N, K), np.uint16)
    W[owners] = w_own
    offs = np.cumsum(sizes).astype(np.int32)
    say(f"grouped rowwise E={E} N={N} K={K} M_total={M}, {owners.size} experts with rows")
    qa, sa = fp8mm.fp8_quantize_rowwise(bf16_dev(act))
    qw, sw = fp8mm.fp8_quantize_rowwise(bf16_dev(W.reshape(E * N, K)))
    out = fp8mm.fp8_scaled_grouped_mm(qa, qw.reshape(E, N, K), _offs_dev(offs), sa, sw.reshape(E, N))
    ra, rsa = quant.quantize_rowwise(act)
    rq_own, rs_own = quant.quantize_rowwise(w_own.reshape(-1, K))
    rw = np.zeros((E, N, K), np.uint8)
    rw[owners] = rq_own.reshape(owners.size, N, K)
    rsw = np.ones((E, N), np.float32)
    rsw[owners] = rs_own.reshape(owners.size, N)
    ref, written = gemm.grouped_mm(ra, rw, offs, rsa, rsw, out_dtype=None)
    assert written.all()
    _assert_close(out_f64(out), ref, f"grouped rowwise E=2^16 K={K}")


def test_grouped_weight_gradient_more_than_64_experts():
    sizes = _many_experts_sizes()
    got, ref = _grouped_grad_weight_case(sizes, 128, 256, seed=152, out_dtype=torch.float32)
    for e in np.flatnonzero(sizes == 0):
        assert not got[e].any(), "an expert without tokens gets zeros"
    _assert_close(got, ref, "grouped grad_weight E=150", out_dtype="fp32")


@pytest.mark.parametrize("bias_form", ["shared", "per_expert"])
@pytest.mark.parametrize("layout", ["NK", "KN"])
def test_grouped_blockwise_bias_fp32(layout, bias_form):
    """Both bias forms of the grouped call: one [N] row added to every
    expert's rows, or [E, N] with row e for expert e."""
    got, ref = _grouped_blockwise_case(5, 256, 256, np.array([70, 0, 200, 3, 90]), layout, seed=5,
                                       bias_form=bias_form, out_dtype=torch.float32)
    _assert_close(got, ref, f"grouped blockwise bias ({bias_form}) fp32 {layout}", out_dtype="fp32")


@pytest.mark.parametrize("N", [128, 384])
def test_grouped_rowwise_weights_stored_kn(N):
    """Rowwise x rowwise with expert weights read [K, N] (scale_b per output
    column of each expert)."""
    E, K = 4, 256
    sizes = np.array([40, 0, 150, 66])
    g = workloads.streams(N + 11, 2)
    act = workloads.normal_bf16(g[0], (int(sizes.sum()), K))
    W = workloads.normal_bf16(g[1], (E, N, K), 0.02)              # logical [N, K] per expert
    offs = np.cumsum(sizes).astype(np.int32)
    qa, sa = fp8mm.fp8_quantize_rowwise(bf16_dev(act))
    ra, rsa = quant.quantize_rowwise(act)
    qw, sw = fp8mm.fp8_quantize_rowwise(bf16_dev(W.reshape(E * N, K)))
    rw, rsw = quant.quantize_rowwise(W.reshape(E * N, K))
    qw_kn = qw.reshape(E, N, K).transpose(1, 2).contiguous()      # stored [E, K, N]
    rw_kn = np.ascontiguousarray(rw.reshape(E, N, K).transpose(0, 2, 1))
    out = fp8mm.fp8_scaled_grouped_mm_v2(qa, qw_kn, _offs_dev(offs), sa.reshape(-1), "rowwise",
                                         sw.reshape(-1), "rowwise", b_layout="KN")
    ref, written = gemm.grouped_mm(ra, rw_kn, offs, rsa, rsw.reshape(E, N), out_dtype=None, layout="KN")
    _assert_close(out_f64(out)[written], ref[written], f"grouped rowwise KN N={N}")


@pytest.mark.parametrize("N,ld_pad,out_dtype,K", [(406, 0, torch.bfloat16, 384), (406, 10, torch.bfloat16, 384),
                                                    (406, 2, torch.float32, 384), (512, 0, torch.float32, 384),
                                                    (406, 10, torch.bfloat16, 400)])
def test_grouped_rowwise_short_remainders(N, ld_pad, out_dtype, K):
    """Experts whose last m-tile holds 1 to 64 rows or 65 to 128 rows (the
    two short-tile layouts: all waves on a 64 x 256 or 128 x 256 block), next
    to full tiles; N = 406 ends
    the last 256-column tile after 150 columns (a lane's group of four partly
    outside it); out with ld = N or padded (16-byte vector stores where the
    padding aligns every row); a bias shared by the experts ([N]); K = 400
    ends the last K step after 16 of its 128 bytes."""
    sizes = np.array([256 + 1, 64, 0, 256 + 63, 65, 17, 256, 256 + 40, 3, 256 + 100, 128, 97])
    E = len(sizes)
    g = workloads.streams(N + ld_pad + K, 3)
    M = int(sizes.sum())
    act = workloads.normal_bf16(g[0], (M + 4, K))                 # 4 trailing rows no expert owns
    W = workloads.normal_bf16(g[1], (E * N, K), 0.02)
    bias = workloads.normal_bf16(g[2], (N,), 0.5)
    offs = np.cumsum(sizes).astype(np.int32)
    qa, sa = fp8mm.fp8_quantize_rowwise(bf16_dev(act))
    ra, rsa = quant.quantize_rowwise(act)
    qw, sw = fp8mm.fp8_quantize_rowwise(bf16_dev(W))
    rw, rsw = quant.quantize_rowwise(W)
    full = torch.zeros((M + 4, N + ld_pad), dtype=out_dtype, device="cuda")
    out = full[:, :N]
    say(f"grouped rowwise short remainders N={N} K={K} ld={N + ld_pad} {out_dtype}")
    fp8mm.fp8_scaled_grouped_mm(qa, qw.reshape(E, N, K), _offs_dev(offs), sa.reshape(-1), sw.reshape(E, N),
                                bias=bf16_dev(bias), out_dtype=out_dtype, out=out)
    ref, written = gemm.grouped_mm(ra, rw.reshape(E, N, K), offs, rsa, rsw.reshape(E, N),
                                   bias=quant.bf16_to_f32(bias), out_dtype=None)
    got = out_f64(full)
    assert np.all(got[:, N:] == 0), "columns past N must not be written"
    assert np.all(got[:, :N][~written] == 0), "rows no expert owns must not be written"
    _assert_close(got[:, :N][written], ref[written], f"grouped rowwise short N={N}",
                  out_dtype="fp32" if out_dtype == torch.float32 else "bf16")


def test_grouped_out_argument_is_checked():
    E, N, K = 2, 128, 128
    qa = torch.zeros((10, K), dtype=torch.uint8, device="cuda")
    qw = torch.zeros((E, N, K), dtype=torch.uint8, device="cuda")
    sa = torch.ones(10, device="cuda")
    sw = torch.ones(E * N, device="cuda")
    offs = _offs_dev([4, 10])
    for out in (torch.zeros((10, N), dtype=torch.bfloat16, device="cuda"),     # dtype: fp32 asked
                torch.zeros((9, N), dtype=torch.float32, device="cuda")):       # shape
        with pytest.raises(ValueError):
            fp8mm.fp8_scaled_grouped_mm(qa, qw, offs, sa, sw.reshape(E, N), out_dtype=torch.float32, out=out)
        with pytest.raises(ValueError):
            fp8mm.fp8_scaled_grouped_mm_v2(qa, qw, offs, sa, "rowwise", sw, "rowwise", out_dtype=torch.float32,
                                           out=out)


def test_grouped_v2_rowwise_matches_v1():
    E, N, K = 6, 256, 384
    sizes = np.array([10, 200, 0, 31, 128, 77])
    g = workloads.streams(41, 2)
    act = workloads.normal_bf16(g[0], (int(sizes.sum()), K))
    W = workloads.normal_bf16(g[1], (E * N, K), 0.02)
    qa, sa = fp8mm.fp8_quantize_rowwise(bf16_dev(act))
    qw, sw = fp8mm.fp8_quantize_rowwise(bf16_dev(W))
    offs = _offs_dev(np.cumsum(sizes))
    v1 = fp8mm.fp8_scaled_grouped_mm(qa, qw.reshape(E, N, K), offs, sa.reshape(-1), sw.reshape(E, N))
    v2 = fp8mm.fp8_scaled_grouped_mm_v2(qa, qw.reshape(E, N, K), offs, sa.reshape(-1), "rowwise",
                                        sw.reshape(-1), "rowwise")
    assert torch.equal(v1, v2)


def test_grouped_blockwise_full_moe_shape_sampled():
    """E = 64, 16384 tokens, N = 1408, K = 2048 (the grouped MoE shape) in the
    blockwise recipe, forward ([N, K] weights) and input gradient (the same
    weights read [K, N]); 48 sampled rows (all of their columns)."""
    inp = workloads.grouped()
    act, W, offs = inp["act"], inp["W"], inp["offs"]
    E, N, K = W.shape
    M = act.shape[0]
    qa, sa = fp8mm.fp8_quantize_blockwise(bf16_dev(act), (1, 128))
    qw, sw = fp8mm.fp8_quantize_blockwise(bf16_dev(W.reshape(E * N, K)), (128, 128))
    od = _offs_dev(offs)
    say("grouped blockwise 16384x1408x2048 E=64 forward")
    out = out_f64(fp8mm.fp8_scaled_grouped_mm_v2(qa, qw.reshape(E, N, K), od, sa, "1x128",
                                                 sw.reshape(E, N // 128, K // 128), "128x128"))
    rows = np.sort(np.random.default_rng(7).choice(M, 48, replace=False))
    experts = np.searchsorted(offs, rows, side="right")
    rq, rs = quant.quantize_blockwise(act[rows], 1, 128)            # 1x128 groups are row-local
    got, ref = [], []
    for t, (i, e) in enumerate(zip(rows, experts)):
        wq, ws = quant.quantize_blockwise(W[e], 128, 128)
        ref.append(gemm.scaled_mm_exact(rq[t:t + 1], wq, rs[:, t:t + 1], "1x128", ws, "128x128")[0])
        got.append(out[i])
    _assert_close(np.array(got), np.array(ref), "grouped blockwise MoE shape sampled")


def test_grouped_blockwise_input_gradient_moe_shape_sampled():
    """Input gradient of the grouped MoE layer: grad_output [16384, 1408]
    (1x128) times each expert's stored [1408, 2048] weight read [K, N]."""
    inp = workloads.grouped_backward()
    go, W, offs = inp["grad_output"], inp["W"], inp["offs"]
    E, Nw, Kw = W.shape                      # contraction over Nw = 1408, output width Kw = 2048
    M = go.shape[0]
    qg, sg = fp8mm.fp8_quantize_blockwise(bf16_dev(go), (1, 128))
    qw, sw = fp8mm.fp8_quantize_blockwise(bf16_dev(W.reshape(E * Nw, Kw)), (128, 128))
    say("grouped blockwise input gradient 16384x2048x1408 E=64")
    out = out_f64(fp8mm.fp8_scaled_grouped_mm_v2(qg, qw.reshape(E, Nw, Kw), _offs_dev(offs), sg, "1x128",
                                                 sw.reshape(E, Nw // 128, Kw // 128), "128x128", b_layout="KN"))
    rows = np.sort(np.random.default_rng(8).choice(M, 48, replace=False))
    experts = np.searchsorted(offs, rows, side="right")
    rq, rs = quant.quantize_blockwise(go[rows], 1, 128)
    got, ref = [], []
    for t, (i, e) in enumerate(zip(rows, experts)):
        wq, ws = quant.quantize_blockwise(W[e], 128, 128)
        ref.append(gemm.scaled_mm_exact(rq[t:t + 1], wq, rs[:, t:t + 1], "1x128", ws, "128x128", layout="KN")[0])
        got.append(out[i])
    _assert_close(np.array(got), np.array(ref), "grouped blockwise input gradient sampled")


# ------------------------------------------------------ grouped weight gradient

def _check_grouped_quant(bits, offs):
    q, s = fp8mm.fp8_quantize_grouped_128x1(bf16_dev(bits), _offs_dev(offs))
    rq, rs, _ = quant.quantize_grouped_128x1(bits, offs)
    nb = rs.shape[0]
    gq, gs = host(q), host(s)
    assert np.array_equal(gq[:, :128 * nb], rq), "grouped 128x1 codes"
    assert np.array_equal(gs[:nb], rs), "grouped 128x1 scales"
    return q, s, rq, rs


@pytest.mark.parametrize("sizes,C", [
    ([130, 5, 0, 257, 1, 128, 0, 300], 64),
    ([0, 0, 0], 32),
    ([1000], 48),
    ([128] * 9, 256)])
def test_grouped_128x1_quant_bit_exact(sizes, C):
    offs = np.cumsum(sizes).astype(np.int32)
    T = int(offs[-1]) + 3                                       # 3 trailing rows no expert owns
    x = workloads.normal_bf16(workloads.streams(len(sizes) + C, 1)[0], (T, C), 2.0)
    say(f"grouped 128x1 quant sizes={sizes} C={C}")
    _check_grouped_quant(x, offs)


def _grouped_grad_weight_case(sizes, N_out, K_in, seed, out_dtype):
    offs = np.cumsum(sizes).astype(np.int32)
    T = int(offs[-1]) + 2
    g = workloads.streams(seed, 2)
    go = workloads.normal_bf16(g[0], (T, N_out), 1e-3)
    x = workloads.normal_bf16(g[1], (T, K_in))
    qg, sg, rqg, rsg = _check_grouped_quant(go, offs)
    qx, sx, rqx, rsx = _check_grouped_quant(x, offs)
    say(f"grouped grad_weight sizes={list(sizes)} N_out={N_out} K_in={K_in} {out_dtype}")
    out = fp8mm.fp8_grouped_linear_grad_weight(qg, sg, qx, sx, _offs_dev(offs), T, out_dtype=out_dtype)
    ref = gemm.grouped_grad_weight(rqg, rsg, rqx, rsx, offs, out_dtype=None)
    return out_f64(out), ref


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("sizes,N_out,K_in", [
    ([130, 0, 5, 257, 128, 1], 256, 384),
    ([40, 90], 208, 144),                      # ragged output tiles
    ([700], 128, 128),
    ([3] * 20, 64, 256)])
def test_grouped_weight_gradient(sizes, N_out, K_in, out_dtype):
    got, ref = _grouped_grad_weight_case(np.array(sizes), N_out, K_in, seed=N_out + K_in, out_dtype=out_dtype)
    od = "bf16" if out_dtype == torch.bfloat16 else "fp32"
    for e, m in enumerate(sizes):
        if m == 0:
            assert not got[e].any(), "an expert without tokens gets zeros"
    _assert_close(got, ref, f"grouped grad_weight {sizes} {N_out}x{K_in}", out_dtype=od)


def test_grouped_weight_gradient_moe_shape():
    """E = 64 experts over 16384 tokens, grad_output [16384, 1408], input
    [16384, 2048]: the quantizer on the full shape (bit-exact) and the
    gradients of 6 experts in full."""
    inp = workloads.grouped_backward()
    go, x, offs = inp["grad_output"], inp["act"], inp["offs"]
    T = go.shape[0]
    say("grouped 128x1 quant + grad_weight, MoE shape")
    qg, sg, rqg, rsg = _check_grouped_quant(go, offs)
    qx, sx, rqx, rsx = _check_grouped_quant(x, offs)
    out = out_f64(fp8mm.fp8_grouped_linear_grad_weight(qg, sg, qx, sx, _offs_dev(offs), T))
    assert out.shape == (64, 1408, 2048)
    pick = [0, 1, 17, 40, 62, 63]
    sizes = np.diff(np.concatenate([[0], offs]))
    # the oracle on the picked experts only: the same runs, the other experts emptied
    keep = np.zeros(64, bool)
    keep[pick] = True
    sub = np.cumsum(np.where(keep, sizes, 0)).astype(np.int32)
    starts = np.concatenate([[0], offs[:-1]])
    rows = np.concatenate([np.arange(starts[e], offs[e]) for e in pick])
    rqg2, rsg2, _ = quant.quantize_grouped_128x1(go[rows], sub)
    rqx2, rsx2, _ = quant.quantize_grouped_128x1(x[rows], sub)
    ref = gemm.grouped_grad_weight(rqg2, rsg2, rqx2, rsx2, sub, out_dtype=None)
    _assert_close(out[pick], ref[pick], "grouped grad_weight MoE shape, 6 experts")


def test_grouped_all_experts_empty():
    """Offsets all zero: the grouped GEMM writes no row, the per-expert
    weight gradient writes zeros for every expert, the quantizer no run."""
    E, N, K, T = 4, 256, 256, 37
    g = workloads.streams(99, 3)
    act = workloads.normal_bf16(g[0], (T, K))
    W = workloads.normal_bf16(g[1], (E, N, K), 0.02)
    go = workloads.normal_bf16(g[2], (T, N), 1e-3)
    offs = _offs_dev(np.zeros(E, np.int32))
    qa, sa = fp8mm.fp8_quantize_blockwise(bf16_dev(act), (1, 128))
    qw, sw = fp8mm.fp8_quantize_blockwise(bf16_dev(W.reshape(E * N, K)), (128, 128))
    out = torch.full((T, N), 3.0, dtype=torch.bfloat16, device="cuda")
    fp8mm.fp8_scaled_grouped_mm_v2(qa, qw.view(E, N, K), offs, sa, "1x128", sw.view(E, N // 128, K // 128),
                                   "128x128", out=out)
    assert bool((out == 3.0).all()), "no row belongs to an expert"
    qg, sg = fp8mm.fp8_quantize_grouped_128x1(bf16_dev(go), offs)
    qx, sx = fp8mm.fp8_quantize_grouped_128x1(bf16_dev(act), offs)
    gw = fp8mm.fp8_grouped_linear_grad_weight(qg, sg, qx, sx, offs, T, out_dtype=torch.float32)
    assert gw.shape == (E, N, K) and not bool(gw.any())


def test_grouped_weight_gradient_runs_of_exactly_128_and_single_tokens():
    got, ref = _grouped_grad_weight_case(np.array([128, 1, 256, 0, 1, 127]), 128, 256, seed=5,
                                         out_dtype=torch.bfloat16)
    assert not got[3].any()
    _assert_close(got, ref, "grouped grad_weight whole and single-token runs")


@pytest.mark.parametrize("sizes,C", [([130, 5, 0, 257, 1, 128, 0, 300], 128), ([700, 40], 256), ([0, 0], 128)])
def test_grouped_dual_quant_bit_exact(sizes, C):
    """One read, both layouts: the 1x128 codes of every owned row and the
    per-expert runs, each bit-exact against the oracle."""
    offs = np.cumsum(sizes).astype(np.int32)
    T = int(offs[-1]) + 3                                       # 3 trailing rows no expert owns
    x = workloads.normal_bf16(workloads.streams(len(sizes) + 7 * C, 1)[0], (T, C), 2.0)
    say(f"grouped dual quant sizes={sizes} C={C}")
    q_row, s_row, q_t, s_t = fp8mm.fp8_quantize_grouped_dual(bf16_dev(x), _offs_dev(offs))
    M = int(offs[-1])
    if M:
        rq, rs = quant.quantize_blockwise(x[:M], 1, 128)
        assert np.array_equal(host(q_row)[:M], rq), "1x128 codes of the owned rows"
        assert np.array_equal(host(s_row)[:, :M], rs), "1x128 scales of the owned rows"
    rq, rs, _ = quant.quantize_grouped_128x1(x, offs)
    nb = rs.shape[0]
    assert np.array_equal(host(q_t)[:, :128 * nb], rq), "runs"
    assert np.array_equal(host(s_t)[:nb], rs), "run scales"


def test_grouped_random_sweep():
    """Seeded random grouped problems: expert count and sizes (empty experts
    included), recipe, weight layout, N and K within the ABI's rules; the
    grouped GEMM and the per-expert weight gradient against the oracle."""
    rng = np.random.default_rng(20260202)
    for case in range(16):
        E = int(rng.integers(1, 13))
        sizes = rng.integers(0, 400, size=E) * (rng.random(E) > 0.2)
        blockwise = bool(rng.random() < 0.5)
        layout = "NK" if rng.random() < 0.5 else "KN"
        K = int(rng.integers(1, 7)) * 128
        N = int(rng.integers(1, 5)) * 128 if blockwise else int(rng.integers(1, 40)) * 16
        say(f"grouped sweep {case}: E={E} sizes={[int(v) for v in sizes]} {'blockwise' if blockwise else 'rowwise'} "
            f"{layout} N={N} K={K}")
        if blockwise:
            got, ref = _grouped_blockwise_case(E, N, K, np.array(sizes), layout, seed=300 + case)
        else:
            offs = np.cumsum(sizes).astype(np.int32)
            g = workloads.streams(300 + case, 2)
            act = workloads.normal_bf16(g[0], (int(offs[-1]) + 2, K))
            W = workloads.normal_bf16(g[1], (E * N, K), 0.02)
            qa, sa = fp8mm.fp8_quantize_rowwise(bf16_dev(act))
            ra, rsa = quant.quantize_rowwise(act)
            qw, sw = fp8mm.fp8_quantize_rowwise(bf16_dev(W))
            rw, rsw = quant.quantize_rowwise(W)
            qwe, rwe = qw.view(E, N, K), rw.reshape(E, N, K)
            if layout == "KN":
                qwe, rwe = qwe.transpose(1, 2).contiguous(), np.ascontiguousarray(rwe.transpose(0, 2, 1))
            out = fp8mm.fp8_scaled_grouped_mm_v2(qa, qwe, _offs_dev(offs), sa.reshape(-1), "rowwise",
                                                 sw.reshape(-1), "rowwise", b_layout=layout)
            ref, written = gemm.grouped_mm(ra, rwe, offs, rsa, rsw.reshape(E, N), out_dtype=None, layout=layout)
            g_all = out_f64(out)
            assert not g_all[~written].any()
            got, ref = g_all[written], ref[written]
        if got.size:
            _assert_close(got, ref, f"grouped sweep {case}")
        # the per-expert weight gradient on the same routing
        N_out, K_in = int(rng.integers(1, 20)) * 16, int(rng.integers(1, 20)) * 16
        gw, rgw = _grouped_grad_weight_case(np.array(sizes), N_out, K_in, seed=400 + case,
                                            out_dtype=torch.float32 if case % 2 else torch.bfloat16)
        for e, m in enumerate(sizes):
            if m == 0:
                assert not gw[e].any()
        if np.abs(rgw).max() > 0:
            _assert_close(gw, rgw, f"grouped grad_weight sweep {case}", out_dtype="fp32" if case % 2 else "bf16")
