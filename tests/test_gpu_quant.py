"""GPU parity of the quantization kernels: codes and scales bit-exact against
the CPU oracle, through the C ABI (Python binding)."""

import numpy as np
import pytest
import torch

import precision_matmul_amd as fp8mm
import workloads
from oracle import e4m3, mx, quant
from tests.gpu_util import bf16_dev, host, say

pytestmark = pytest.mark.gpu


def _check(q_gpu, s_gpu, q_ref, s_ref, what):
    qg, sg = host(q_gpu), host(s_gpu)
    assert qg.shape == q_ref.shape, (what, qg.shape, q_ref.shape)
    assert sg.reshape(-1).shape == s_ref.reshape(-1).shape, (what, sg.shape, s_ref.shape)
    bad_s = np.flatnonzero(sg.reshape(-1).view(np.uint32) != s_ref.reshape(-1).view(np.uint32))
    assert bad_s.size == 0, (what, "scales differ at", bad_s[:8], sg.reshape(-1)[bad_s[:4]], s_ref.reshape(-1)[bad_s[:4]])
    bad = np.argwhere(qg != q_ref)
    assert bad.size == 0, (what, "codes differ at", bad[:8], qg[tuple(bad[0])], q_ref[tuple(bad[0])])


def _special_rows(ncols):
    """Rows whose amax is 448 (scale exactly 1): every E4M3 midpoint, its bf16
    neighbours and the subnormal range pass through the cast unchanged."""
    t = e4m3.decode_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    vals = np.concatenate([mids, t, np.array([2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 1e-30, 0.0])])
    v32 = vals.astype(np.float32)
    bits = workloads.f32_to_bf16_bits(v32).astype(np.int32)
    cand = np.concatenate([bits, bits + 1, bits - 1, bits | 0x8000])
    cand = cand[(cand >= 0) & (cand < 0x10000)].astype(np.uint16)
    mag = quant.bf16_to_f32(cand)
    cand = cand[np.isfinite(mag) & (np.abs(mag) <= 448.0)]
    rows = []
    for i in range(0, cand.size, ncols - 1):
        chunk = cand[i:i + ncols - 1]
        row = np.zeros(ncols, np.uint16)
        row[:chunk.size] = chunk
        row[-1] = workloads.f32_to_bf16_bits(np.array([448.0], np.float32))[0]
        rows.append(row)
    return np.stack(rows)


@pytest.mark.parametrize("rows,cols", [(8, 4096), (37, 1040), (5, 16), (3, 8704), (64, 8192)])
def test_rowwise_bitexact(rows, cols):
    say(f"rowwise {rows}x{cols}")
    x = workloads.rowwise(M=rows, N=16, K=cols)["x"]
    q, s = fp8mm.fp8_quantize_rowwise(bf16_dev(x))
    rq, rs = quant.quantize_rowwise(x)
    _check(q, s, rq, rs, f"rowwise {rows}x{cols}")


def test_rowwise_midpoints_ties_subnormals_and_tiny_rows():
    x = _special_rows(512)
    tiny = workloads.f32_to_bf16_bits(np.array([[1e-9] * 512, [0.0] * 512, [-3e-38] * 512], np.float32))
    x = np.concatenate([x, tiny, (x[:2] | 0x8000).astype(np.uint16)])
    q, s = fp8mm.fp8_quantize_rowwise(bf16_dev(x))
    rq, rs = quant.quantize_rowwise(x)
    _check(q, s, rq, rs, "rowwise specials")
    q, s = fp8mm.fp8_quantize_rowwise(bf16_dev(x), eps=0.0)
    rq, rs = quant.quantize_rowwise(x, eps=0.0)
    _check(q, s, rq, rs, "rowwise specials eps=0")


@pytest.mark.parametrize("rows,cols", [(256, 256), (100, 48), (1, 16), (384, 1024)])
def test_tensorwise_bitexact(rows, cols):
    say(f"tensorwise {rows}x{cols}")
    x = workloads.tensorwise(n=cols, m=rows, k=cols)["A"][:rows, :cols]
    q, s = fp8mm.fp8_quantize_tensorwise(bf16_dev(x))
    rq, rs = quant.quantize_tensorwise(x)
    _check(q, s, rq, rs, f"tensorwise {rows}x{cols}")


def test_tensorwise_specials_tiny_scale_and_empty():
    x = _special_rows(256)
    q, s = fp8mm.fp8_quantize_tensorwise(bf16_dev(x))
    rq, rs = quant.quantize_tensorwise(x)
    _check(q, s, rq, rs, "tensorwise specials")
    # amax ~1e-30: the scale is below 2^-90 and takes the plain division path
    rng = np.random.default_rng(3)
    tiny = workloads.f32_to_bf16_bits((rng.standard_normal((64, 128)) * 1e-30).astype(np.float32))
    q, s = fp8mm.fp8_quantize_tensorwise(bf16_dev(tiny))
    rq, rs = quant.quantize_tensorwise(tiny)
    _check(q, s, rq, rs, "tensorwise tiny")
    z = np.zeros((32, 64), np.uint16)
    z[3:] = 0x8000
    q, s = fp8mm.fp8_quantize_tensorwise(bf16_dev(z))
    rq, rs = quant.quantize_tensorwise(z)
    _check(q, s, rq, rs, "tensorwise zeros")
    q, s = fp8mm.fp8_quantize_tensorwise(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"))
    assert q.shape == (0, 64) and host(s).reshape(-1)[0] == 1.0


_BLOCK_CASES = [((1, 128), 257, 1024), ((1, 128), 16, 128), ((1, 128), 33, 640),
                ((128, 128), 384, 512), ((128, 128), 128, 128),
                ((128, 1), 256, 384), ((128, 1), 128, 144), ((128, 1), 384, 16)]


# transpose_out exists for (128, 1) only
@pytest.mark.parametrize("block,rows,cols,transpose",
                         [c + (False,) for c in _BLOCK_CASES] + [c + (True,) for c in _BLOCK_CASES if c[0] == (128, 1)])
def test_blockwise_bitexact(block, rows, cols, transpose):
    say(f"blockwise {block} {rows}x{cols} T={transpose}")
    rng = np.random.default_rng(rows * 7 + cols)
    x = workloads.f32_to_bf16_bits((rng.standard_normal((rows, cols)) *
                                    np.exp2(rng.integers(-20, 20, size=(rows, 1)))).astype(np.float32))
    q, s = fp8mm.fp8_quantize_blockwise(bf16_dev(x), block, transpose_out=transpose)
    rq, rs = quant.quantize_blockwise(x, block[0], block[1], transpose_out=transpose)
    _check(q, s, rq, rs, f"blockwise {block} {rows}x{cols} T={transpose}")


def test_blockwise_specials():
    x = _special_rows(128)
    x = np.concatenate([x, np.zeros(((-x.shape[0]) % 128, 128), np.uint16)])
    for block in ((1, 128), (128, 128), (128, 1)):
        q, s = fp8mm.fp8_quantize_blockwise(bf16_dev(x), block)
        rq, rs = quant.quantize_blockwise(x, *block)
        _check(q, s, rq, rs, f"specials {block}")


def _every_bf16_under(amax_bits):
    """A [128, 4096] bf16 block whose every row, 128-column group, 128-row
    column group and 128x128 block has amax exactly bf16(amax_bits): row 0 and
    column 0 of each 128-column group hold the amax, and the other slots hold
    every finite bf16 pattern of magnitude <= amax (both signs), cycled."""
    amax = quant.bf16_to_f32(np.array([amax_bits], np.uint16))[0]
    pats = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    mag = quant.bf16_to_f32(pats)
    pats = pats[np.isfinite(mag) & (np.abs(mag) <= amax)]
    x = np.full((128, 4096), amax_bits, np.uint16)
    slots = np.ones((128, 4096), bool)
    slots[0, :] = False
    slots[:, ::128] = False
    n = int(slots.sum())
    assert pats.size <= n
    x[slots] = np.resize(pats, n)
    return x


def test_every_bf16_value_at_several_scales():
    """Exhaustive over the bf16 inputs: for each amax (scale amax/448 exactly
    1, a power of two, an awkward ratio, large, tiny and below 2^-90), every
    bf16 value that the amax admits goes through each quantizer's cast and
    must give the oracle's code."""
    amaxes = [448.0, 1.0, 3.140625, 61440.0, 2.0 ** -20, 1e-30]
    bits = workloads.f32_to_bf16_bits(np.array(amaxes, np.float32))
    blocks = [_every_bf16_under(int(b)) for b in bits]
    for b, blk in zip(amaxes, blocks):
        say(f"tensorwise every bf16 under {b}")
        q, s = fp8mm.fp8_quantize_tensorwise(bf16_dev(blk))
        rq, rs = quant.quantize_tensorwise(blk)
        _check(q, s, rq, rs, f"tensorwise every bf16 under {b}")
    x = np.concatenate(blocks)
    say("rowwise / blockwise every bf16")
    q, s = fp8mm.fp8_quantize_rowwise(bf16_dev(x), eps=0.0)
    rq, rs = quant.quantize_rowwise(x, eps=0.0)
    _check(q, s, rq, rs, "rowwise every bf16")
    for block in ((1, 128), (128, 128), (128, 1)):
        for transpose in ([False, True] if block == (128, 1) else [False]):
            q, s = fp8mm.fp8_quantize_blockwise(bf16_dev(x), block, transpose_out=transpose)
            rq, rs = quant.quantize_blockwise(x, *block, transpose_out=transpose)
            _check(q, s, rq, rs, f"every bf16 {block} T={transpose}")


def test_every_bf16_value_at_64_random_scales():
    """The same exhaustive inputs at 64 seeded random amax values (exponent
    and mantissa uniform over the finite bf16 range, so the scales reach from
    the IEEE-division range below 2^-90 to ~1e35), through the rowwise
    (with and without its epsilon) and blockwise quantizers: 33.5 M values,
    every code against the oracle's table encoder."""
    rng = np.random.default_rng(20260064)
    bits = [(int(rng.integers(1, 255)) << 7) | int(rng.integers(0, 128)) for _ in range(64)]
    x = np.concatenate([_every_bf16_under(b) for b in bits])
    say(f"every bf16 at 64 random scales: {x.shape}")
    xd = bf16_dev(x)
    for eps in (0.0, None):
        q, s = fp8mm.fp8_quantize_rowwise(xd) if eps is None else fp8mm.fp8_quantize_rowwise(xd, eps=eps)
        rq, rs = quant.quantize_rowwise(x) if eps is None else quant.quantize_rowwise(x, eps=eps)
        _check(q, s, rq, rs, f"rowwise every bf16, 64 scales, eps={eps}")
    for block in ((1, 128), (128, 128), (128, 1)):
        q, s = fp8mm.fp8_quantize_blockwise(xd, block)
        rq, rs = quant.quantize_blockwise(x, *block)
        _check(q, s, rq, rs, f"every bf16, 64 scales, {block}")


@pytest.mark.parametrize("rows,cols", [(128, 128), (256, 384), (384, 1024)])
def test_dual_layout_quantize_bitexact(rows, cols):
    """One read of grad_output, both backward operands: 1x128 row codes and
    128x1 codes written transposed, each equal to the oracle's."""
    say(f"dual {rows}x{cols}")
    rng = np.random.default_rng(rows * 3 + cols)
    x = workloads.f32_to_bf16_bits((rng.standard_normal((rows, cols)) *
                                    np.exp2(rng.integers(-20, 20, size=(rows, 1)))).astype(np.float32))
    q_row, s_row, q_col, s_col = fp8mm.fp8_quantize_blockwise_dual(bf16_dev(x))
    rq, rs = quant.quantize_blockwise(x, 1, 128)
    _check(q_row, s_row, rq, rs, f"dual 1x128 {rows}x{cols}")
    rq, rs = quant.quantize_blockwise(x, 128, 1, transpose_out=True)
    _check(q_col, s_col, rq, rs, f"dual 128x1^T {rows}x{cols}")


def test_dual_layout_quantize_full_size_grad_output():
    """The grad_output of the weight-gradient workload, [16640, 5120] ~N(0,
    1e-3): the dual pass equals the two single-layout passes everywhere, and
    the oracle on a 256-row slab (two 128-token groups)."""
    g = workloads.grad_weight()["grad_output"]
    xd = bf16_dev(g)
    q_row, s_row, q_col, s_col = fp8mm.fp8_quantize_blockwise_dual(xd)
    a, sa = fp8mm.fp8_quantize_blockwise(xd, (1, 128))
    b, sb = fp8mm.fp8_quantize_blockwise(xd, (128, 1), transpose_out=True)
    assert torch.equal(q_row, a) and torch.equal(s_row, sa)
    assert torch.equal(q_col, b) and torch.equal(s_col, sb)
    slab = g[4096:4352]
    rq, rs = quant.quantize_blockwise(slab, 1, 128)
    _check(q_row[4096:4352], s_row[:, 4096:4352], rq, rs, "dual 1x128 slab")
    rq, rs = quant.quantize_blockwise(slab, 128, 1, transpose_out=True)
    _check(q_col[:, 4096:4352], s_col[32:34], rq, rs, "dual 128x1^T slab")


def _check_mx(q_gpu, s_gpu, q_ref, s_ref, what):
    qg, sg = host(q_gpu), host(s_gpu)
    assert qg.shape == q_ref.shape and sg.shape == s_ref.shape, (what, qg.shape, sg.shape)
    bad_s = np.argwhere(sg != s_ref)
    assert bad_s.size == 0, (what, "scale bytes differ at", bad_s[:8], sg[tuple(bad_s[0])], s_ref[tuple(bad_s[0])])
    bad = np.argwhere(qg != q_ref)
    assert bad.size == 0, (what, "codes differ at", bad[:8], qg[tuple(bad[0])], q_ref[tuple(bad[0])])


@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 96), (256, 1024), (64, 8192)])
def test_mx_quantize_bitexact(rows, cols):
    say(f"mx {rows}x{cols}")
    rng = np.random.default_rng(rows * 5 + cols)
    x = workloads.f32_to_bf16_bits((rng.standard_normal((rows, cols)) *
                                    np.exp2(rng.integers(-60, 60, size=(rows, 1)))).astype(np.float32))
    q, s = fp8mm.fp8_quantize_mx(bf16_dev(x))
    rq, rs = mx.quantize_mx(x)
    _check_mx(q, s, rq, rs, f"mx {rows}x{cols}")


def test_mx_quantize_every_bf16_and_special_blocks():
    """Every bf16 value at six block maxima (the 32-blocks of these matrices
    have maxima of every size below the chosen one), zero blocks, blocks of
    subnormals and blocks whose maximum saturates."""
    amaxes = [448.0, 1.0, 3.140625, 61440.0, 2.0 ** -20, 1e-30]
    bits = workloads.f32_to_bf16_bits(np.array(amaxes, np.float32))
    x = np.concatenate([_every_bf16_under(int(b)) for b in bits])
    special = np.zeros((4, 128), np.float32)
    special[1, :32] = 2.0 ** -130
    special[1, 32:64] = -(2.0 ** -133)
    special[2, :32] = 1.0
    special[2, 7] = 1.99                      # quotient ~509: saturates
    special[3] = np.linspace(-3e38, 3e38, 128, dtype=np.float32)
    sb = workloads.f32_to_bf16_bits(special)
    x = np.concatenate([x, np.tile(sb, (1, x.shape[1] // 128))])
    q, s = fp8mm.fp8_quantize_mx(bf16_dev(x))
    rq, rs = mx.quantize_mx(x)
    _check_mx(q, s, rq, rs, "mx every bf16 + special blocks")


def test_quantize_is_deterministic_across_runs():
    x = workloads.blockwise(M=512, N=128, K=2048)["input"]
    xd = bf16_dev(x)
    q1, s1 = fp8mm.fp8_quantize_tensorwise(xd)
    q2, s2 = fp8mm.fp8_quantize_tensorwise(xd)
    assert np.array_equal(host(q1), host(q2)) and np.array_equal(host(s1), host(s2))


# ---- the benchmark shapes, checked on sampled rows / blocks / columns ----

def test_full_size_activation_1x128_sampled_rows():
    x = workloads.blockwise()["input"]                     # [16640, 8192]
    q, s = fp8mm.fp8_quantize_blockwise(bf16_dev(x), (1, 128))
    qh, sh = host(q), host(s)
    rows = np.random.default_rng(0).choice(x.shape[0], 48, replace=False)
    rq, rs = quant.quantize_blockwise(x[rows], 1, 128)
    assert np.array_equal(qh[rows], rq) and np.array_equal(sh[:, rows], rs)


def test_full_size_weight_128x128_sampled_slabs():
    w = workloads.blockwise()["weight"]                    # [5120, 8192]
    q, s = fp8mm.fp8_quantize_blockwise(bf16_dev(w), (128, 128))
    qh, sh = host(q), host(s)
    for slab in (0, 17, 39):
        rq, rs = quant.quantize_blockwise(w[slab * 128:(slab + 1) * 128], 128, 128)
        assert np.array_equal(qh[slab * 128:(slab + 1) * 128], rq) and np.array_equal(sh[slab], rs[0])


def test_full_size_grad_weight_operand_128x1_sampled_columns():
    g = workloads.grad_weight()["grad_output"]             # [16640, 5120]
    q, s = fp8mm.fp8_quantize_blockwise(bf16_dev(g), (128, 1), transpose_out=True)
    qh, sh = host(q), host(s)
    cols = np.random.default_rng(1).choice(g.shape[1], 40, replace=False)
    rq, rs = quant.quantize_blockwise(np.ascontiguousarray(g[:, cols]), 128, 1, transpose_out=True)
    assert np.array_equal(qh[cols], rq) and np.array_equal(sh[:, cols], rs)


def test_full_size_rowwise_moe_weights_sampled_rows():
    W = workloads.grouped()["W"].reshape(64 * 1408, 2048)
    q, s = fp8mm.fp8_quantize_rowwise(bf16_dev(W))
    qh, sh = host(q), host(s)
    rows = np.random.default_rng(2).choice(W.shape[0], 256, replace=False)
    rq, rs = quant.quantize_rowwise(W[rows])
    assert np.array_equal(qh[rows], rq) and np.array_equal(sh[rows, 0], rs)


def test_quantizer_random_sweep():
    """Seeded random shapes and magnitudes through every quantizer entry
    point, each bit-exact against the oracle.  Rows mix scales 2^-30 .. 2^30,
    and an x with ld_x > cols exercises the strided read."""
    rng = np.random.default_rng(20260303)
    kinds = ["tensorwise", "rowwise", "1x128", "128x128", "128x1", "128x1T", "dual", "mx", "grouped",
             "grouped_dual"]
    for case in range(30):
        kind = kinds[case % len(kinds)]
        if kind in ("128x128", "128x1", "128x1T", "dual"):
            rows = int(rng.integers(1, 6)) * 128
        else:
            rows = int(rng.integers(1, 700))
        if kind in ("1x128", "128x128", "dual", "grouped_dual"):
            cols = int(rng.integers(1, 9)) * 128
        elif kind == "mx":
            cols = int(rng.integers(1, 40)) * 32
        else:
            cols = int(rng.integers(1, 80)) * 16
        pad = int(rng.integers(0, 3)) * 8
        scale_rows = np.exp2(rng.integers(-30, 30, size=(rows, 1))).astype(np.float32)
        full = workloads.f32_to_bf16_bits((rng.standard_normal((rows, cols + pad)) * scale_rows).astype(np.float32))
        x = np.ascontiguousarray(full[:, :cols])
        xd = bf16_dev(full)[:, :cols]                     # leading dimension cols + pad
        say(f"quant sweep {case}: {kind} {rows}x{cols} ld={cols + pad}")
        what = f"quant sweep {case} {kind} {rows}x{cols}"
        if kind == "tensorwise":
            _check(*fp8mm.fp8_quantize_tensorwise(xd), *quant.quantize_tensorwise(x), what)
        elif kind == "rowwise":
            _check(*fp8mm.fp8_quantize_rowwise(xd), *quant.quantize_rowwise(x), what)
        elif kind in ("1x128", "128x128", "128x1"):
            blk = {"1x128": (1, 128), "128x128": (128, 128), "128x1": (128, 1)}[kind]
            _check(*fp8mm.fp8_quantize_blockwise(xd, blk), *quant.quantize_blockwise(x, *blk), what)
        elif kind == "128x1T":
            _check(*fp8mm.fp8_quantize_blockwise(xd, (128, 1), transpose_out=True),
                   *quant.quantize_blockwise(x, 128, 1, transpose_out=True), what)
        elif kind == "dual":
            q_row, s_row, q_col, s_col = fp8mm.fp8_quantize_blockwise_dual(xd)
            _check(q_row, s_row, *quant.quantize_blockwise(x, 1, 128), what + " rows")
            _check(q_col, s_col, *quant.quantize_blockwise(x, 128, 1, transpose_out=True), what + " cols")
        elif kind == "mx":
            q, s = fp8mm.fp8_quantize_mx(xd)
            rq, rs = mx.quantize_mx(x)
            assert np.array_equal(host(q), rq) and np.array_equal(host(s), rs), what
        else:
            E = int(rng.integers(1, 9))
            sizes = rng.multinomial(max(rows - int(rng.integers(0, 3)), 0), [1.0 / E] * E)
            offs = np.cumsum(sizes).astype(np.int32)
            od = torch.from_numpy(offs).cuda()
            rq, rs, _ = quant.quantize_grouped_128x1(x, offs)
            nb = rs.shape[0]
            if kind == "grouped":
                q_t, s_t = fp8mm.fp8_quantize_grouped_128x1(xd, od)
            else:
                q_row, s_row, q_t, s_t = fp8mm.fp8_quantize_grouped_dual(xd, od)
                M = int(offs[-1])
                if M:
                    rq1, rs1 = quant.quantize_blockwise(x[:M], 1, 128)
                    assert np.array_equal(host(q_row)[:M], rq1), what + " row codes"
                    assert np.array_equal(host(s_row)[:, :M], rs1), what + " row scales"
            assert np.array_equal(host(q_t)[:, :128 * nb], rq), what + " runs"
            assert np.array_equal(host(s_t)[:nb], rs), what + " run scales"
