"""Stream and graph behaviour of the library: every call enqueues on the
caller's current stream and on nothing else, allocates nothing and never
synchronizes, so the same calls give the same bits on a side stream and when
captured into a HIP graph and replayed.

The shape 16640 x 5120 x 2048 in the blockwise recipe takes the streaming
kernel on the first 16384 rows, the 128 x 128 generic kernel split along K
on the 256-row tail (its fp32 partials staged in the output's head rows) and
the in-order reduction, so the graph holds every launch kind of a GEMM call.
Each replay runs on fresh inputs copied into the captured input buffers, with
eager library calls and synchronizations in between, and is compared bit for
bit with the eager result on the same inputs.
"""

import numpy as np
import pytest
import torch

import precision_matmul_amd as fp8mm
import workloads
from tests.gpu_util import bf16_dev, say

pytestmark = pytest.mark.gpu

M, N, K = 16640, 5120, 2048


def _inputs(seed):
    g = workloads.streams(seed, 2)
    return (bf16_dev(workloads.normal_bf16(g[0], (M, K))),
            bf16_dev(workloads.normal_bf16(g[1], (N, K), 0.02)))


def _step(x, w):
    qx, sx = fp8mm.fp8_quantize_blockwise(x, (1, 128))
    qw, sw = fp8mm.fp8_quantize_blockwise(w, (128, 128))
    return qx, sx, qw, sw, fp8mm.fp8_scaled_mm(qx, qw, sx, "1x128", sw, "128x128")


def _same(a, b, what):
    torch.cuda.synchronize()
    assert a.dtype == b.dtype and a.shape == b.shape, what
    assert torch.equal(a, b), what


def test_side_stream_gives_the_same_bits():
    x, w = _inputs(901)
    say("default stream step 16640x5120x2048")
    ref = _step(x, w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    say("side stream step 16640x5120x2048")
    with torch.cuda.stream(side):
        got = _step(x, w)
    torch.cuda.current_stream().wait_stream(side)
    for r, g, what in zip(ref, got, ("x codes", "x scales", "w codes", "w scales", "out")):
        _same(r, g, f"side stream: {what}")


def test_graph_replays_match_eager():
    x_static, w_static = _inputs(902)
    # warm-up on a side stream, as graph capture asks
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(x_static, w_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("capturing quantize x2 + blockwise GEMM 16640x5120x2048")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = _step(x_static, w_static)
    torch.cuda.synchronize()
    for rep in range(3):
        x_new, w_new = _inputs(910 + rep)
        say(f"replay {rep}")
        x_static.copy_(x_new)
        w_static.copy_(w_new)
        graph.replay()
        torch.cuda.synchronize()
        # eager library work between replays (also overwrites other memory)
        eager = _step(x_new, w_new)
        torch.cuda.synchronize()
        for c, e, what in zip(captured, eager, ("x codes", "x scales", "w codes", "w scales", "out")):
            _same(c, e, f"replay {rep}: {what}")
        assert float(eager[4].float().abs().max()) > 0, "the output is not trivially zero"


def test_grouped_graph_follows_new_routing():
    """The grouped GEMM reads its offsets on the device: one captured call
    follows a routing that changes between replays (expert sizes redrawn,
    empty experts included), matching the eager call on the same routing."""
    E, Ng, Kg, T = 16, 1408, 2048, 4096
    g = workloads.streams(920, 2)
    W = bf16_dev(workloads.normal_bf16(g[0], (E * Ng, Kg), 0.02))
    qw, sw = fp8mm.fp8_quantize_blockwise(W, (128, 128))
    qw, sw = qw.view(E, Ng, Kg), sw.view(E, Ng // 128, Kg // 128)
    x_static = bf16_dev(workloads.normal_bf16(g[1], (T, Kg)))
    offs_static = torch.zeros(E, dtype=torch.int32, device="cuda")

    def routing(seed):
        r = np.random.default_rng(seed)
        sizes = r.multinomial(T, r.dirichlet(np.ones(E)))
        sizes[r.integers(0, E)] = 0
        sizes[0] += T - sizes.sum()
        return torch.from_numpy(np.cumsum(sizes).astype(np.int32)).cuda()

    def call(x, offs):
        qx, sx = fp8mm.fp8_quantize_blockwise(x, (1, 128))
        out = torch.zeros((T, Ng), dtype=torch.bfloat16, device="cuda")
        return fp8mm.fp8_scaled_grouped_mm_v2(qx, qw, offs, sx, "1x128", sw, "128x128", out=out)

    offs_static.copy_(routing(930))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(x_static, offs_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("capturing grouped blockwise GEMM E=16 4096x1408x2048")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = call(x_static, offs_static)
    torch.cuda.synchronize()
    for rep in range(3):
        offs = routing(931 + rep)
        x_new = bf16_dev(workloads.normal_bf16(workloads.streams(940 + rep, 1)[0], (T, Kg)))
        say(f"grouped replay {rep}: offsets {offs.tolist()[:4]}...")
        offs_static.copy_(offs)
        x_static.copy_(x_new)
        graph.replay()
        torch.cuda.synchronize()
        eager = call(x_new, offs)
        _same(captured, eager, f"grouped replay {rep}")
        assert float(eager.float().abs().max()) > 0
