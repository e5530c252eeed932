"""Benchmark of the FP8 scaled-GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
                    [--no-cpu-baseline] [--no-recipes] [--workload NAME]

One step = one pass of the whole hot path over the workload's synthetic
inputs (already resident in HBM): dynamic quantization of both operands
(group amax -> scale -> saturating E4M3 cast) and the scaled GEMM with its
scale application and bf16 epilogue.  The default workload is the blockwise
1x128 x 128x128 forward GEMM at M=16640, N=5120, K=8192 (the shape the
method's published blockwise table and its 60 %-of-peak target use).

Printed: one JSON line with the step throughput (GEMM flops 2*M*N*K per step
over the step time), the roofline of the dominant kernel (the GEMM, timed
with HIP events on the stream it is launched on), per-recipe kernel-level
numbers for every workload, and the CPU oracle timed on a bounded sample.
"""

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_DENSE_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA (no sparsity)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    # On a fresh load the device's power controller first lets the shader
    # clock run (1.77 GHz for the first two GEMM calls), then pulls it down
    # (1.61 GHz at calls 3-5) and takes about 30 calls (40 ms) of back-to-back
    # steps to settle at its sustained clock (1.83 GHz); the GEMM's cycle
    # count stays the same throughout, so its time follows the clock.  The
    # settle phase runs the step back to back for this long before the
    # warm-up steps, so the timed steps see the sustained clock.
    ap.add_argument("--settle-ms", type=float, default=200.0)
    # The GEMM operands' codes: the quantizers' output (default), or, keeping
    # shapes, scales and every instruction of the step, all 0x00 (zero) or all
    # 0x38 (1.0).  Shows how far the device clock, hence the GEMM's rate,
    # follows the switching activity of the data under the power limit.
    ap.add_argument("--codes", choices=("quantized", "zero", "one"), default="quantized")
    ap.add_argument("--workload", default="blockwise_fwd_16640x5120x8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-recipes", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device-to-device copy (3 times), so that a rocprofv3 "
                         "counter run sees FETCH_SIZE / WRITE_SIZE of a kernel with known traffic")
    return ap.parse_args()


# --------------------------------------------------------------------------
# workloads: (name, builder) -> dict with 'step' (callable), 'flops',
# 'gemm' (callable launching only the GEMM), 'gemm_bytes' (algorithmic)
# --------------------------------------------------------------------------

def _dev_bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def build_workloads(torch, fp8mm, workloads):
    W = {}

    def blockwise_fwd(M, N, K):
        inp = workloads.blockwise(M=M, N=N, K=K)
        x, w = _dev_bf16(inp["input"], torch), _dev_bf16(inp["weight"], torch)
        state = {}

        def quant():
            state["qx"], state["sx"] = fp8mm.fp8_quantize_blockwise(x, (1, 128))
            state["qw"], state["sw"] = fp8mm.fp8_quantize_blockwise(w, (128, 128))

        def gemm():
            return fp8mm.fp8_scaled_mm(state["qx"], state["qw"], state["sx"], "1x128", state["sw"], "128x128")

        return dict(quant=quant, gemm=gemm, state=state, flops=2.0 * M * N * K,
                    gemm_bytes=M * K + N * K + 4 * (K // 128) * (M + N // 128) + 2 * M * N,
                    quant_bytes=3 * (M * K + N * K) + 4 * ((K // 128) * M + (N // 128) * (K // 128)),
                    shape=(M, N, K), recipe="blockwise_1x128_128x128")

    def blockwise_grad_input(M, N, K):
        # grad_input[M, K] = grad_output[M, N] @ weight[N, K]
        inp = workloads.blockwise(M=M, N=N, K=K)
        g, w = _dev_bf16(inp["grad_output"], torch), _dev_bf16(inp["weight"], torch)
        state = {}

        def quant():
            state["qg"], state["sg"] = fp8mm.fp8_quantize_blockwise(g, (1, 128))
            state["qw"], state["sw"] = fp8mm.fp8_quantize_blockwise(w, (128, 128))

        def gemm():
            return fp8mm.fp8_linear_grad_input(state["qg"], state["sg"], "1x128", state["qw"], state["sw"], "128x128")

        return dict(quant=quant, gemm=gemm, state=state, flops=2.0 * M * N * K,
                    gemm_bytes=M * N + N * K + 4 * (N // 128) * (M + K // 128) + 2 * M * K,
                    quant_bytes=3 * (M * N + N * K), shape=(M, K, N), recipe="blockwise_1x128_128x128 (KN)")

    def blockwise_grad_weight(T, N_out, K_in):
        inp = workloads.grad_weight(T=T, N_out=N_out, K_in=K_in)
        g, x = _dev_bf16(inp["grad_output"], torch), _dev_bf16(inp["input"], torch)
        state = {}

        def quant():
            state["qg"], state["sg"] = fp8mm.fp8_quantize_blockwise(g, (128, 1), transpose_out=True)
            state["qx"], state["sx"] = fp8mm.fp8_quantize_blockwise(x, (128, 1), transpose_out=True)

        def gemm():
            return fp8mm.fp8_linear_grad_weight(state["qg"], state["sg"], state["qx"], state["sx"])

        return dict(quant=quant, gemm=gemm, state=state, flops=2.0 * T * N_out * K_in,
                    gemm_bytes=T * (N_out + K_in) + 4 * (T // 128) * (N_out + K_in) + 2 * N_out * K_in,
                    quant_bytes=3 * T * (N_out + K_in), shape=(N_out, K_in, T), recipe="blockwise_1x128_128x1")

    def rowwise(M, N, K):
        inp = workloads.rowwise(M=M, N=N, K=K)
        x, w, b = _dev_bf16(inp["x"], torch), _dev_bf16(inp["w"], torch), _dev_bf16(inp["bias"], torch)
        state = {}

        def quant():
            state["qx"], state["sx"] = fp8mm.fp8_quantize_rowwise(x)
            state["qw"], state["sw"] = fp8mm.fp8_quantize_rowwise(w)

        def gemm():
            return fp8mm.fp8_scaled_mm(state["qx"], state["qw"], state["sx"], "rowwise", state["sw"], "rowwise", bias=b)

        return dict(quant=quant, gemm=gemm, state=state, flops=2.0 * M * N * K,
                    gemm_bytes=M * K + N * K + 4 * (M + N) + 2 * N + 2 * M * N,
                    quant_bytes=3 * (M * K + N * K) + 4 * (M + N), shape=(M, N, K), recipe="rowwise_rowwise")

    def mxfp8(M, N, K):
        # the blockwise forward operands, quantized MXFP8 (E8M0 per 32 along K)
        inp = workloads.blockwise(M=M, N=N, K=K)
        x, w = _dev_bf16(inp["input"], torch), _dev_bf16(inp["weight"], torch)
        state = {}

        def quant():
            state["qx"], state["sx"] = fp8mm.fp8_quantize_mx(x)
            state["qw"], state["sw"] = fp8mm.fp8_quantize_mx(w)

        def gemm():
            return fp8mm.fp8_scaled_mm(state["qx"], state["qw"], state["sx"], "mxfp8", state["sw"], "mxfp8")

        return dict(quant=quant, gemm=gemm, state=state, flops=2.0 * M * N * K,
                    gemm_bytes=M * K + N * K + (M + N) * (K // 32) + 2 * M * N,
                    quant_bytes=3 * (M * K + N * K) + (M + N) * (K // 32), shape=(M, N, K), recipe="mxfp8_mxfp8")

    def tensorwise(n):
        inp = workloads.tensorwise(n=n)
        a, b = _dev_bf16(inp["A"], torch), _dev_bf16(inp["B"], torch)
        state = {}

        def quant():
            state["qa"], state["sa"] = fp8mm.fp8_quantize_tensorwise(a)
            state["qb"], state["sb"] = fp8mm.fp8_quantize_tensorwise(b)

        def gemm():
            return fp8mm.fp8_scaled_mm(state["qa"], state["qb"], state["sa"], "tensorwise", state["sb"], "tensorwise")

        return dict(quant=quant, gemm=gemm, state=state, flops=2.0 * n ** 3, gemm_bytes=2 * n * n + 8 + 2 * n * n,
                    quant_bytes=6 * n * n, shape=(n, n, n), recipe="tensorwise_tensorwise")

    def grouped():
        inp = workloads.grouped()
        act = _dev_bf16(inp["act"], torch)
        E, N, K = inp["W"].shape
        Wd = _dev_bf16(inp["W"].reshape(E * N, K), torch)
        offs = torch.from_numpy(inp["offs"]).cuda()
        M = int(inp["offs"][-1])
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        state = {}

        def quant():
            state["qa"], state["sa"] = fp8mm.fp8_quantize_rowwise(act)
            state["qw"], state["sw"] = fp8mm.fp8_quantize_rowwise(Wd)

        def gemm():
            return fp8mm.fp8_scaled_grouped_mm(state["qa"], state["qw"].view(E, N, K), offs, state["sa"],
                                               state["sw"].view(E, N), out=out)

        return dict(quant=quant, gemm=gemm, state=state, flops=2.0 * M * N * K,
                    gemm_bytes=M * K + E * N * K + 4 * (M + E * N) + 4 * E + 2 * M * N,
                    quant_bytes=3 * (M * K + E * N * K) + 4 * (M + E * N), shape=(M, N, K, E),
                    recipe="grouped_rowwise_E64")

    def grouped_blockwise(layout):
        # NK: the MoE forward, out [16384, 1408] = act [16384, 2048] @ W[e]^T;
        # KN: its input gradient, [16384, 2048] = grad_output [16384, 1408] @
        # W[e], the stored [1408, 2048] expert weights read [K, N]
        inp = workloads.grouped_backward()
        E, Nw, Kw = inp["W"].shape
        Wd = _dev_bf16(inp["W"].reshape(E * Nw, Kw), torch)
        a = _dev_bf16(inp["act"] if layout == "NK" else inp["grad_output"], torch)
        offs = torch.from_numpy(inp["offs"]).cuda()
        M = int(inp["offs"][-1])
        N, K = (Nw, Kw) if layout == "NK" else (Kw, Nw)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        state = {}

        def quant():
            state["qa"], state["sa"] = fp8mm.fp8_quantize_blockwise(a, (1, 128))
            state["qw"], state["sw"] = fp8mm.fp8_quantize_blockwise(Wd, (128, 128))

        def gemm():
            return fp8mm.fp8_scaled_grouped_mm_v2(state["qa"], state["qw"].view(E, Nw, Kw), offs, state["sa"], "1x128",
                                                  state["sw"].view(E, Nw // 128, Kw // 128), "128x128",
                                                  b_layout=layout, out=out)

        scales = 4 * ((K // 128) * M + E * (Nw // 128) * (Kw // 128))
        return dict(quant=quant, gemm=gemm, state=state, flops=2.0 * M * N * K,
                    gemm_bytes=M * K + E * N * K + scales + 4 * E + 2 * M * N,
                    quant_bytes=3 * (M * K + E * N * K) + scales, shape=(M, N, K, E),
                    recipe="grouped_blockwise_1x128_128x128" + (" (KN)" if layout == "KN" else ""))

    def grouped_grad_weight():
        # grad_w[e] [1408, 2048] = grad_output[rows_e].t() @ act[rows_e], 64 experts
        inp = workloads.grouped_backward()
        g, x = _dev_bf16(inp["grad_output"], torch), _dev_bf16(inp["act"], torch)
        offs = torch.from_numpy(inp["offs"]).cuda()
        T, N_out = g.shape
        K_in = x.shape[1]
        E = offs.numel()
        runs = int(np.sum((np.diff(np.concatenate([[0], inp["offs"]])) + 127) // 128))
        state = {}

        def quant():
            state["qg"], state["sg"] = fp8mm.fp8_quantize_grouped_128x1(g, offs)
            state["qx"], state["sx"] = fp8mm.fp8_quantize_grouped_128x1(x, offs)

        def gemm():
            return fp8mm.fp8_grouped_linear_grad_weight(state["qg"], state["sg"], state["qx"], state["sx"], offs, T)

        scales = 4 * runs * (N_out + K_in)
        return dict(quant=quant, gemm=gemm, state=state, flops=2.0 * T * N_out * K_in,
                    gemm_bytes=T * (N_out + K_in) + scales + 4 * E + 2 * E * N_out * K_in,
                    quant_bytes=3 * T * (N_out + K_in) + scales, shape=(N_out, K_in, T, E),
                    recipe="grouped_weight_gradient_1x128_128x1")

    W["tensorwise_256"] = lambda: tensorwise(256)
    W["rowwise_8192x4096x4096"] = lambda: rowwise(8192, 4096, 4096)
    W["blockwise_fwd_16640x5120x8192"] = lambda: blockwise_fwd(16640, 5120, 8192)
    W["blockwise_fwd_16640x8192x5120"] = lambda: blockwise_fwd(16640, 8192, 5120)
    W["blockwise_grad_input_16640x8192x5120"] = lambda: blockwise_grad_input(16640, 5120, 8192)
    W["blockwise_grad_input_16640x5120x8192"] = lambda: blockwise_grad_input(16640, 8192, 5120)
    W["blockwise_grad_weight_5120x8192x16640"] = lambda: blockwise_grad_weight(16640, 5120, 8192)
    W["grouped_moe_E64_16384x1408x2048"] = grouped
    W["mxfp8_16640x5120x8192"] = lambda: mxfp8(16640, 5120, 8192)
    W["grouped_blockwise_E64_16384x1408x2048"] = lambda: grouped_blockwise("NK")
    W["grouped_blockwise_grad_input_E64_16384x2048x1408"] = lambda: grouped_blockwise("KN")
    W["grouped_grad_weight_E64_1408x2048_T16384"] = grouped_grad_weight
    return W


def copy_ceiling_gbps(torch):
    """Measured HBM ceiling for the quantize passes: a 1 GiB device-to-device
    copy (read + write bytes per second), median of 10."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    med, _, _, _ = time_kernel(torch, lambda: dst.copy_(src), 10)
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * (1 << 30) / (med * 1e-3) / 1e9


def time_kernel(torch, fn, iters, warmup=3):
    """Device time (ms) of fn's launches, HIP events on the current stream:
    (median, mean, min, max)."""
    for _ in range(warmup):
        fn()
    evs = []
    for _ in range(iters):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        evs.append((s, e))
    torch.cuda.synchronize()
    t = sorted(s.elapsed_time(e) for s, e in evs)
    return t[len(t) // 2], float(np.mean(t)), t[0], t[-1]


def time_cold(torch, fn, flush, iters=20, warmup=3, clean=True):
    """Device time (ms) of fn with HBM-resident operands: before each timed
    call a 512 MiB buffer (twice the 256 MiB MALL) is overwritten outside the
    events, then (clean) a second 512 MiB buffer is read, also outside the
    events.  The read evicts the overwritten lines, so their write-back to
    HBM happens before the timed call instead of inside it, and leaves clean
    lines of other data in the caches: the timed call reads its operands
    from HBM and pays for no one else's writes.  clean=False times the call
    right after the overwrite (caches full of dirty lines).  (median, min,
    max)."""
    for _ in range(warmup):
        fn()
    t = []
    for _ in range(iters):
        flush[0].fill_(1)
        if clean:
            flush[1].view(torch.int32).max()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        t.append(s.elapsed_time(e))
    t.sort()
    return t[len(t) // 2], t[0], t[-1]


def time_graph(torch, fn, calls=10, iters=20):
    """Device time (ms) per call of fn replayed from a HIP graph that holds
    `calls` back-to-back calls (no host launch gaps): median over iters
    replays / calls.  None if the calls cannot be captured."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                fn()
        g.replay()
        torch.cuda.synchronize()
        evs = []
        for _ in range(iters):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            g.replay()
            e.record()
            evs.append((s, e))
        torch.cuda.synchronize()
        t = sorted(s.elapsed_time(e) for s, e in evs)
        del g
        return t[len(t) // 2] / calls
    except RuntimeError as exc:
        print(f"[bench] graph capture failed: {exc}", file=sys.stderr, flush=True)
        return None


def cpu_baseline(workloads):
    """The oracle (untuned numpy + OpenBLAS float64) on the default workload:
    the whole 16640x5120x8192 blockwise forward step (quantize the input and
    the weight, then the GEMM), about 10-15 s on the host's cores."""
    from oracle import gemm as ogemm
    from oracle import quant as oquant

    from threadpoolctl import threadpool_info, threadpool_limits

    Ms, N, K = 16640, 5120, 8192
    inp = workloads.blockwise(M=16640, N=N, K=K)
    x = inp["input"][:Ms]
    w = inp["weight"]
    # every host core this process may run on, set explicitly on the BLAS
    # library numpy uses (the oracle's only multi-threaded step is its matmul)
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores, user_api="blas"):
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        t0 = time.perf_counter()
        qx, sx = oquant.quantize_blockwise(x, 1, 128)
        qw, sw = oquant.quantize_blockwise(w, 128, 128)
        ogemm.scaled_mm(qx, qw, sx, "1x128", sw, "128x128")
        dt = time.perf_counter() - t0
    threads = max((i.get("num_threads", 1) for i in blas), default=1)
    lib = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({os.path.basename(i.get('filepath', ''))})"
                    for i in blas) or "none found"
    print(f"[bench] cpu baseline: {cores} cores, BLAS {lib}, {threads} threads", file=sys.stderr, flush=True)
    return {"value": round(2.0 * Ms * N * K / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "host_cores_available": cores, "blas": lib, "blas_threads": int(threads),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"the whole blockwise 1x128_128x128 forward step at {Ms}x{N}x{K}: numpy oracle "
                      f"quantization of the input and the weight, float64 GEMM ({2.0 * Ms * N * K / 1e9:.0f} "
                      f"GFLOP), rounding to bf16"}


GEMM_SOURCES = ("gemm.hip", "gemm_sym.hip", "gemm_grp.hip", "gemm_common.hpp", "grouped.hpp", "launch.hpp")


def gemm_source_sha():
    """sha256 over the GEMM kernel sources, in GEMM_SOURCES order."""
    import hashlib

    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, "precision_matmul_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def measured_profile(workload):
    """Counter figures of one GEMM call from the committed summary
    profiles/<workload>.md: HBM bytes (FETCH_SIZE + WRITE_SIZE summed over the
    call's launches, each scaled by what the counter reads for a plain copy of
    known size) and the kernels the call launches.  Traffic is None when there
    is no summary, or when the GEMM sources have changed since the counters
    were taken (the summary records their sha256)."""
    path = os.path.join(ROOT, "profiles", workload + ".md")
    try:
        text = open(path).read()
        sha = gemm_source_sha()
    except OSError:
        return None, None
    got = dict(re.findall(r"^(traffic_bytes_per_call|gemm_sources_sha256|gemm_call_kernels): *(.+)$", text, re.M))
    kernels = got.get("gemm_call_kernels")
    if got.get("gemm_sources_sha256", "").strip() != sha or "traffic_bytes_per_call" not in got:
        return None, kernels
    return int(got["traffic_bytes_per_call"]), kernels


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library is a single-GPU kernel library with no collectives)",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    import precision_matmul_amd as fp8mm
    import workloads

    fp8mm._lib.load()
    torch.cuda.init()
    W = build_workloads(torch, fp8mm, workloads)
    if args.workload not in W:
        raise SystemExit(f"unknown workload {args.workload}; choose from {sorted(W)}")

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("[bench] calibration copy: 3 x 512 MiB device-to-device", file=sys.stderr, flush=True)

    print(f"[bench] building inputs for {args.workload}", file=sys.stderr, flush=True)
    wl = W[args.workload]()
    torch.cuda.synchronize()

    if args.codes != "quantized":
        # quantize once, then pin the GEMM operands to constant codes: the
        # step still runs the quantizers (into fresh buffers) and the GEMM
        quant0 = wl["quant"]
        quant0()
        state = wl["state"]
        code = 0 if args.codes == "zero" else 0x38
        fixed = {k: (torch.full_like(v, code) if k.startswith("q") else v) for k, v in state.items()}

        def quant_fixed():
            quant0()
            state.update(fixed)
        wl["quant"] = quant_fixed

    def step():
        wl["quant"]()
        return wl["gemm"]()

    settle_steps = 0
    t_settle = time.perf_counter() + args.settle_ms * 1e-3
    while args.settle_ms > 0:
        step()
        settle_steps += 1
        if settle_steps % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() >= t_settle:
                break
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    gemm_events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        wl["quant"]()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        wl["gemm"]()
        e.record()
        gemm_events.append((s, e))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    gemm_ms = float(np.mean([s.elapsed_time(e) for s, e in gemm_events]))
    value = wl["flops"] / (ms_step * 1e-3) / 1e12
    achieved = wl["flops"] / (gemm_ms * 1e-3) / 1e12
    print(f"[bench] step {ms_step:.3f} ms, gemm {gemm_ms:.3f} ms ({achieved:.1f} TFLOP/s)", file=sys.stderr,
          flush=True)

    traffic, call_kernels = measured_profile(args.workload)
    # The pages' own GEMM-only figures for these shapes (pytorch/ao PR #2784,
    # "improve fp8 blockwise gemm perf", the two tables; hardware not named):
    # context for the GEMM alone, not for the step `value`.
    pages_gemm = {"blockwise_fwd_16640x5120x8192": 1008.91, "blockwise_fwd_16640x8192x5120": 1002.23,
                  "blockwise_grad_weight_5120x8192x16640": 808.271}.get(args.workload)

    result = {
        "metric": "FP8 scaled-GEMM TFLOP/s at 1 MI355X + % of FP8 MFMA peak, per recipe",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settle_steps,
                   "why": "untimed back-to-back steps before the warm-up steps, until the device's power "
                          "controller has settled the shader clock after its fresh-load transient"},
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic (seeded bf16 normals, shapes of the method's benchmarks)" if args.codes == "quantized" else
                f"synthetic shapes; GEMM operand codes replaced by constant {args.codes} codes (clock study, not a "
                "benchmark figure)",
        "config": {"workload": args.workload, "recipe": wl["recipe"], "shape_MNK": list(wl["shape"]),
                   "step": "quantize both operands + scaled GEMM, bf16 out", "out_dtype": "bf16"},
        "roofline": {"bound": "mfma", "kernel": "GEMM call, " + wl["recipe"] + ": " + (call_kernels or "see profile"),
                     "achieved": round(achieved, 2), "peak": FP8_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP8_DENSE_PEAK_TFLOPS, 4), "traffic": traffic,
                     "algorithmic_bytes": wl["gemm_bytes"], "gemm_ms": round(gemm_ms, 4)},
    }
    if pages_gemm is not None:
        result["context_pages_gemm"] = {
            "tflops": pages_gemm, "hardware": "not named on the page",
            "gemm_over_pages": round(achieved / pages_gemm, 3),
            "note": "the pages time the GEMM alone; value above is the whole step (quantize + GEMM)"}

    if not args.no_recipes:
        copy_gbs = copy_ceiling_gbps(torch)
        result["copy_ceiling_GBps"] = round(copy_gbs, 1)
        flush = (torch.empty(512 << 20, dtype=torch.uint8, device="cuda"),
                 torch.ones(512 << 20, dtype=torch.uint8, device="cuda"))
        per = {}
        for name, make in W.items():
            print(f"[bench] recipe workload {name}", file=sys.stderr, flush=True)
            w2 = wl if name == args.workload else make()
            w2["quant"]()
            q_med, _, q_min, q_max = time_kernel(torch, w2["quant"], 20)
            g_med, _, g_min, g_max = time_kernel(torch, w2["gemm"], 50, warmup=10)
            q_gbs = w2["quant_bytes"] / (q_med * 1e-3) / 1e9
            g_graph = time_graph(torch, w2["gemm"])
            c_med, c_min, c_max = time_cold(torch, w2["gemm"], flush)
            d_med, _, _ = time_cold(torch, w2["gemm"], flush, clean=False)
            # Primary figures: cold, operands read from HBM (time_cold);
            # warm (back to back, the operands possibly still in the 256 MiB
            # MALL) and cold with the caches full of another kernel's dirty
            # lines beside them.
            per[name] = {"recipe": w2["recipe"],
                         "gemm_ms_cold": round(c_med, 4), "gemm_ms_cold_min_max": [round(c_min, 4), round(c_max, 4)],
                         "gemm_ms_cold_dirty_cache": round(d_med, 4),
                         "gemm_tflops": round(w2["flops"] / (c_med * 1e-3) / 1e12, 2),
                         "gemm_frac_fp8_peak": round(w2["flops"] / (c_med * 1e-3) / 1e12 / FP8_DENSE_PEAK_TFLOPS, 4),
                         "gemm_ms_warm": round(g_med, 4),
                         "gemm_ms_warm_min_max": [round(g_min, 4), round(g_max, 4)],
                         "gemm_ms_graph_warm": None if g_graph is None else round(g_graph, 4),
                         "gemm_tflops_warm": round(w2["flops"] / (g_med * 1e-3) / 1e12, 2),
                         "quant_ms": round(q_med, 4),
                         "quant_ms_min_max": [round(q_min, 4), round(q_max, 4)],
                         "quant_GBps": round(q_gbs, 1),
                         "quant_frac_hbm_peak": round(q_gbs / HBM_PEAK_GBS, 4),
                         "quant_frac_copy_ceiling": round(q_gbs / copy_gbs, 4)}
            # HBM-bound GEMMs (the grouped MoE shape): the fraction of the
            # attainable roofline, min(peak flops, bytes at 8 TB/s)
            t_roof = max(w2["flops"] / (FP8_DENSE_PEAK_TFLOPS * 1e12), w2["gemm_bytes"] / (HBM_PEAK_GBS * 1e9))
            per[name]["gemm_bound"] = "mfma" if w2["flops"] / (FP8_DENSE_PEAK_TFLOPS * 1e12) >= t_roof else "hbm"
            per[name]["gemm_frac_attainable_roofline"] = round(t_roof / (c_med * 1e-3), 4)
            per[name]["gemm_frac_attainable_roofline_warm"] = round(t_roof / (g_med * 1e-3), 4)
            if w2 is not wl:
                del w2
            torch.cuda.empty_cache()
        result["per_recipe"] = per
        del flush
        # The backward's quantize of grad_output [16640, 5120]: one dual-layout
        # pass (1x128 codes + 128x1 codes written transposed) against the two
        # single-layout passes it replaces.
        print("[bench] dual-layout quantize of grad_output", file=sys.stderr, flush=True)
        go = _dev_bf16(workloads.grad_weight()["grad_output"], torch)
        T, C = go.shape
        d_med, _, d_min, d_max = time_kernel(torch, lambda: fp8mm.fp8_quantize_blockwise_dual(go), 20)
        sep_med, _, _, _ = time_kernel(torch, lambda: (fp8mm.fp8_quantize_blockwise(go, (1, 128)),
                                                       fp8mm.fp8_quantize_blockwise(go, (128, 1), transpose_out=True)),
                                       20)
        dual_bytes = 4 * T * C + 4 * (T * (C // 128) + (T // 128) * C)
        d_gbs = dual_bytes / (d_med * 1e-3) / 1e9
        result["grad_output_dual_quant"] = {
            "shape": [T, C], "dual_ms": round(d_med, 4), "dual_ms_min_max": [round(d_min, 4), round(d_max, 4)],
            "two_single_passes_ms": round(sep_med, 4), "dual_GBps": round(d_gbs, 1),
            "dual_frac_hbm_peak": round(d_gbs / HBM_PEAK_GBS, 4), "dual_frac_copy_ceiling": round(d_gbs / copy_gbs, 4),
            "algorithmic_bytes": dual_bytes}
        del go
        # The FP8 blockwise linear layer as one autograd op: forward, grad_input
        # and grad_weight with every quantize, at the shapes of the blockwise
        # forward, grad_input and grad_weight workloads.
        print("[bench] linear layer step (forward + backward)", file=sys.stderr, flush=True)
        inp = workloads.blockwise(M=16640, N=5120, K=8192)
        xl = _dev_bf16(inp["input"], torch).requires_grad_(True)
        wl_ = _dev_bf16(inp["weight"], torch).requires_grad_(True)
        gl = _dev_bf16(workloads.grad_weight()["grad_output"], torch)
        del inp

        def layer_step():
            xl.grad = None
            wl_.grad = None
            fp8mm.fp8_blockwise_linear(xl, wl_).backward(gl)

        l_med, _, l_min, l_max = time_kernel(torch, layer_step, 10, warmup=3)
        l_flops = 3 * 2.0 * 16640 * 5120 * 8192
        result["linear_layer_step"] = {
            "shape_T_Kin_Nout": [16640, 8192, 5120], "ms": round(l_med, 4),
            "ms_min_max": [round(l_min, 4), round(l_max, 4)],
            "tflops": round(l_flops / (l_med * 1e-3) / 1e12, 2),
            "frac_fp8_peak": round(l_flops / (l_med * 1e-3) / 1e12 / FP8_DENSE_PEAK_TFLOPS, 4),
            "step": "dual quantize of input, 128x128 quantize of weight, forward GEMM; dual quantize of "
                    "grad_output, grad_input GEMM, grad_weight GEMM"}
        del xl, wl_, gl
        torch.cuda.empty_cache()
        # The MoE expert layer as one autograd op (E = 64, 16384 tokens,
        # K_in = 2048, N_out = 1408): grouped forward, grouped input gradient
        # and per-expert weight gradient with every quantize.
        print("[bench] grouped (MoE) layer step (forward + backward)", file=sys.stderr, flush=True)
        inp = workloads.grouped_backward()
        xg = _dev_bf16(inp["act"], torch).requires_grad_(True)
        E_, N_, K_ = inp["W"].shape
        wg = _dev_bf16(inp["W"], torch).requires_grad_(True)
        gg = _dev_bf16(inp["grad_output"], torch)
        og = torch.from_numpy(inp["offs"]).cuda()
        Tg = int(inp["offs"][-1])
        del inp

        def moe_step():
            xg.grad = None
            wg.grad = None
            fp8mm.fp8_grouped_linear(xg, wg, og).backward(gg)

        m_med, _, m_min, m_max = time_kernel(torch, moe_step, 10, warmup=3)
        m_flops = 3 * 2.0 * Tg * N_ * K_
        result["grouped_layer_step"] = {
            "shape_T_Kin_Nout_E": [Tg, K_, N_, E_], "ms": round(m_med, 4),
            "ms_min_max": [round(m_min, 4), round(m_max, 4)],
            "tflops": round(m_flops / (m_med * 1e-3) / 1e12, 2),
            "step": "dual-layout (1x128 + per-expert runs) quantize of x, 128x128 quantize of the expert weights, "
                    "grouped forward; dual-layout quantize of grad_output, grouped input gradient, per-expert "
                    "weight gradient"}
        del xg, wg, gg, og
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(workloads)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
