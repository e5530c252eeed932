"""Seeded synthetic inputs for the FP8 scaled-GEMM workloads.

This module only draws random numbers and rounds them to bfloat16 input
tensors; it holds none of the method's arithmetic (no scaling, no FP8
encoding, no GEMM).  Both the CPU oracle checks and the GPU library tests take
their inputs from here; nothing else is shared between the two.

Recipe: configuration i uses ``numpy.random.Generator(PCG64(SeedSequence(
20260000 + i)))`` spawned into one child stream per tensor, in the order the
tensors are listed; each tensor is float32 ``standard_normal * sigma`` rounded
to bfloat16 (round to nearest even).  bfloat16 tensors are returned as numpy
``uint16`` bit patterns.

Workloads (shapes of the pages' benchmarks; the pages name no dataset, the
blockwise shapes are the llama4 w1/w3 and w2 GEMMs of pytorch/ao PR #2784,
"improve fp8 blockwise gemm perf"):
  0 tensorwise   A, B [256, 256] ~N(0,1)
  1 rowwise      x [8192, 4096] ~N(0,1) with 1% of columns (41, seeded) x50,
                 w [4096, 4096] ~N(0, 0.02), bias [4096] ~N(0, 0.01)
  2 blockwise    input [M, K] ~N(0,1), weight [N, K] ~N(0, 0.02), grad_output
                 [M, N] ~N(0,1) for (M, N, K) in (16640, 5120, 8192) and
                 (16640, 8192, 5120)
  3 grad_weight  grad_output [16640, 5120] ~N(0, 1e-3), input [16640, 8192]
                 ~N(0, 1)
  4 grouped MoE  act [16384, 2048] ~N(0,1), W [64, 1408, 2048] ~N(0, 0.02),
                 group sizes ~ multinomial(16384, uniform over 64), offsets =
                 cumulative int32 end offsets
  5 grouped MoE backward: the tensors and routing of 4, plus grad_output
                 [16384, 1408] ~N(0, 1e-3) (the dense weight gradient's
                 grad_output distribution)
Every generator takes optional smaller sizes so that the same distributions
serve the oracle-sized parity cases.
"""

import numpy as np

SEED_BASE = 20260000


def streams(seed, n):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(n)]


def f32_to_bf16_bits(x):
    """Round float32 to bfloat16 (nearest, ties to even); uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((b >> 16) & 1) + np.uint32(0x7FFF)
    out = ((b + r) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        out = np.where(nan, np.uint16(0x7FC0), out)
    return out


def normal_bf16(gen, shape, sigma=1.0):
    x = gen.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(x)


def tensorwise(n=256, m=None, k=None, seed=SEED_BASE + 0):
    m = n if m is None else m
    k = n if k is None else k
    g = streams(seed, 2)
    return {"A": normal_bf16(g[0], (m, k)), "B": normal_bf16(g[1], (n, k))}


def rowwise(M=8192, N=4096, K=4096, seed=SEED_BASE + 1):
    g = streams(seed, 4)
    x = g[0].standard_normal((M, K), dtype=np.float32)
    cols = g[1].choice(K, size=int(round(0.01 * K)), replace=False)
    x[:, cols] *= np.float32(50.0)
    return {"x": f32_to_bf16_bits(x), "outlier_cols": np.sort(cols),
            "w": normal_bf16(g[2], (N, K), 0.02),
            "bias": normal_bf16(g[3], (N,), 0.01)}


def blockwise(M=16640, N=5120, K=8192, seed=SEED_BASE + 2):
    """Forward input@weight.t() and grad_input grad_output@weight operands."""
    g = streams(seed, 3)
    return {"input": normal_bf16(g[0], (M, K)),
            "weight": normal_bf16(g[1], (N, K), 0.02),
            "grad_output": normal_bf16(g[2], (M, N))}


def grad_weight(T=16640, N_out=5120, K_in=8192, seed=SEED_BASE + 3):
    g = streams(seed, 2)
    return {"grad_output": normal_bf16(g[0], (T, N_out), 1e-3),
            "input": normal_bf16(g[1], (T, K_in))}


def grouped(E=64, N=1408, K=2048, M_total=16384, seed=SEED_BASE + 4):
    g = streams(seed, 3)
    sizes = g[2].multinomial(M_total, [1.0 / E] * E)
    offs = np.cumsum(sizes).astype(np.int32)
    return {"act": normal_bf16(g[0], (M_total, K)),
            "W": normal_bf16(g[1], (E, N, K), 0.02),
            "sizes": sizes.astype(np.int64), "offs": offs}


def grouped_backward(E=64, N=1408, K=2048, M_total=16384, seed=SEED_BASE + 5):
    fwd = grouped(E=E, N=N, K=K, M_total=M_total)
    g = streams(seed, 1)
    fwd["grad_output"] = normal_bf16(g[0], (M_total, N), 1e-3)
    return fwd
