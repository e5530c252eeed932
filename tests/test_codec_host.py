"""Host build of the quantizers' quotient code (csrc/fp8_codec.hpp), checked
exhaustively against IEEE float division over the quantizers' input domain.

The cast divides each value by its group's scale (DiffSynth-Engine PR #160,
"per-token scaling for fp8 linear", "Highlights": the per-token scale with a
small epsilon; pytorch/ao PR #2784, "improve fp8 blockwise gemm perf": the
blockwise groups) and must produce the correctly rounded float32 quotient
before the E4M3 rounding.  The kernels compute it from the reciprocal and
one FMA correction; tests/host/div_by_scale_check.cpp compiles that same
header for the host and compares every (amax, x) pair: every positive finite
bf16 amax, both scale forms, every bf16 x of either sign with |x| <= amax
(2.1e9 pairs, a few seconds on 8 cores).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "div_by_scale_check.cpp")
CSRC = os.path.join(ROOT, "precision_matmul_amd", "csrc")


def _clang():
    for exe in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if exe and os.path.exists(exe):
            return exe
    pytest.fail("no clang++ to build the host check of fp8_codec.hpp")


def test_div_by_scale_matches_ieee_division_exhaustively(tmp_path):
    exe = tmp_path / "div_by_scale_check"
    # -ffp-contract=off as well as the header's own pragma: the check's IEEE
    # reference x / s must not be fused into anything either
    cmd = [_clang(), "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", "-x", "c++", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", f"-I{CSRC}", SRC, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(max(1, min(8, len(os.sched_getaffinity(0))))))
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout)
    got = dict(kv.split("=") for kv in r.stdout.split())
    assert int(got["pairs"]) == 2096505890, got           # every pair of the domain was visited
    assert got["differ_big"] == "0" and got["differ_code"] == "0" and got["wrong_switch"] == "0", got
    assert r.returncode == 0
