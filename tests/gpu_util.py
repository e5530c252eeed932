"""Shared helpers of the GPU parity tests (marshalling only)."""

import numpy as np
import torch

DEV = torch.device("cuda:0")

# GEMM tolerance of the method's parity bar: relative Frobenius error <= 1e-3
# and elementwise |err| <= 4e-3 * max|ref|, against the float64 oracle rounded
# once to the output dtype.
TOL_FRO = 1e-3
TOL_MAX = 4e-3


def bf16_dev(bits):
    """numpy uint16 bf16 bit patterns -> device torch.bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def out_f64(t):
    """GPU output (bf16 or fp32) -> float64 numpy."""
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def say(msg):
    print(msg, flush=True)
