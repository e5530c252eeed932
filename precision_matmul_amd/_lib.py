"""ctypes declarations of the C ABI in include/fp8mm.h.

Loading fails loudly when ``libfp8mm.so`` has not been built: there is no
fallback implementation anywhere in this package.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8mm.so")

OK, EINVAL, ENOTIMPL, ERUNTIME = 0, 1, 2, 3
RECIPES = {"tensorwise": 0, "rowwise": 1, "1x128": 2, "128x128": 3, "128x1": 4, "mxfp8": 5}
B_LAYOUTS = {"NK": 0, "KN": 1}
OUT_BF16, OUT_FP32 = 0, 1

# Every exported entry point: name -> (restype, argtypes).
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i = ctypes.c_int
_f = ctypes.c_float
SIGNATURES = {
    "fp8_quantize_tensorwise": (_i, [_p, _i64, _i64, _i64, _p, _i64, _p, _p]),
    "fp8_quantize_rowwise": (_i, [_p, _i64, _i64, _i64, _f, _p, _i64, _p, _p]),
    "fp8_quantize_blockwise": (_i, [_p, _i64, _i64, _i64, _i, _i, _i, _p, _i64, _p, _p]),
    "fp8_quantize_blockwise_dual": (_i, [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p]),
    "fp8_quantize_mx": (_i, [_p, _i64, _i64, _i64, _p, _i64, _p, _p]),
    "fp8_scaled_mm": (_i, [_p, _i64, _i64, _i64, _p, _i64, _i64, _i, _p, _i, _p, _i, _p, _i, _p, _i64, _p]),
    "fp8_scaled_grouped_mm": (_i, [_p, _i64, _i64, _p, _i64, _i64, _p, _p, _p, _p, _i, _p, _i64, _p]),
    "fp8_scaled_grouped_mm_v2": (_i, [_p, _i64, _i64, _p, _i64, _i64, _i, _p, _p, _i, _p, _i, _p, _i, _i, _p, _i64,
                                      _p]),
    "fp8mm_grouped_runs_capacity": (_i64, [_i64, _i64]),
    "fp8_quantize_grouped_128x1": (_i, [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p]),
    "fp8_quantize_grouped_dual": (_i, [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _i64, _p, _p]),
    "fp8_grouped_linear_grad_weight": (_i, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _p, _i64, _i, _p, _p]),
    "fp8_linear_forward": (_i, [_p, _i64, _i64, _p, _i, _p, _i64, _p, _i, _p, _i, _p, _p]),
    "fp8_linear_grad_input": (_i, [_p, _i64, _i64, _p, _i, _p, _i64, _p, _i, _i, _p, _p]),
    "fp8_linear_grad_weight": (_i, [_p, _i64, _i64, _p, _p, _i64, _p, _i, _p, _p]),
    "fp8mm_recipe_pair_supported": (_i, [_i, _i, _i]),
    "fp8mm_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load():
    """Load libfp8mm.so (once) and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m precision_matmul_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status, what):
    if status == OK:
        return
    msg = load().fp8mm_last_error().decode(errors="replace")
    text = f"{what}: {msg}"
    if status == EINVAL:
        raise ValueError(text)
    if status == ENOTIMPL:
        raise NotImplementedError(text)
    raise RuntimeError(text)
