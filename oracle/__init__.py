"""CPU oracle for the FP8 scaled matrix multiply.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

The oracle is a plain, slow, obviously-correct restatement of what the method
computes, written from the definitions:

* ``e4m3``  - the 256-code FP8 E4M3 ("e4m3fn") decode table and a
  round-to-nearest-even, saturating encoder (OCP 8-bit floating point
  specification, E4M3 encoding).
* ``quant`` - dynamic quantization: group amax, scale = amax / 448, then
  ``code = enc(x / scale)`` for the tensorwise, rowwise (per-token, with an
  epsilon) and blockwise (1x128, 128x128, 128x1) groupings.
* ``gemm``  - the scaled matrix multiply evaluated as "dequantize both operands,
  then one matmul" in float64, rounded once to the output dtype; the grouped
  (MoE) variants (forward, input gradient, per-expert weight gradient) and the
  three linear call forms are reductions to it.

It shares no code, tables or constants with the HIP library, and imports
nothing from it.  Every floating-point step is numpy float32 (where the method
fixes fp32) or float64.
"""

from . import e4m3, quant, gemm  # noqa: F401
