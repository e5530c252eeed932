"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.

Every call below is made with arguments that fail validation, so nothing is
ever enqueued (fake non-null pointers are never dereferenced)."""

import ctypes
import os
import re

import pytest

from precision_matmul_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8mm.h")
FAKE = 0x1000          # 16-byte aligned, never dereferenced


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_\w+|fp8mm_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfp8mm.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) == 17, names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_recipe_pair_table(lib):
    R = _lib.RECIPES
    ok = {("tensorwise", "tensorwise"), ("rowwise", "rowwise"), ("1x128", "128x128"), ("1x128", "128x1")}
    for a in R:
        for b in R:
            for layout in (0, 1):
                want = (a, b) in ok or ((a, b) == ("mxfp8", "mxfp8") and layout == 0)
                assert lib.fp8mm_recipe_pair_supported(R[a], R[b], layout) == int(want), (a, b, layout)
    assert lib.fp8mm_recipe_pair_supported(0, 0, 7) == 0


def _mm(lib, **kw):
    a = dict(A=FAKE, M=64, K=256, lda=256, B=FAKE, N=64, ldb=256, layout=0, sa=FAKE, ra=0, sb=FAKE, rb=0,
             bias=None, od=0, out=FAKE, ldo=64, st=None)
    a.update(kw)
    return lib.fp8_scaled_mm(a["A"], a["M"], a["K"], a["lda"], a["B"], a["N"], a["ldb"], a["layout"], a["sa"],
                             a["ra"], a["sb"], a["rb"], a["bias"], a["od"], a["out"], a["ldo"], a["st"])


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), _lib.EINVAL),
    (dict(out=None), _lib.EINVAL),
    (dict(sb=None), _lib.EINVAL),
    (dict(M=-1), _lib.EINVAL),
    (dict(K=100, lda=112, ldb=112), _lib.EINVAL),                 # K % 16
    (dict(lda=128), _lib.EINVAL),                                  # lda < K
    (dict(lda=264), _lib.EINVAL),                                  # lda % 16
    (dict(ldb=200), _lib.EINVAL),
    (dict(ldo=32), _lib.EINVAL),
    (dict(A=FAKE + 8), _lib.EINVAL),                               # alignment
    (dict(ra=9), _lib.EINVAL),                                     # unknown enum
    (dict(layout=3), _lib.EINVAL),
    (dict(od=5), _lib.EINVAL),
    (dict(ra=1, rb=0), _lib.ENOTIMPL),                             # rowwise x tensorwise
    (dict(ra=3, rb=2), _lib.ENOTIMPL),                             # 128x128 x 1x128
    (dict(ra=2, rb=3, K=144, lda=144, ldb=144), _lib.EINVAL),      # blockwise K % 128
    (dict(ra=2, rb=3, N=100, ldo=100), _lib.EINVAL),               # 128x128 needs N % 128
    (dict(ra=0, rb=0, layout=1, ldb=32), _lib.EINVAL),             # KN: ldb >= N
    (dict(ra=5, rb=5, layout=1), _lib.ENOTIMPL),                   # mxfp8 with B stored [K, N]
    (dict(ra=5, rb=5, K=160, lda=160, ldb=160), _lib.EINVAL),      # mxfp8 K % 128
    (dict(ra=5, rb=2), _lib.ENOTIMPL),                             # mxfp8 x 1x128
    (dict(ra=6), _lib.EINVAL),                                     # unknown enum
    (dict(ra=2, rb=3, M=2 ** 30), _lib.EINVAL),                    # 1x128 scales above 2^30 elements
])
def test_scaled_mm_rejects_before_launch(lib, kw, code):
    assert _mm(lib, **kw) == code
    assert lib.fp8mm_last_error().decode()


@pytest.mark.parametrize("kw", [
    dict(ra=2, rb=3, M=2 ** 30, N=128, ldo=128, K=128, lda=128, ldb=128),        # 1x128 scales: (K/128) M
    dict(ra=2, rb=4, N=2 ** 30, ldo=2 ** 30, K=128, lda=128, ldb=128),           # 128x1 scales: (K/128) N
])
def test_scale_arrays_of_exactly_2_30_elements_are_rejected(lib, kw):
    # each scale array is addressed through one 32-bit byte range: 4 x 2^30
    # bytes do not fit, so the limit is exclusive
    assert _mm(lib, **kw) == _lib.EINVAL
    assert "2^30" in lib.fp8mm_last_error().decode()


def test_status_maps_to_python_exceptions(lib):
    assert _mm(lib, ra=1, rb=0) == _lib.ENOTIMPL
    with pytest.raises(NotImplementedError):
        _lib.check(_lib.ENOTIMPL, "x")
    with pytest.raises(ValueError):
        _lib.check(_lib.EINVAL, "x")
    with pytest.raises(RuntimeError):
        _lib.check(_lib.ERUNTIME, "x")


def test_grouped_requires_offsets_and_checks_shapes(lib):
    f = lib.fp8_scaled_grouped_mm
    # A, M_total, K, B, E, N, offsets, sa, sb, bias, od, out, ldo, stream
    assert f(FAKE, 64, 256, FAKE, 4, 64, None, FAKE, FAKE, None, 0, FAKE, 64, None) == _lib.EINVAL
    assert "offsets" in lib.fp8mm_last_error().decode()
    assert f(FAKE, 64, 100, FAKE, 4, 64, FAKE, FAKE, FAKE, None, 0, FAKE, 64, None) == _lib.EINVAL
    assert f(FAKE, 64, 256, FAKE, -1, 64, FAKE, FAKE, FAKE, None, 0, FAKE, 64, None) == _lib.EINVAL
    assert f(FAKE, 64, 256, FAKE, 4, 64, FAKE, FAKE, FAKE, None, 0, FAKE, 32, None) == _lib.EINVAL
    assert f(FAKE, 64, 256, FAKE, 4, 64, FAKE, FAKE, FAKE, None, 9, FAKE, 64, None) == _lib.EINVAL


def test_grouped_v2_checks_recipes_and_shapes(lib):
    f = lib.fp8_scaled_grouped_mm_v2

    def call(**kw):
        a = dict(A=FAKE, M=64, K=256, B=FAKE, E=4, N=128, layout=0, offs=FAKE, sa=FAKE, ra=2, sb=FAKE, rb=3,
                 bias=None, per_expert=0, od=0, out=FAKE, ldo=128)
        a.update(kw)
        return f(a["A"], a["M"], a["K"], a["B"], a["E"], a["N"], a["layout"], a["offs"], a["sa"], a["ra"], a["sb"],
                 a["rb"], a["bias"], a["per_expert"], a["od"], a["out"], a["ldo"], None)

    assert call(offs=None) == _lib.EINVAL
    assert call(ra=0, rb=0) == _lib.ENOTIMPL                   # tensorwise grouped
    assert call(ra=2, rb=4) == _lib.ENOTIMPL                   # 1x128 x 128x1 grouped
    assert call(ra=5, rb=5) == _lib.ENOTIMPL                   # mxfp8 grouped
    assert call(ra=7) == _lib.EINVAL                           # unknown enum
    assert call(K=192) == _lib.EINVAL                          # blockwise K % 128
    assert call(N=64, ldo=64) == _lib.EINVAL                   # 128x128 needs N % 128
    assert call(layout=2) == _lib.EINVAL
    assert call(ra=1, rb=1, layout=1, N=24, ldo=24) == _lib.EINVAL   # B stored [K, N]: N % 16
    assert call(ldo=64) == _lib.EINVAL
    assert call(A=FAKE + 8) == _lib.EINVAL
    assert call(E=-1) == _lib.EINVAL
    assert call(E=(1 << 16) + 1) == _lib.EINVAL                # expert count cap
    assert "E <= 2^16" in lib.fp8mm_last_error().decode()
    assert call(per_expert=2) == _lib.EINVAL                   # bias form: 0 ([N]) or 1 ([E, N])
    assert "bias_per_expert" in lib.fp8mm_last_error().decode()
    assert call(M=0) == _lib.OK                                # empty: nothing to do
    assert call(M=0, bias=FAKE, per_expert=1) == _lib.OK


def test_grouped_weight_gradient_entries_check_capacity(lib):
    assert lib.fp8mm_grouped_runs_capacity(16384, 64) == 128 + 64
    assert lib.fp8mm_grouped_runs_capacity(127, 3) == 3
    assert lib.fp8mm_grouped_runs_capacity(-1, 3) == -1
    q = lib.fp8_quantize_grouped_128x1
    # x, T, C, ld_x, offsets, E, q_t, ld_q, scale, stream
    cap = 128 * (1000 // 128 + 8)
    assert q(FAKE, 1000, 64, 64, FAKE, 8, FAKE, cap - 16, FAKE, None) == _lib.EINVAL    # ld_q below the runs
    assert q(FAKE, 1000, 64, 64, None, 8, FAKE, cap, FAKE, None) == _lib.EINVAL         # offsets NULL
    assert q(FAKE, 1000, 72, 72, FAKE, 8, FAKE, cap, FAKE, None) == _lib.EINVAL         # C % 16
    assert q(FAKE, 1000, 64, 64, FAKE, 8, FAKE, cap + 8, FAKE, None) == _lib.EINVAL     # ld_q % 16
    assert q(FAKE, 1000, 64, 64, FAKE, 8, FAKE, cap, None, None) == _lib.EINVAL         # scale NULL
    assert q(FAKE, 1000, 64, 64, FAKE, -1, FAKE, cap, FAKE, None) == _lib.EINVAL
    assert q(FAKE, 1000, 64, 64, FAKE, (1 << 16) + 1, FAKE, cap, FAKE, None) == _lib.EINVAL
    assert "2^16" in lib.fp8mm_last_error().decode()
    g = lib.fp8_grouped_linear_grad_weight
    # gt_q, N_out, gt_scale, xt_q, K_in, xt_scale, ld, T, offsets, E, od, grad_w, stream
    assert g(FAKE, 64, FAKE, FAKE, 64, FAKE, cap - 128, 1000, FAKE, 8, 0, FAKE, None) == _lib.EINVAL
    assert g(FAKE, 64, FAKE, FAKE, 64, FAKE, cap, 1000, None, 8, 0, FAKE, None) == _lib.EINVAL
    assert g(FAKE, 64, FAKE, FAKE, 64, FAKE, cap, 1000, FAKE, 8, 4, FAKE, None) == _lib.EINVAL
    assert g(FAKE + 4, 64, FAKE, FAKE, 64, FAKE, cap, 1000, FAKE, 8, 0, FAKE, None) == _lib.EINVAL
    assert g(FAKE, 64, None, FAKE, 64, FAKE, cap, 1000, FAKE, 8, 0, FAKE, None) == _lib.EINVAL
    assert g(FAKE, 0, FAKE, FAKE, 64, FAKE, cap, 1000, FAKE, 8, 0, FAKE, None) == _lib.OK
    assert g(FAKE, 64, FAKE, FAKE, 64, FAKE, cap, 1000, FAKE, (1 << 16) + 1, 0, FAKE, None) == _lib.EINVAL
    assert "E <= 2^16" in lib.fp8mm_last_error().decode()
    big = 1 << 22                                                 # ld / 128 = 32768 runs
    assert g(FAKE, 1 << 16, FAKE, FAKE, 64, FAKE, big, 1000, FAKE, 8, 0, FAKE, None) == _lib.EINVAL   # scales


def test_grouped_dual_quantizer_rejects_before_launch(lib):
    d = lib.fp8_quantize_grouped_dual
    cap = 128 * (1000 // 128 + 8)
    # x, T, C, ld_x, offsets, E, q_row, ld_q_row, scale_row, q_t, ld_q, scale_t, stream
    assert d(FAKE, 1000, 64, 64, FAKE, 8, FAKE, 64, FAKE, FAKE, cap, FAKE, None) == _lib.EINVAL      # C % 128
    assert d(FAKE, 1000, 128, 128, FAKE, 8, FAKE, 112, FAKE, FAKE, cap, FAKE, None) == _lib.EINVAL   # ld_q_row
    assert d(FAKE, 1000, 128, 128, FAKE, 8, None, 128, FAKE, FAKE, cap, FAKE, None) == _lib.EINVAL   # q_row NULL
    assert d(FAKE, 1000, 128, 128, FAKE, 8, FAKE + 8, 128, FAKE, FAKE, cap, FAKE, None) == _lib.EINVAL
    assert d(FAKE, 1000, 128, 128, FAKE, 8, FAKE, 128, FAKE, FAKE, cap - 128, FAKE, None) == _lib.EINVAL
    assert d(FAKE, 1000, 128, 128, None, 8, FAKE, 128, FAKE, FAKE, cap, FAKE, None) == _lib.EINVAL   # offsets
    assert d(FAKE, 1000, 128, 128, FAKE, (1 << 16) + 1, FAKE, 128, FAKE, FAKE, cap, FAKE, None) == _lib.EINVAL


def test_quantizers_reject_before_launch(lib):
    # x, rows, cols, ld_x, q, ld_q, scale, stream
    assert lib.fp8_quantize_tensorwise(None, 4, 16, 16, FAKE, 16, FAKE, None) == _lib.EINVAL
    assert lib.fp8_quantize_tensorwise(FAKE, 4, 20, 24, FAKE, 32, FAKE, None) == _lib.EINVAL   # cols % 16
    assert lib.fp8_quantize_tensorwise(FAKE, 4, 16, 12, FAKE, 16, FAKE, None) == _lib.EINVAL   # ld_x < cols
    assert lib.fp8_quantize_tensorwise(FAKE, 4, 16, 16, FAKE, 8, FAKE, None) == _lib.EINVAL    # ld_q
    assert lib.fp8_quantize_rowwise(FAKE, 4, 16, 16, ctypes.c_float(-1.0), FAKE, 16, FAKE, None) == _lib.EINVAL
    assert lib.fp8_quantize_rowwise(FAKE, 4, 16, 16, ctypes.c_float(float("nan")), FAKE, 16, FAKE, None) == _lib.EINVAL
    qb = lib.fp8_quantize_blockwise
    # x, rows, cols, ld_x, br, bc, transpose, q, ld_q, scale, stream
    assert qb(FAKE, 128, 128, 128, 64, 64, 0, FAKE, 128, FAKE, None) == _lib.ENOTIMPL
    assert qb(FAKE, 128, 128, 128, 1, 128, 1, FAKE, 128, FAKE, None) == _lib.ENOTIMPL          # transpose only 128x1
    assert qb(FAKE, 100, 128, 128, 128, 128, 0, FAKE, 128, FAKE, None) == _lib.EINVAL          # rows % 128
    assert qb(FAKE, 128, 144, 144, 1, 128, 0, FAKE, 144, FAKE, None) == _lib.EINVAL            # cols % 128
    assert qb(FAKE, 256, 64, 64, 128, 1, 1, FAKE, 128, FAKE, None) == _lib.EINVAL              # ld_q < rows (T)
    assert qb(FAKE, 256, 64, 64, 128, 1, 2, FAKE, 256, FAKE, None) == _lib.EINVAL              # transpose flag


def test_dual_quantizer_rejects_before_launch(lib):
    qd = lib.fp8_quantize_blockwise_dual
    # x, rows, cols, ld_x, q_row, ld_q_row, scale_row, q_col_t, ld_q_col, scale_col, stream
    assert qd(FAKE, 200, 256, 256, FAKE, 256, FAKE, FAKE, 208, FAKE, None) == _lib.EINVAL       # rows % 128
    assert qd(FAKE, 256, 144, 144, FAKE, 144, FAKE, FAKE, 256, FAKE, None) == _lib.EINVAL       # cols % 128
    assert qd(FAKE, 256, 256, 256, FAKE, 128, FAKE, FAKE, 256, FAKE, None) == _lib.EINVAL       # ld_q_row < cols
    assert qd(FAKE, 256, 256, 256, FAKE, 256, FAKE, FAKE, 128, FAKE, None) == _lib.EINVAL       # ld_q_col < rows
    assert qd(FAKE, 256, 256, 256, FAKE, 256, FAKE, None, 256, FAKE, None) == _lib.EINVAL       # q_col_t NULL
    assert qd(FAKE, 256, 256, 256, FAKE, 256, FAKE, FAKE + 8, 256, FAKE, None) == _lib.EINVAL   # alignment
    assert qd(FAKE, 256, 256, 256, FAKE, 256, FAKE, FAKE, 256, None, None) == _lib.EINVAL       # scale_col NULL


def test_mx_quantizer_rejects_before_launch(lib):
    qm = lib.fp8_quantize_mx
    # x, rows, cols, ld_x, q, ld_q, scale, stream
    assert qm(FAKE, 4, 48, 48, FAKE, 48, FAKE, None) == _lib.EINVAL        # cols % 32
    assert qm(FAKE, 4, 64, 64, FAKE, 48, FAKE, None) == _lib.EINVAL        # ld_q < cols
    assert qm(FAKE, 4, 64, 64, FAKE, 64, None, None) == _lib.EINVAL        # scale NULL
    assert qm(FAKE, 4, 64, 64, FAKE + 4, 64, FAKE, None) == _lib.EINVAL    # alignment


def test_call_forms_validate_through_scaled_mm(lib):
    # grad_input with K_in not a multiple of 128 under 128x128 weights -> EINVAL
    assert lib.fp8_linear_grad_input(FAKE, 64, 256, FAKE, 2, FAKE, 200, FAKE, 3, 0, FAKE, None) == _lib.EINVAL
    # grad_weight with T not a multiple of 128 -> EINVAL
    assert lib.fp8_linear_grad_weight(FAKE, 64, 200, FAKE, FAKE, 64, FAKE, 0, FAKE, None) == _lib.EINVAL
    # forward with an unsupported pair -> ENOTIMPL
    assert lib.fp8_linear_forward(FAKE, 64, 256, FAKE, 2, FAKE, 64, FAKE, 1, None, 0, FAKE, None) == _lib.ENOTIMPL


def test_product_path_does_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "precision_matmul_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("the oracle", ""), f


def test_header_is_plain_c_and_the_library_links_from_c(tmp_path):
    """The boundary is usable from C: the header compiles as C99 with
    warnings on, and a C program linked against libfp8mm.so makes host-only
    calls (the recipe table, an argument rejection and its message)."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "fp8mm.h"
int main(void) {
  if (!fp8mm_recipe_pair_supported(FP8MM_BLOCK_1x128, FP8MM_BLOCK_128x128, FP8MM_B_NK)) return 1;
  if (fp8mm_recipe_pair_supported(FP8MM_ROWWISE, FP8MM_TENSORWISE, FP8MM_B_NK)) return 2;
  fp8mm_status st = fp8_scaled_mm(0, 64, 256, 256, 0, 64, 256, FP8MM_B_NK, 0, FP8MM_TENSORWISE, 0,
                                  FP8MM_TENSORWISE, 0, FP8MM_OUT_BF16, 0, 64, 0);
  if (st != FP8MM_EINVAL || strlen(fp8mm_last_error()) == 0) return 3;
  if (fp8mm_grouped_runs_capacity(16384, 64) != 192) return 4;
  printf("ok\n");
  return 0;
}
''')
    exe = tmp_path / "abi"
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
           "-I/opt/rocm/include", str(src), f"-L{libdir}", "-lfp8mm", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (run.returncode, run.stdout, run.stderr)
