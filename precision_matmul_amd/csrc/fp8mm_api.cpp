// C ABI of the FP8 scaled-GEMM library: host-side argument validation, the
// recipe-pair table and kernel dispatch.  Nothing here allocates, frees or
// synchronizes; every accepted call only enqueues kernels on the caller's
// stream.
//
// The explicit per-operand recipe checked against a table of accepted pairs,
// and the split of failures into value errors, not-implemented errors and
// runtime errors, follow the design discussed in pytorch PR #164141 ("Add
// _scaled_mm_v2 API").  Unsupported combinations fail loudly instead of
// falling back to a dequantized matmul (pytorch/ao PR #4390, "Add
// _grouped_mm dispatch handler to Float8Tensor", review).
#include <stdarg.h>
#include <stdio.h>

#include "fp8mm.h"
#include "launch.hpp"
#include "quant_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

fp8mm_status fail(fp8mm_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

fp8mm_status ok() {
  g_last_error[0] = '\0';
  return FP8MM_OK;
}

fp8mm_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FP8MM_ERUNTIME, "%s: HIP error %d (%s)", what, int(e), hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Offsets are formed in 32-bit buffer descriptors: keep one tile's span of
// an operand below 2^31 bytes, and a scale array below 2^32 bytes.
constexpr int64_t kMaxLd = int64_t(1) << 22;
constexpr int64_t kMaxScales = int64_t(1) << 30;   // exclusive: 4 * count must fit in 32 bits
// Every workgroup of a grouped kernel scans the E offsets to find its expert,
// and the grouped grids grow with E: cap E so that a call stays a bounded
// amount of work.
constexpr int64_t kMaxExperts = int64_t(1) << 16;

struct PairRule {
  fp8mm_recipe a;
  fp8mm_recipe b;
  fp8mm::Epi epi;
  const char* name;
};

// The accepted (recipe_a, recipe_b) pairs.  Each operand names its own
// recipe; nothing is inferred from scale shapes.
constexpr PairRule kPairs[] = {
    {FP8MM_TENSORWISE, FP8MM_TENSORWISE, fp8mm::Epi::Tensor, "tensorwise_tensorwise"},
    {FP8MM_ROWWISE, FP8MM_ROWWISE, fp8mm::Epi::Row, "rowwise_rowwise"},
    {FP8MM_BLOCK_1x128, FP8MM_BLOCK_128x128, fp8mm::Epi::Block128x128, "blockwise_1x128_128x128"},
    {FP8MM_MXFP8, FP8MM_MXFP8, fp8mm::Epi::MX, "mxfp8_mxfp8"},
    {FP8MM_BLOCK_1x128, FP8MM_BLOCK_128x1, fp8mm::Epi::Block128x1, "blockwise_1x128_128x1"},
};

const PairRule* find_pair(fp8mm_recipe a, fp8mm_recipe b) {
  for (const PairRule& r : kPairs)
    if (r.a == a && r.b == b) return &r;
  return nullptr;
}

bool valid_recipe(int r) { return r >= FP8MM_TENSORWISE && r <= FP8MM_MXFP8; }

}  // namespace

extern "C" {

const char* fp8mm_last_error(void) { return g_last_error; }

int fp8mm_recipe_pair_supported(fp8mm_recipe recipe_a, fp8mm_recipe recipe_b, fp8mm_b_layout b_layout) {
  if (b_layout != FP8MM_B_NK && b_layout != FP8MM_B_KN) return 0;
  const PairRule* rule = find_pair(recipe_a, recipe_b);
  if (rule && rule->epi == fp8mm::Epi::MX && b_layout != FP8MM_B_NK) return 0;
  return rule != nullptr ? 1 : 0;
}

// ----------------------------------------------------------------- quantize

static fp8mm_status check_quant_common(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                       const uint8_t* q, const float* scale) {
  if (rows < 0 || cols < 0) return fail(FP8MM_EINVAL, "negative shape [%lld, %lld]", (long long)rows, (long long)cols);
  // x and q may be NULL for an empty matrix; whether scale may be NULL
  // depends on whether the recipe writes any scale (checked by the caller).
  if (rows > 0 && cols > 0 && (!x || !q))
    return fail(FP8MM_EINVAL, "null pointer (x=%p q=%p)", x, (const void*)q);
  (void)scale;
  if (cols % 16 != 0) return fail(FP8MM_EINVAL, "cols (%lld) must be a multiple of 16", (long long)cols);
  if (ld_x < cols || ld_x % 8 != 0 || ld_x > kMaxLd)
    return fail(FP8MM_EINVAL, "ld_x (%lld) must be >= cols (%lld), a multiple of 8 and <= 2^22", (long long)ld_x, (long long)cols);
  if (!aligned16(x) || !aligned16(q)) return fail(FP8MM_EINVAL, "x and q must be 16-byte aligned");
  if (rows > (int64_t(1) << 31) - 1 || cols > (int64_t(1) << 31) - 1) return fail(FP8MM_EINVAL, "rows and cols must be < 2^31");
  return FP8MM_OK;
}

fp8mm_status fp8_quantize_tensorwise(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                                     int64_t ld_q, float* scale, hipStream_t stream) {
  fp8mm_status st = check_quant_common(x, rows, cols, ld_x, q, scale);
  if (st != FP8MM_OK) return st;
  if (!scale) return fail(FP8MM_EINVAL, "scale must not be NULL");
  if (ld_q < cols || ld_q % 16 != 0) return fail(FP8MM_EINVAL, "ld_q (%lld) must be >= cols and a multiple of 16", (long long)ld_q);
  return from_hip(fp8mm::launch_quant_tensorwise(static_cast<const uint16_t*>(x), rows, cols, ld_x, q, ld_q, scale, stream),
                  "fp8_quantize_tensorwise");
}

fp8mm_status fp8_quantize_rowwise(const void* x, int64_t rows, int64_t cols, int64_t ld_x, float eps, uint8_t* q,
                                  int64_t ld_q, float* scale, hipStream_t stream) {
  fp8mm_status st = check_quant_common(x, rows, cols, ld_x, q, scale);
  if (st != FP8MM_OK) return st;
  if (!scale && rows > 0) return fail(FP8MM_EINVAL, "scale must not be NULL");
  if (ld_q < cols || ld_q % 16 != 0) return fail(FP8MM_EINVAL, "ld_q (%lld) must be >= cols and a multiple of 16", (long long)ld_q);
  if (!(eps >= 0.0f) || eps != eps || eps > 1e30f) return fail(FP8MM_EINVAL, "eps must be a finite value >= 0");
  return from_hip(fp8mm::launch_quant_rowwise(static_cast<const uint16_t*>(x), rows, cols, ld_x, eps, q, ld_q, scale, stream),
                  "fp8_quantize_rowwise");
}

fp8mm_status fp8_quantize_blockwise(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int block_rows,
                                    int block_cols, int transpose_out, uint8_t* q, int64_t ld_q, float* scale,
                                    hipStream_t stream) {
  fp8mm_status st = check_quant_common(x, rows, cols, ld_x, q, scale);
  if (st != FP8MM_OK) return st;
  if (!scale && rows > 0 && cols > 0) return fail(FP8MM_EINVAL, "scale must not be NULL");
  const bool b1x128 = block_rows == 1 && block_cols == 128;
  const bool b128x128 = block_rows == 128 && block_cols == 128;
  const bool b128x1 = block_rows == 128 && block_cols == 1;
  if (!b1x128 && !b128x128 && !b128x1)
    return fail(FP8MM_ENOTIMPL, "block shape (%d, %d) is not one of (1,128), (128,128), (128,1)", block_rows, block_cols);
  if (transpose_out != 0 && transpose_out != 1) return fail(FP8MM_EINVAL, "transpose_out must be 0 or 1");
  if (transpose_out && !b128x1) return fail(FP8MM_ENOTIMPL, "transpose_out is only implemented for block (128, 1)");
  if (rows % block_rows != 0 || cols % block_cols != 0)
    return fail(FP8MM_EINVAL, "shape [%lld, %lld] is not a multiple of block (%d, %d)", (long long)rows, (long long)cols,
                block_rows, block_cols);
  const int64_t q_width = transpose_out ? rows : cols;
  if (ld_q < q_width || ld_q % 16 != 0 || ld_q > kMaxLd)
    return fail(FP8MM_EINVAL, "ld_q (%lld) must be >= %lld and a multiple of 16", (long long)ld_q, (long long)q_width);
  return from_hip(fp8mm::launch_quant_blockwise(static_cast<const uint16_t*>(x), rows, cols, ld_x, block_rows, block_cols,
                                                transpose_out, q, ld_q, scale, stream),
                  "fp8_quantize_blockwise");
}

fp8mm_status fp8_quantize_mx(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                             uint8_t* scale, hipStream_t stream) {
  fp8mm_status st = check_quant_common(x, rows, cols, ld_x, q, nullptr);
  if (st != FP8MM_OK) return st;
  if (!scale && rows > 0 && cols > 0) return fail(FP8MM_EINVAL, "scale must not be NULL");
  if (cols % 32 != 0) return fail(FP8MM_EINVAL, "cols (%lld) must be a multiple of 32", (long long)cols);
  if (ld_q < cols || ld_q % 16 != 0 || ld_q > kMaxLd)
    return fail(FP8MM_EINVAL, "ld_q (%lld) must be >= cols (%lld) and a multiple of 16", (long long)ld_q,
                (long long)cols);
  return from_hip(fp8mm::launch_quant_mx(static_cast<const uint16_t*>(x), rows, cols, ld_x, q, ld_q, scale, stream),
                  "fp8_quantize_mx");
}

fp8mm_status fp8_quantize_blockwise_dual(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q_row,
                                         int64_t ld_q_row, float* scale_row, uint8_t* q_col_t, int64_t ld_q_col,
                                         float* scale_col, hipStream_t stream) {
  fp8mm_status st = check_quant_common(x, rows, cols, ld_x, q_row, scale_row);
  if (st != FP8MM_OK) return st;
  if (rows > 0 && cols > 0 && (!q_col_t || !scale_row || !scale_col))
    return fail(FP8MM_EINVAL, "null pointer argument (q_col_t, scale_row and scale_col are required)");
  if (!aligned16(q_col_t)) return fail(FP8MM_EINVAL, "q_col_t must be 16-byte aligned");
  if (rows % 128 != 0 || cols % 128 != 0)
    return fail(FP8MM_EINVAL, "shape [%lld, %lld] is not a multiple of 128", (long long)rows, (long long)cols);
  if (ld_q_row < cols || ld_q_row % 16 != 0 || ld_q_row > kMaxLd)
    return fail(FP8MM_EINVAL, "ld_q_row (%lld) must be >= cols (%lld) and a multiple of 16", (long long)ld_q_row,
                (long long)cols);
  if (ld_q_col < rows || ld_q_col % 16 != 0 || ld_q_col > kMaxLd)
    return fail(FP8MM_EINVAL, "ld_q_col (%lld) must be >= rows (%lld) and a multiple of 16", (long long)ld_q_col,
                (long long)rows);
  return from_hip(fp8mm::launch_quant_blockwise_dual(static_cast<const uint16_t*>(x), rows, cols, ld_x, q_row,
                                                     ld_q_row, scale_row, q_col_t, ld_q_col, scale_col, stream),
                  "fp8_quantize_blockwise_dual");
}

// --------------------------------------------------------------------- GEMM

fp8mm_status fp8_scaled_mm(const uint8_t* A, int64_t M, int64_t K, int64_t lda, const uint8_t* B, int64_t N,
                           int64_t ldb, fp8mm_b_layout b_layout, const float* scale_a, fp8mm_recipe recipe_a,
                           const float* scale_b, fp8mm_recipe recipe_b, const void* bias, fp8mm_out_dtype out_dtype,
                           void* out, int64_t ldo, hipStream_t stream) {
  if (!valid_recipe(recipe_a) || !valid_recipe(recipe_b)) return fail(FP8MM_EINVAL, "unknown recipe value");
  if (b_layout != FP8MM_B_NK && b_layout != FP8MM_B_KN) return fail(FP8MM_EINVAL, "unknown B layout");
  if (out_dtype != FP8MM_OUT_BF16 && out_dtype != FP8MM_OUT_FP32) return fail(FP8MM_EINVAL, "unknown out_dtype");
  if (M < 0 || N < 0 || K < 0) return fail(FP8MM_EINVAL, "negative shape M=%lld N=%lld K=%lld", (long long)M, (long long)N, (long long)K);
  if (M > (int64_t(1) << 31) - 1 || N > (int64_t(1) << 31) - 1) return fail(FP8MM_EINVAL, "M and N must be < 2^31");
  const PairRule* rule = find_pair(recipe_a, recipe_b);
  if (!rule) return fail(FP8MM_ENOTIMPL, "recipe pair (%d, %d) is not implemented", int(recipe_a), int(recipe_b));
  const bool blockwise = rule->epi == fp8mm::Epi::Block128x128 || rule->epi == fp8mm::Epi::Block128x1 ||
                         rule->epi == fp8mm::Epi::MX;
  if (rule->epi == fp8mm::Epi::MX && b_layout != FP8MM_B_NK)
    return fail(FP8MM_ENOTIMPL, "mxfp8 is implemented for B stored [N, K] only");
  if (K % 16 != 0) return fail(FP8MM_EINVAL, "K (%lld) must be a multiple of 16", (long long)K);
  if (blockwise && K % 128 != 0) return fail(FP8MM_EINVAL, "%s needs K %% 128 == 0 (K=%lld)", rule->name, (long long)K);
  if (rule->epi == fp8mm::Epi::Block128x128 && N % 128 != 0)
    return fail(FP8MM_EINVAL, "%s needs N %% 128 == 0 (N=%lld)", rule->name, (long long)N);
  if (lda < K || lda % 16 != 0 || lda > kMaxLd) return fail(FP8MM_EINVAL, "lda (%lld) must be >= K, a multiple of 16 and <= 2^22", (long long)lda);
  // the kernels address each scale array through one 32-bit buffer range
  if (blockwise && ((K / 128) * M >= kMaxScales || (K / 128) * N >= kMaxScales))
    return fail(FP8MM_EINVAL, "scale arrays of (K/128) x M or (K/128) x N of 2^30 elements or more are not supported");
  const int64_t b_width = b_layout == FP8MM_B_NK ? K : N;
  if (ldb < b_width || ldb % 16 != 0 || ldb > kMaxLd)
    return fail(FP8MM_EINVAL, "ldb (%lld) must be >= %lld, a multiple of 16 and <= 2^22", (long long)ldb, (long long)b_width);
  if (b_layout == FP8MM_B_KN && K * ldb > (int64_t(1) << 31))
    return fail(FP8MM_EINVAL, "B stored [K, N] must span fewer than 2^31 bytes");
  if (ldo < N) return fail(FP8MM_EINVAL, "ldo (%lld) must be >= N (%lld)", (long long)ldo, (long long)N);
  if (M == 0 || N == 0) return ok();
  if (!scale_a || !scale_b || !out) return fail(FP8MM_EINVAL, "null pointer argument (scales and out are required)");
  if (K > 0 && (!A || !B)) return fail(FP8MM_EINVAL, "null pointer argument (A and B are required when K > 0)");
  if (!aligned16(A) || !aligned16(B)) return fail(FP8MM_EINVAL, "A and B must be 16-byte aligned");
  fp8mm::GemmProblem p{};
  p.A = A;
  p.B = B;
  p.sa = scale_a;
  p.sb = scale_b;
  p.bias = static_cast<const uint16_t*>(bias);
  p.out = out;
  p.M = M;
  p.N = N;
  p.K = K;
  p.lda = lda;
  p.ldb = ldb;
  p.ldo = ldo;
  p.epi = rule->epi;
  p.b_kn = b_layout == FP8MM_B_KN;
  p.out_bf16 = out_dtype == FP8MM_OUT_BF16;
  p.offsets = nullptr;
  p.E = 0;
  p.row_begin = 0;
  p.row_end = M;
  return from_hip(fp8mm::launch_gemm(p, stream), "fp8_scaled_mm");
}

fp8mm_status fp8_scaled_grouped_mm(const uint8_t* A, int64_t M_total, int64_t K, const uint8_t* B_EnK, int64_t E,
                                   int64_t N, const int32_t* offsets, const float* scale_a, const float* scale_b,
                                   const void* bias, fp8mm_out_dtype out_dtype, void* out, int64_t ldo,
                                   hipStream_t stream) {
  if (!offsets) return fail(FP8MM_EINVAL, "offsets are required for the grouped GEMM");
  if (out_dtype != FP8MM_OUT_BF16 && out_dtype != FP8MM_OUT_FP32) return fail(FP8MM_EINVAL, "unknown out_dtype");
  if (M_total < 0 || K < 0 || N < 0 || E < 0) return fail(FP8MM_EINVAL, "negative shape");
  if (M_total > (int64_t(1) << 31) - 1 || N > (int64_t(1) << 31) - 1 || E > kMaxExperts)
    return fail(FP8MM_EINVAL, "M_total and N must be < 2^31 and E <= 2^16");
  if (K % 16 != 0 || K > kMaxLd) return fail(FP8MM_EINVAL, "K (%lld) must be a multiple of 16 and <= 2^22", (long long)K);
  if (ldo < N) return fail(FP8MM_EINVAL, "ldo (%lld) must be >= N (%lld)", (long long)ldo, (long long)N);
  if (M_total == 0 || N == 0 || E == 0) return ok();
  if (!scale_a || !scale_b || !out) return fail(FP8MM_EINVAL, "null pointer argument (scales and out are required)");
  if (K > 0 && (!A || !B_EnK)) return fail(FP8MM_EINVAL, "null pointer argument (A and B_EnK are required when K > 0)");
  if (!aligned16(A) || !aligned16(B_EnK)) return fail(FP8MM_EINVAL, "A and B_EnK must be 16-byte aligned");
  fp8mm::GemmProblem p{};
  p.A = A;
  p.B = B_EnK;
  p.sa = scale_a;
  p.sb = scale_b;
  p.bias = static_cast<const uint16_t*>(bias);
  p.out = out;
  p.M = M_total;
  p.N = N;
  p.K = K;
  p.lda = K;
  p.ldb = K;
  p.ldo = ldo;
  p.bias_stride_e = 0;   // one bf16 [N] bias row for every expert
  p.epi = fp8mm::Epi::Row;
  p.b_kn = false;
  p.out_bf16 = out_dtype == FP8MM_OUT_BF16;
  p.offsets = offsets;
  p.E = E;
  p.row_begin = 0;
  p.row_end = M_total;
  return from_hip(fp8mm::launch_gemm(p, stream), "fp8_scaled_grouped_mm");
}

fp8mm_status fp8_scaled_grouped_mm_v2(const uint8_t* A, int64_t M_total, int64_t K, const uint8_t* B_E, int64_t E,
                                      int64_t N, fp8mm_b_layout b_layout, const int32_t* offsets,
                                      const float* scale_a, fp8mm_recipe recipe_a, const float* scale_b,
                                      fp8mm_recipe recipe_b, const void* bias, int bias_per_expert,
                                      fp8mm_out_dtype out_dtype, void* out, int64_t ldo, hipStream_t stream) {
  if (!valid_recipe(recipe_a) || !valid_recipe(recipe_b)) return fail(FP8MM_EINVAL, "unknown recipe value");
  if (bias_per_expert != 0 && bias_per_expert != 1) return fail(FP8MM_EINVAL, "bias_per_expert must be 0 or 1");
  if (b_layout != FP8MM_B_NK && b_layout != FP8MM_B_KN) return fail(FP8MM_EINVAL, "unknown B layout");
  if (!offsets) return fail(FP8MM_EINVAL, "offsets are required for the grouped GEMM");
  if (out_dtype != FP8MM_OUT_BF16 && out_dtype != FP8MM_OUT_FP32) return fail(FP8MM_EINVAL, "unknown out_dtype");
  if (M_total < 0 || K < 0 || N < 0 || E < 0) return fail(FP8MM_EINVAL, "negative shape");
  if (M_total > (int64_t(1) << 31) - 1 || N > (int64_t(1) << 31) - 1 || E > kMaxExperts)
    return fail(FP8MM_EINVAL, "M_total and N must be < 2^31 and E <= 2^16");
  fp8mm::Epi epi;
  if (recipe_a == FP8MM_ROWWISE && recipe_b == FP8MM_ROWWISE)
    epi = fp8mm::Epi::Row;
  else if (recipe_a == FP8MM_BLOCK_1x128 && recipe_b == FP8MM_BLOCK_128x128)
    epi = fp8mm::Epi::Block128x128;
  else
    return fail(FP8MM_ENOTIMPL, "grouped recipe pair (%d, %d) is not implemented (rowwise x rowwise or "
                "1x128 x 128x128)", int(recipe_a), int(recipe_b));
  if (K % 16 != 0 || K > kMaxLd) return fail(FP8MM_EINVAL, "K (%lld) must be a multiple of 16 and <= 2^22", (long long)K);
  if (epi == fp8mm::Epi::Block128x128 && (K % 128 != 0 || N % 128 != 0))
    return fail(FP8MM_EINVAL, "1x128 x 128x128 needs K %% 128 == 0 and N %% 128 == 0 (K=%lld N=%lld)", (long long)K,
                (long long)N);
  if (epi == fp8mm::Epi::Block128x128 && (K / 128) * M_total >= kMaxScales)
    return fail(FP8MM_EINVAL, "scale_a of (K/128) x M_total of 2^30 elements or more is not supported");
  if (b_layout == FP8MM_B_KN) {
    if (N % 16 != 0 || N > kMaxLd) return fail(FP8MM_EINVAL, "B stored [K, N] needs N %% 16 == 0 and N <= 2^22");
    if (K * N > (int64_t(1) << 31)) return fail(FP8MM_EINVAL, "each expert's B stored [K, N] must span fewer than 2^31 bytes");
  }
  if (ldo < N) return fail(FP8MM_EINVAL, "ldo (%lld) must be >= N (%lld)", (long long)ldo, (long long)N);
  if (M_total == 0 || N == 0 || E == 0) return ok();
  if (!scale_a || !scale_b || !out) return fail(FP8MM_EINVAL, "null pointer argument (scales and out are required)");
  if (K > 0 && (!A || !B_E)) return fail(FP8MM_EINVAL, "null pointer argument (A and B_E are required when K > 0)");
  if (!aligned16(A) || !aligned16(B_E)) return fail(FP8MM_EINVAL, "A and B_E must be 16-byte aligned");
  fp8mm::GemmProblem p{};
  p.A = A;
  p.B = B_E;
  p.sa = scale_a;
  p.sb = scale_b;
  p.bias = static_cast<const uint16_t*>(bias);
  p.bias_stride_e = bias_per_expert ? N : 0;
  p.out = out;
  p.M = M_total;
  p.N = N;
  p.K = K;
  p.lda = K;
  p.ldb = b_layout == FP8MM_B_NK ? K : N;
  p.ldo = ldo;
  p.epi = epi;
  p.b_kn = b_layout == FP8MM_B_KN;
  p.out_bf16 = out_dtype == FP8MM_OUT_BF16;
  p.offsets = offsets;
  p.E = E;
  p.row_begin = 0;
  p.row_end = M_total;
  return from_hip(fp8mm::launch_gemm(p, stream), "fp8_scaled_grouped_mm_v2");
}

int64_t fp8mm_grouped_runs_capacity(int64_t T, int64_t E) {
  if (T < 0 || E < 0) return -1;
  return T / 128 + E;
}

fp8mm_status fp8_quantize_grouped_128x1(const void* x, int64_t T, int64_t C, int64_t ld_x, const int32_t* offsets,
                                        int64_t E, uint8_t* q_t, int64_t ld_q, float* scale, hipStream_t stream) {
  fp8mm_status st = check_quant_common(x, T, C, ld_x, q_t, scale);
  if (st != FP8MM_OK) return st;
  if (E < 0 || E > kMaxExperts) return fail(FP8MM_EINVAL, "E (%lld) must be in [0, 2^16]", (long long)E);
  if (!offsets && E > 0) return fail(FP8MM_EINVAL, "offsets are required");
  const int64_t runs = T / 128 + E;
  if (ld_q < 128 * runs || ld_q % 16 != 0 || ld_q > kMaxLd)
    return fail(FP8MM_EINVAL, "ld_q (%lld) must be >= 128 (T/128 + E) = %lld, a multiple of 16 and <= 2^22",
                (long long)ld_q, (long long)(128 * runs));
  if (C / 128 + 1 > 65535) return fail(FP8MM_EINVAL, "C (%lld) must be below 128 x 65535", (long long)C);
  if (T == 0 || C == 0 || E == 0) return ok();
  if (!scale) return fail(FP8MM_EINVAL, "scale must not be NULL");
  return from_hip(fp8mm::launch_quant_grouped_128x1(static_cast<const uint16_t*>(x), T, C, ld_x, offsets, E, q_t,
                                                    ld_q, scale, nullptr, 0, nullptr, stream),
                  "fp8_quantize_grouped_128x1");
}

fp8mm_status fp8_quantize_grouped_dual(const void* x, int64_t T, int64_t C, int64_t ld_x, const int32_t* offsets,
                                       int64_t E, uint8_t* q_row, int64_t ld_q_row, float* scale_row, uint8_t* q_t,
                                       int64_t ld_q, float* scale_t, hipStream_t stream) {
  fp8mm_status st = check_quant_common(x, T, C, ld_x, q_t, scale_t);
  if (st != FP8MM_OK) return st;
  if (E < 0 || E > kMaxExperts) return fail(FP8MM_EINVAL, "E (%lld) must be in [0, 2^16]", (long long)E);
  if (!offsets && E > 0) return fail(FP8MM_EINVAL, "offsets are required");
  if (C % 128 != 0) return fail(FP8MM_EINVAL, "C (%lld) must be a multiple of 128", (long long)C);
  const int64_t runs = T / 128 + E;
  if (ld_q < 128 * runs || ld_q % 16 != 0 || ld_q > kMaxLd)
    return fail(FP8MM_EINVAL, "ld_q (%lld) must be >= 128 (T/128 + E) = %lld, a multiple of 16 and <= 2^22",
                (long long)ld_q, (long long)(128 * runs));
  if (ld_q_row < C || ld_q_row % 16 != 0 || ld_q_row > kMaxLd)
    return fail(FP8MM_EINVAL, "ld_q_row (%lld) must be >= C (%lld), a multiple of 16 and <= 2^22",
                (long long)ld_q_row, (long long)C);
  if (C / 128 + 1 > 65535) return fail(FP8MM_EINVAL, "C (%lld) must be below 128 x 65535", (long long)C);
  if (T == 0 || C == 0 || E == 0) return ok();
  if (!q_row || !scale_row || !scale_t) return fail(FP8MM_EINVAL, "null pointer argument (q_row, scale_row, scale_t)");
  if (!aligned16(q_row)) return fail(FP8MM_EINVAL, "q_row must be 16-byte aligned");
  return from_hip(fp8mm::launch_quant_grouped_128x1(static_cast<const uint16_t*>(x), T, C, ld_x, offsets, E, q_t,
                                                    ld_q, scale_t, q_row, ld_q_row, scale_row, stream),
                  "fp8_quantize_grouped_dual");
}

fp8mm_status fp8_grouped_linear_grad_weight(const uint8_t* gt_q, int64_t N_out, const float* gt_scale,
                                            const uint8_t* xt_q, int64_t K_in, const float* xt_scale, int64_t ld,
                                            int64_t T, const int32_t* offsets, int64_t E, fp8mm_out_dtype out_dtype,
                                            void* grad_w, hipStream_t stream) {
  if (out_dtype != FP8MM_OUT_BF16 && out_dtype != FP8MM_OUT_FP32) return fail(FP8MM_EINVAL, "unknown out_dtype");
  if (N_out < 0 || K_in < 0 || T < 0 || E < 0) return fail(FP8MM_EINVAL, "negative shape");
  if (N_out > (int64_t(1) << 31) - 1 || K_in > (int64_t(1) << 31) - 1 || E > kMaxExperts)
    return fail(FP8MM_EINVAL, "N_out and K_in must be < 2^31 and E <= 2^16");
  if (!offsets && E > 0) return fail(FP8MM_EINVAL, "offsets are required");
  const int64_t runs = T / 128 + E;
  if (ld < 128 * runs || ld % 16 != 0 || ld > kMaxLd)
    return fail(FP8MM_EINVAL, "ld (%lld) must be >= 128 (T/128 + E) = %lld, a multiple of 16 and <= 2^22",
                (long long)ld, (long long)(128 * runs));
  if ((ld / 128) * N_out >= kMaxScales || (ld / 128) * K_in >= kMaxScales)
    return fail(FP8MM_EINVAL, "scale arrays of (ld/128) x N_out or (ld/128) x K_in of 2^30 elements or more are not supported");
  if (N_out == 0 || K_in == 0 || E == 0) return ok();
  const int64_t tiles = ((N_out + 127) / 128) * ((K_in + 127) / 128) * E;
  if (tiles > (int64_t(1) << 31) - 8) return fail(FP8MM_EINVAL, "too many output tiles");
  if (!gt_q || !xt_q || !gt_scale || !xt_scale || !grad_w) return fail(FP8MM_EINVAL, "null pointer argument");
  if (!aligned16(gt_q) || !aligned16(xt_q)) return fail(FP8MM_EINVAL, "gt_q and xt_q must be 16-byte aligned");
  fp8mm::GemmProblem p{};
  p.A = gt_q;
  p.B = xt_q;
  p.sa = gt_scale;
  p.sb = xt_scale;
  p.bias = nullptr;
  p.out = grad_w;
  p.M = N_out;
  p.N = K_in;
  p.K = 0;
  p.lda = ld;
  p.ldb = ld;
  p.ldo = K_in;
  p.epi = fp8mm::Epi::Block128x1;
  p.b_kn = false;
  p.out_bf16 = out_dtype == FP8MM_OUT_BF16;
  p.offsets = offsets;
  p.E = E;
  p.row_begin = 0;
  p.row_end = N_out;
  p.group_k = true;
  p.tokens = T;
  return from_hip(fp8mm::launch_gemm(p, stream), "fp8_grouped_linear_grad_weight");
}

// ------------------------------------------------------------- call forms

fp8mm_status fp8_linear_forward(const uint8_t* x_q, int64_t M, int64_t K, const float* x_scale,
                                fp8mm_recipe x_recipe, const uint8_t* w_q, int64_t N, const float* w_scale,
                                fp8mm_recipe w_recipe, const void* bias, fp8mm_out_dtype out_dtype, void* out,
                                hipStream_t stream) {
  return fp8_scaled_mm(x_q, M, K, K, w_q, N, K, FP8MM_B_NK, x_scale, x_recipe, w_scale, w_recipe, bias, out_dtype,
                       out, N, stream);
}

fp8mm_status fp8_linear_grad_input(const uint8_t* g_q, int64_t M, int64_t N_out, const float* g_scale,
                                   fp8mm_recipe g_recipe, const uint8_t* w_q, int64_t K_in, const float* w_scale,
                                   fp8mm_recipe w_recipe, fp8mm_out_dtype out_dtype, void* grad_in,
                                   hipStream_t stream) {
  // contraction over N_out: A = grad_output [M, N_out], B = weight [N_out, K_in] read as [K, N]
  return fp8_scaled_mm(g_q, M, N_out, N_out, w_q, K_in, K_in, FP8MM_B_KN, g_scale, g_recipe, w_scale, w_recipe,
                       nullptr, out_dtype, grad_in, K_in, stream);
}

fp8mm_status fp8_linear_grad_weight(const uint8_t* gt_q, int64_t N_out, int64_t T, const float* gt_scale,
                                    const uint8_t* xt_q, int64_t K_in, const float* xt_scale,
                                    fp8mm_out_dtype out_dtype, void* grad_w, hipStream_t stream) {
  return fp8_scaled_mm(gt_q, N_out, T, T, xt_q, K_in, T, FP8MM_B_NK, gt_scale, FP8MM_BLOCK_1x128, xt_scale,
                       FP8MM_BLOCK_128x1, nullptr, out_dtype, grad_w, K_in, stream);
}

}  // extern "C"
