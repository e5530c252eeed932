/*
 * fp8mm.h - C ABI of the MI355X (gfx950) FP8 scaled matrix-multiply library.
 *
 * The library computes   out = (A_fp8 * s_a) @ (B_fp8 * s_b)^T (+ bias)
 * with FP8 E4M3 ("e4m3fn", max 448) operand codes and float32 scales, and the
 * dynamic quantization pass that produces those codes and scales.
 *
 * Conventions shared by every entry point
 *   - Every pointer except the ones marked "host" is a DEVICE pointer owned by
 *     the caller.  The library never allocates, never frees and never
 *     synchronizes: each call validates its arguments on the host, enqueues
 *     kernels on `stream` and returns.  A NULL stream is the default stream.
 *   - Plain GEMMs may use their own output as scratch: when the last round
 *     of output tiles would leave most compute units idle, those rows are
 *     split along K and their fp32 partials are staged in the first rows of
 *     `out` (only when its rows are contiguous, ldo == N), which the same
 *     call overwrites with their results afterwards, in stream order.
 *   - Matrices are row-major with an explicit leading dimension in elements.
 *     bf16 is IEEE bfloat16 (uint16 storage); FP8 codes are uint8.
 *   - Arguments are checked synchronously before anything is enqueued; a bad
 *     argument returns FP8MM_EINVAL, a valid but unsupported combination
 *     FP8MM_ENOTIMPL, and nothing is launched in either case.  A HIP launch
 *     error returns FP8MM_ERUNTIME.  fp8mm_last_error() then gives a message.
 *     (Error classes follow the review of pytorch PR #164141, "Add
 *     _scaled_mm_v2 API": bad arguments are value errors, valid-but-missing
 *     paths are not-implemented errors, device failures runtime errors.)
 *   - There is no silent fallback: an unsupported path is an error, never a
 *     dequantize-and-matmul substitute (pytorch/ao PR #4390, "Add _grouped_mm
 *     dispatch handler to Float8Tensor", review).
 *   - Alignment: base pointers of x, q, A and B are 16-byte aligned, their
 *     leading dimensions are multiples of 16 bytes.
 */
#ifndef FP8MM_H
#define FP8MM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8MM_OK = 0,
  FP8MM_EINVAL = 1,   /* invalid argument (ValueError)                      */
  FP8MM_ENOTIMPL = 2, /* valid but unsupported combination (NotImplemented) */
  FP8MM_ERUNTIME = 3  /* HIP launch or device error (RuntimeError)           */
} fp8mm_status;

/* Scaling recipe of one operand (pytorch PR #164141, "Add _scaled_mm_v2
 * API": the recipe of each operand is stated explicitly, never inferred).
 * Scale arrays are dense float32, C order:
 *   TENSORWISE      [1]
 *   ROWWISE         A: [M]          B: [N]
 *   BLOCK_1x128     A only: [K/128, M]        (k-block major)
 *   BLOCK_128x128   B only: [N/128, K/128] for B_NK, [K/128, N/128] for B_KN
 *                   (the quantizer's grid of B as stored)
 *   BLOCK_128x1     B only: [K/128, N]  (128 along the contraction x 1 along
 *                   N: the weight-gradient recipe of pytorch/ao PR #2784,
 *                   "improve fp8 blockwise gemm perf", second table)
 *   MXFP8           A: uint8 [M, K/32], B (B_NK only): uint8 [N, K/32] --
 *                   E8M0 bytes (2^(byte - 127)), one per 32 elements along
 *                   K, row-major; see fp8_quantize_mx.  The "mxfp8" recipe
 *                   named by pytorch PR #164141, read as the OCP
 *                   Microscaling format with E4M3 elements.              */
typedef enum {
  FP8MM_TENSORWISE = 0,
  FP8MM_ROWWISE = 1,
  FP8MM_BLOCK_1x128 = 2,
  FP8MM_BLOCK_128x128 = 3,
  FP8MM_BLOCK_128x1 = 4,
  FP8MM_MXFP8 = 5
} fp8mm_recipe;

/* Storage of the B operand.  B_NK: B[N, K], K contiguous (a weight as
 * stored for input @ weight.t()).  B_KN: B[K, N], N contiguous (a weight as
 * stored for grad_output @ weight). */
typedef enum { FP8MM_B_NK = 0, FP8MM_B_KN = 1 } fp8mm_b_layout;

typedef enum { FP8MM_OUT_BF16 = 0, FP8MM_OUT_FP32 = 1 } fp8mm_out_dtype;

/* ---------------------------------------------------------------------------
 * Dynamic quantization.  x: bf16 [rows, cols], leading dimension ld_x.
 * q: uint8 E4M3 codes, leading dimension ld_q.  scale: float32 (layout below).
 * For every scaling group G:  amax = max|x| over G;  s = fl32(amax / 448)
 * (rowwise: fl32(fl32(amax / 448) + eps));  a scale of 0 becomes 1.0;
 * code = e4m3(fl32(x / s)) rounded to nearest-even, saturated to +-448, sign
 * kept.  The scale written is the dequantization multiplier (value = code*s).
 * Sources: per-token scale from the row's max-abs value and division by it
 * plus a small epsilon before the cast (DiffSynth-Engine PR #160, "per-token
 * scaling for fp8 linear", "Highlights"); dequantization multipliers passed
 * to the GEMM (ColossalAI PR #6419, "Fix: Handle LowLevelZeroPlugin with
 * use_fp8=True", "Forward pass").
 * Requirements: cols % 16 == 0, ld_x >= cols with ld_x % 8 == 0,
 * ld_q % 16 == 0.  rows or cols of 0 is allowed (nothing but scales written).
 * Results are bit-exact: independent of launch shape and run-to-run.
 * ------------------------------------------------------------------------- */

/* One scale for the whole tensor: scale[1].  ld_q >= cols.  Enqueues four
 * small kernels (clear, amax, cast, finalize); `scale` doubles as the amax
 * accumulator while they run. */
fp8mm_status fp8_quantize_tensorwise(const void* x, int64_t rows, int64_t cols,
                                     int64_t ld_x, uint8_t* q, int64_t ld_q,
                                     float* scale, hipStream_t stream);

/* One scale per row (per token): scale[rows].  eps >= 0 (1e-12 for the
 * per-token recipe).  ld_q >= cols. */
fp8mm_status fp8_quantize_rowwise(const void* x, int64_t rows, int64_t cols,
                                  int64_t ld_x, float eps, uint8_t* q,
                                  int64_t ld_q, float* scale,
                                  hipStream_t stream);

/* Block groups of block_rows x block_cols, one of
 *   (1, 128)   scale[cols/128, rows]            (activation, k-block major)
 *   (128, 128) scale[rows/128, cols/128]        (weight)
 *   (128, 1)   scale[rows/128, cols]            (weight-gradient operands)
 * rows % block_rows == 0 and cols % block_cols == 0.
 * transpose_out = 1 (only with (128, 1)) writes the codes transposed,
 * q[cols, rows] with ld_q >= rows (rows % 16 == 0), so that the token
 * dimension becomes the contiguous contraction dimension of the weight-
 * gradient GEMM; otherwise q[rows, cols] with ld_q >= cols. */
fp8mm_status fp8_quantize_blockwise(const void* x, int64_t rows, int64_t cols,
                                    int64_t ld_x, int block_rows,
                                    int block_cols, int transpose_out,
                                    uint8_t* q, int64_t ld_q, float* scale,
                                    hipStream_t stream);

/* MXFP8 quantization (the "mxfp8" recipe of pytorch PR #164141, "Add
 * _scaled_mm_v2 API", read as OCP Microscaling with E4M3 elements): each run
 * of 32 consecutive elements of a row shares the power-of-two scale 2^E,
 * E = floor(log2(amax)) - 8 clamped to [-127, 127] (an all-zero block:
 * -127), stored as the E8M0 byte E + 127; codes are the nearest-even E4M3 of
 * x / 2^E, saturating to +-448.
 *   x: bf16 [rows, cols], cols % 32 == 0 (the contraction dimension of a GEMM
 *      operand); q: uint8 [rows, cols], ld_q >= cols, multiple of 16;
 *   scale: uint8 [rows, cols / 32], dense row-major.
 * Errors as for fp8_quantize_blockwise. */
fp8mm_status fp8_quantize_mx(const void* x, int64_t rows, int64_t cols,
                             int64_t ld_x, uint8_t* q, int64_t ld_q,
                             uint8_t* scale, hipStream_t stream);

/* Dual-layout blockwise quantization of a linear layer's grad_output (one
 * read of x, two results).  The backward uses grad_output twice: for
 * grad_input = grad_output @ weight with 1x128 scales, and for grad_weight =
 * grad_output.t() @ input with 128 tokens per scale (ColossalAI PR #6419,
 * "Fix: Handle LowLevelZeroPlugin with use_fp8=True", Backward pass; pytorch/ao
 * PR #2784, "improve fp8 blockwise gemm perf", the 1x128_128x128 and
 * 1x128_128x1 tables).  The results are exactly those of
 *   fp8_quantize_blockwise(x, ..., 1, 128, 0, q_row, ld_q_row, scale_row)
 *   fp8_quantize_blockwise(x, ..., 128, 1, 1, q_col_t, ld_q_col, scale_col)
 *   x:         bf16 [rows, cols], ld_x >= cols; rows and cols multiples of 128.
 *   q_row:     uint8 [rows, cols], ld_q_row >= cols (multiple of 16);
 *              scale_row float32 [cols/128, rows].
 *   q_col_t:   uint8 [cols, rows] (x transposed), ld_q_col >= rows (multiple
 *              of 16); scale_col float32 [rows/128, cols].
 * The two outputs must not overlap each other or x.  Errors as for
 * fp8_quantize_blockwise; shapes not divisible by 128 are FP8MM_EINVAL. */
fp8mm_status fp8_quantize_blockwise_dual(const void* x, int64_t rows,
                                         int64_t cols, int64_t ld_x,
                                         uint8_t* q_row, int64_t ld_q_row,
                                         float* scale_row, uint8_t* q_col_t,
                                         int64_t ld_q_col, float* scale_col,
                                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Scaled GEMM:  out[M, N] = sum_k (A[i,k] s_a(i,k)) (B(j,k) s_b(j,k)) (+bias[j])
 * with float32 accumulation on the matrix cores and one final rounding to
 * out_dtype (bf16 round-to-nearest-even or fp32).  The formulation is the
 * fused scaled-mm call whose dequantize-then-matmul equivalent is spelled out
 * in ColossalAI PR #6419 ("Forward pass", "Backward pass").
 *   A: uint8 [M, K], leading dimension lda (K contiguous).
 *   B: uint8 [N, K] (B_NK, ldb >= K) or [K, N] (B_KN, ldb >= N).
 *   scale_a / scale_b: float32 in the layouts of fp8mm_recipe (MXFP8: the
 *   pointers carry its uint8 E8M0 bytes, passed unchanged).
 *   bias: NULL or bf16 [N], added in fp32 before the rounding.
 *   out: bf16 or fp32 [M, N], leading dimension ldo >= N.
 * Accepted (recipe_a, recipe_b) pairs, anything else -> FP8MM_ENOTIMPL:
 *   (TENSORWISE, TENSORWISE)  (ROWWISE, ROWWISE)
 *   (BLOCK_1x128, BLOCK_128x128)  (BLOCK_1x128, BLOCK_128x1)
 *   (MXFP8, MXFP8) with B_NK (B_KN -> FP8MM_ENOTIMPL)
 * K % 16 == 0; blockwise and MXFP8 recipes need K % 128 == 0 and, for
 * BLOCK_128x128, N % 128 == 0; blockwise scale arrays of 2^30 or more
 * elements ((K/128) M or (K/128) N) are FP8MM_EINVAL.  M, N or K of 0 is
 * allowed. */
fp8mm_status fp8_scaled_mm(const uint8_t* A, int64_t M, int64_t K, int64_t lda,
                           const uint8_t* B, int64_t N, int64_t ldb,
                           fp8mm_b_layout b_layout, const float* scale_a,
                           fp8mm_recipe recipe_a, const float* scale_b,
                           fp8mm_recipe recipe_b, const void* bias,
                           fp8mm_out_dtype out_dtype, void* out, int64_t ldo,
                           hipStream_t stream);

/* Grouped (MoE) scaled GEMM, rowwise x rowwise only, in the canonical form
 * grouped_mm(act, weight.transpose(-2, -1), offs) of pytorch/ao PR #4390
 * ("Add _grouped_mm dispatch handler to Float8Tensor", "Design" and review):
 *   A: uint8 [M_total, K] (lda = K), scale_a float32 [M_total] (per token).
 *   B_EnK: uint8 [E, N, K] expert weights (K contiguous), scale_b [E, N].
 *   offsets: DEVICE int32 [E], cumulative END row offsets: expert e owns rows
 *     [offsets[e-1], offsets[e]) (offsets[-1] = 0); required (NULL -> EINVAL).
 *   bias: NULL or bf16 [N], added to every expert's rows (per-expert bias
 *     rows: fp8_scaled_grouped_mm_v2 with bias_per_expert = 1).
 *   out: [M_total, N], leading dimension ldo >= N.  Rows at or past
 *     offsets[E-1] are not written.
 * Offsets are read on the device only; they are not validated on the host
 * (that would need a synchronization) and must be non-decreasing.  The
 * kernels clamp each to [0, M_total] and treat a decreasing pair as an empty
 * group, so no access leaves the arrays; the next expert then starts at the
 * smaller offset, and rows that two experts cover are written twice (their
 * values are undefined).
 * K % 16 == 0.  E <= 2^16 here and in every other grouped call (each
 * workgroup scans the offsets to find its expert). */
fp8mm_status fp8_scaled_grouped_mm(const uint8_t* A, int64_t M_total,
                                   int64_t K, const uint8_t* B_EnK, int64_t E,
                                   int64_t N, const int32_t* offsets,
                                   const float* scale_a, const float* scale_b,
                                   const void* bias, fp8mm_out_dtype out_dtype,
                                   void* out, int64_t ldo, hipStream_t stream);

/* Grouped (MoE) scaled GEMM with an explicit recipe per operand (the recipe
 * table of pytorch PR #164141, "Add _scaled_mm_v2 API", applied to the
 * grouped form of pytorch/ao PR #4390, "Add _grouped_mm dispatch handler to
 * Float8Tensor").  Expert e multiplies rows [offsets[e-1], offsets[e]) of A
 * by its own B_e:
 *   A: uint8 [M_total, K] (lda = K).
 *   B_E: uint8 [E, N, K] (B_NK: the forward's grouped_mm(act,
 *     weight.transpose(-2, -1)) form) or [E, K, N] (B_KN: e.g. the stored
 *     [E, N_out, K_in] expert weights read by the input gradient, which
 *     contracts over N_out).
 *   (ROWWISE, ROWWISE): scale_a float32 [M_total], scale_b [E, N].
 *   (BLOCK_1x128, BLOCK_128x128): scale_a [K/128, M_total]; scale_b expert
 *     e's 128x128 grid of B_e as stored, [E, N/128, K/128] (B_NK) or
 *     [E, K/128, N/128] (B_KN); K % 128 == 0 and N % 128 == 0.  The pages
 *     give the grouped GEMM only with rowwise scales; this pair is the
 *     blockwise recipe applied per expert.
 *   Any other pair -> FP8MM_ENOTIMPL.
 *   B_KN: N % 16 == 0 and K * N < 2^31.
 *   bias: NULL, or bf16 [N] shared by every expert (bias_per_expert = 0),
 *     or bf16 [E, N], row e for expert e (bias_per_expert = 1); any other
 *     bias_per_expert -> FP8MM_EINVAL.
 *   offsets, out and the treatment of the offsets: as
 *   fp8_scaled_grouped_mm.  K % 16 == 0. */
fp8mm_status fp8_scaled_grouped_mm_v2(const uint8_t* A, int64_t M_total,
                                      int64_t K, const uint8_t* B_E, int64_t E,
                                      int64_t N, fp8mm_b_layout b_layout,
                                      const int32_t* offsets,
                                      const float* scale_a,
                                      fp8mm_recipe recipe_a,
                                      const float* scale_b,
                                      fp8mm_recipe recipe_b, const void* bias,
                                      int bias_per_expert,
                                      fp8mm_out_dtype out_dtype, void* out,
                                      int64_t ldo, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Grouped (MoE) weight gradient: grad_w[e] = grad_output[rows_e].t() @
 * input[rows_e] for every expert e, the weight-gradient call form (ColossalAI
 * PR #6419, "Backward pass"; 1x128 x 128x1 along the tokens, pytorch/ao PR
 * #2784, second table) applied to each expert's own tokens, expert e owning
 * token rows [offsets[e-1], offsets[e]) as in the grouped GEMM.  The pages
 * give 128-token scaling runs only for the dense case; here the runs restart
 * at each expert's first token, so that no scaling group mixes two experts.
 * ------------------------------------------------------------------------- */

/* Run capacity for T tokens and E experts: T/128 + E (each expert adds at
 * most one short run); -1 for negative arguments.  Host only. */
int64_t fp8mm_grouped_runs_capacity(int64_t T, int64_t E);

/* Quantize x bf16 [T, C] (ld_x >= C, C % 16 == 0) in runs of 128 tokens per
 * expert: each expert's rows are cut into runs of 128 from its first row
 * (the last run may be shorter); each run x column is one scaling group,
 * s = fl32(amax / 448) (zero amax -> 1), code = e4m3(x / s) as in
 * fp8_quantize_blockwise.  Runs are numbered over all experts in order; run
 * r is written transposed at columns [128 r, 128 r + 128) of q_t [C, ld_q]
 * (zero codes in the columns past a short run's last token) with its scales
 * at row r of scale [ld_q / 128, C].  ld_q >= 128 x fp8mm_grouped_runs_capacity
 * (T, E) and a multiple of 16.  Columns and scale rows past the last run are
 * not written; rows of x at or past offsets[E-1] are not read.  offsets:
 * DEVICE int32 [E], treated as in the grouped GEMM. */
fp8mm_status fp8_quantize_grouped_128x1(const void* x, int64_t T, int64_t C,
                                        int64_t ld_x, const int32_t* offsets,
                                        int64_t E, uint8_t* q_t, int64_t ld_q,
                                        float* scale, hipStream_t stream);

/* One read of x, both layouts the MoE layer needs of it (the grouped form
 * of fp8_quantize_blockwise_dual): the 1x128 codes q_row [T, ld_q_row] with
 * scales scale_row [C/128, T] (as fp8_quantize_blockwise with block (1, 128))
 * of every row an expert owns, and the per-expert runs q_t / scale_t exactly
 * as fp8_quantize_grouped_128x1 writes them.  C % 128 == 0, ld_q_row >= C
 * and a multiple of 16; rows at or past offsets[E-1] are left unwritten in
 * q_row and scale_row.  Other arguments and errors as
 * fp8_quantize_grouped_128x1. */
fp8mm_status fp8_quantize_grouped_dual(const void* x, int64_t T, int64_t C,
                                       int64_t ld_x, const int32_t* offsets,
                                       int64_t E, uint8_t* q_row,
                                       int64_t ld_q_row, float* scale_row,
                                       uint8_t* q_t, int64_t ld_q,
                                       float* scale_t, hipStream_t stream);

/* grad_w bf16 or fp32 [E, N_out, K_in] (dense) from the two quantizer
 * outputs of the same offsets, T and ld:
 *   gt_q uint8 [N_out, ld], gt_scale float32 [ld/128, N_out]: grad_output
 *     [T, N_out] quantized by fp8_quantize_grouped_128x1;
 *   xt_q uint8 [K_in, ld], xt_scale [ld/128, K_in]: input [T, K_in] likewise.
 * Expert e contracts over its runs only, the zero codes of a short run's
 * missing tokens included (codes there must be zero, as the quantizer writes
 * them); an expert without tokens gets zeros.  Offsets that are not
 * non-decreasing are undefined input; the kernel still reads only the first
 * ld/128 runs. */
fp8mm_status fp8_grouped_linear_grad_weight(const uint8_t* gt_q, int64_t N_out,
                                            const float* gt_scale,
                                            const uint8_t* xt_q, int64_t K_in,
                                            const float* xt_scale, int64_t ld,
                                            int64_t T, const int32_t* offsets,
                                            int64_t E,
                                            fp8mm_out_dtype out_dtype,
                                            void* grad_w, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The three call forms of an FP8 linear layer (ColossalAI PR #6419, "Forward
 * pass" and "Backward pass"; pytorch/ao PR #2784 names the blockwise GEMMs
 * each one uses).  All operands are pre-quantized, dense (leading dimension =
 * row length), and the calls are thin wrappers over fp8_scaled_mm.
 * ------------------------------------------------------------------------- */

/* out[M, N] = input @ weight.t():  input codes [M, K] (recipe x_recipe),
 * weight codes [N, K] (recipe w_recipe, read as B_NK), bias NULL or [N]. */
fp8mm_status fp8_linear_forward(const uint8_t* x_q, int64_t M, int64_t K,
                                const float* x_scale, fp8mm_recipe x_recipe,
                                const uint8_t* w_q, int64_t N,
                                const float* w_scale, fp8mm_recipe w_recipe,
                                const void* bias, fp8mm_out_dtype out_dtype,
                                void* out, hipStream_t stream);

/* grad_input[M, K_in] = grad_output @ weight:  grad_output codes [M, N_out]
 * (recipe g_recipe, contraction over N_out), weight codes as stored
 * [N_out, K_in] (recipe w_recipe, read as B_KN). */
fp8mm_status fp8_linear_grad_input(const uint8_t* g_q, int64_t M,
                                   int64_t N_out, const float* g_scale,
                                   fp8mm_recipe g_recipe, const uint8_t* w_q,
                                   int64_t K_in, const float* w_scale,
                                   fp8mm_recipe w_recipe,
                                   fp8mm_out_dtype out_dtype, void* grad_in,
                                   hipStream_t stream);

/* grad_weight[N_out, K_in] = grad_output.t() @ input, contracting over T
 * tokens.  Both operands come from fp8_quantize_blockwise with block (128, 1)
 * and transpose_out = 1:  gt_q = codes of grad_output^T [N_out, T] with
 * gt_scale [T/128, N_out];  xt_q = codes of input^T [K_in, T] with xt_scale
 * [T/128, K_in].  Recipes: (BLOCK_1x128, BLOCK_128x1), B read as B_NK. */
fp8mm_status fp8_linear_grad_weight(const uint8_t* gt_q, int64_t N_out,
                                    int64_t T, const float* gt_scale,
                                    const uint8_t* xt_q, int64_t K_in,
                                    const float* xt_scale,
                                    fp8mm_out_dtype out_dtype, void* grad_w,
                                    hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Host-only queries (no device access).
 * ------------------------------------------------------------------------- */

/* 1 if fp8_scaled_mm accepts the recipe pair with this B layout, else 0. */
int fp8mm_recipe_pair_supported(fp8mm_recipe recipe_a, fp8mm_recipe recipe_b,
                                fp8mm_b_layout b_layout);

/* Message describing the last non-OK status returned on the calling thread
 * (empty string if none).  Owned by the library; valid until the next call on
 * the same thread. */
const char* fp8mm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8MM_H */
