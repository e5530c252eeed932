// GEMM launchers shared between the C ABI layer and the GEMM kernel sources
// (the quantizer launchers are in quant_launch.hpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mm {

// Scale application of a GEMM.
enum class Epi : int {
  Tensor = 0,       // out = acc * sa[0] * sb[0]
  Row = 1,          // out = acc * sa[i] * sb[j]
  Block128x128 = 2, // acc += P_kb * sa[kb, i] * sb[j/128, kb]   (per 128-K block)
  Block128x1 = 3,   // acc += P_kb * sa[kb, i] * sb[kb, j]
  MX = 4            // MXFP8: E8M0 bytes per 32 K applied by the MFMA; out = acc
};

struct GemmProblem {
  const uint8_t* A;
  const uint8_t* B;
  const float* sa;
  const float* sb;
  const uint16_t* bias;   // bf16 [N] or null; grouped: expert e reads bias + e * bias_stride_e
  int64_t bias_stride_e;  // grouped: 0 (one [N] row for every expert) or N ([E, N])
  void* out;
  int64_t M, N, K;
  int64_t lda, ldb, ldo;
  Epi epi;
  bool b_kn;
  bool out_bf16;
  // grouped (MoE) problems
  const int32_t* offsets; // device [E] end offsets, or null for a plain GEMM
  int64_t E;
  // plain problems: the launch covers output rows [row_begin, row_end)
  int64_t row_begin;
  int64_t row_end;
  // Output addressing: row r of the result goes to out row r - out_row0.
  // With splits > 1 (generic kernel only) the launch runs splits K ranges,
  // range y writing its fp32 partial at out + y * split_stride elements.
  int64_t out_row0;
  int64_t split_stride;
  int splits;
  // Grouped weight gradient (group_k): E problems of M x N, problem e
  // contracting over expert e's runs of 128 tokens on a token axis padded
  // per expert to whole runs (lda = ldb = its length); offsets give the
  // experts' token ranges, clamped to [0, tokens]; A scales [runs, M], B
  // scales [runs, N] (1x128 x 128x1 along the tokens); problem e written at
  // out + e M ldo.
  bool group_k;
  int64_t tokens;
};

hipError_t launch_gemm(const GemmProblem& p, hipStream_t st);
// Streaming schedule, 256 x 256 tiles: plain GEMMs and grouped rowwise GEMMs.
hipError_t launch_gemm_streaming(const GemmProblem& p, hipStream_t st);
// The grouped weight gradient (group_k) on the streaming kernel's 256 x 256 tiles.
hipError_t launch_gemm_group_k_streaming(const GemmProblem& p, hipStream_t st);
// Grouped GEMMs in the weight-streaming regime (experts of a few hundred
// rows, weights stored [N, K]): 320-row m-blocks, one per expert up to 320
// rows, so each weight slice is read about once.
bool grouped_wide_applies(const GemmProblem& p);
hipError_t launch_gemm_grouped_wide(const GemmProblem& p, hipStream_t st);

}  // namespace fp8mm
