// Quantizer launchers shared between the C ABI layer and csrc/quant.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mm {

hipError_t launch_quant_tensorwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   uint8_t* q, int64_t ld_q, float* scale, hipStream_t st);
hipError_t launch_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, float eps,
                                uint8_t* q, int64_t ld_q, float* scale, hipStream_t st);
hipError_t launch_quant_blockwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                  int block_rows, int block_cols, int transpose_out, uint8_t* q,
                                  int64_t ld_q, float* scale, hipStream_t st);
// One read of x, two outputs: 1x128 (row-major codes) and 128x1 written
// transposed.  rows and cols multiples of 128.
hipError_t launch_quant_blockwise_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                       uint8_t* q_row, int64_t ld_q_row, float* scale_row, uint8_t* q_col_t,
                                       int64_t ld_q_col, float* scale_col, hipStream_t st);

// MXFP8: 32-element blocks along rows, E8M0 scale bytes [rows, cols / 32].
hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                           uint8_t* scale, hipStream_t st);

// Grouped 128x1 quantization for the grouped weight gradient: runs of 128
// rows restarted at each expert's first row (expert e owns rows
// [offs[e-1], offs[e])), codes written transposed into q_t [cols, ld_q] with
// run r at columns [128 r, 128 r + 128) (zero codes past a short run's last
// row), scales [runs, cols].  ld_q >= 128 x the run count.  With q_row (cols
// % 128 == 0) the same read also gives the 1x128 codes q_row [rows, ld_q_row]
// and scales scale_row [cols / 128, rows] of every row an expert owns.
hipError_t launch_quant_grouped_128x1(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                      const int32_t* offsets, int64_t E, uint8_t* q_t, int64_t ld_q, float* scale,
                                      uint8_t* q_row, int64_t ld_q_row, float* scale_row, hipStream_t st);

}  // namespace fp8mm
