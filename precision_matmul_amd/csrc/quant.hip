// Dynamic FP8 quantization kernels for gfx950.
//
// Per scaling group: amax -> s = fl32(amax/448) [+eps] -> code = e4m3(x / s).
// (Per-token scaling with an epsilon: DiffSynth-Engine PR #160, "per-token
// scaling for fp8 linear", "Highlights"; the block groupings 1x128, 128x128
// and 128x1: pytorch PR #164141 "Add _scaled_mm_v2 API" and pytorch/ao PR
// #2784 "improve fp8 blockwise gemm perf".)
//
// The pass is HBM-bound (2 bytes read + 1 byte written per element): every
// kernel streams 16-byte loads per lane, keeps a group in registers between
// its amax and its cast, and writes 8 bytes of codes per lane.  amax is taken
// on the bf16 bit patterns (|x| orders like the integer x & 0x7FFF), so the
// reductions are integer max operations and are exact and order-free.
#include "fp8_codec.hpp"
#include "grouped.hpp"
#include "quant_launch.hpp"

namespace fp8mm {
namespace {

struct alignas(16) U16x8 {
  uint32_t w[4];
};

__device__ __forceinline__ U16x8 load16(const uint16_t* p) {
  return *reinterpret_cast<const U16x8*>(p);
}

// max of |x| over the 8 bf16 values, as a bf16 magnitude bit pattern.
__device__ __forceinline__ uint32_t absmax8(const U16x8& v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = v.w[i] & 0x7FFF7FFFu;
    m = max(m, max(a & 0xFFFFu, a >> 16));
  }
  return m;
}

// Elementwise |x| max of two 8-value vectors, kept as packed magnitudes.
__device__ __forceinline__ void absmax_accum(U16x8& acc, const U16x8& v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = v.w[i] & 0x7FFF7FFFu;
    const uint32_t lo = max(acc.w[i] & 0xFFFFu, a & 0xFFFFu);
    const uint32_t hi = max(acc.w[i] >> 16, a >> 16);
    acc.w[i] = lo | (hi << 16);
  }
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Max over aligned groups of 16 lanes.
__device__ __forceinline__ uint32_t group16_max(uint32_t v) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// E4M3 codes of four quotients y = x / s, packed little-endian: round to
// nearest even, saturating to +-448, sign taken from the input x (so that
// -0 and negatives that round to zero give 0x80; the FMA steps of the
// quotient can turn -0 into +0).  The hardware conversion rounds to nearest
// even and agrees with that rule on every float32 of magnitude up to 464;
// clamping larger magnitudes to 448 first (the comparison is false for NaN,
// which stays NaN) extends it to the whole range.
__device__ __forceinline__ float sat448(float y, float x) {
  const float a = __builtin_fabsf(y);
  return __builtin_copysignf(a > 448.0f ? 448.0f : a, x);
}
__device__ __forceinline__ uint32_t pack4(const float* y, const float* x, int stride = 1) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(y[0], x[0]), sat448(y[stride], x[stride]), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(y[2 * stride], x[2 * stride]), sat448(y[3 * stride], x[3 * stride]), w,
                                      true);
  return uint32_t(w);
}

// Quotients fl32(x / s) of 8 values, each with its own cast constants.  The
// exact reciprocal-and-correction path covers every scale >= 2^-90; a wave
// with any smaller scale takes the IEEE division for those values.  The test
// is wave-uniform, so the common case has no per-value branches.
__device__ __forceinline__ void quotients8(const float x[8], const CastScale* const cs[8], float y[8]) {
  bool fast = true;
#pragma unroll
  for (int k = 0; k < 8; ++k) fast = fast && cs[k]->fast;
  if (__all(fast)) {
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = div_by_scale(x[k], cs[k]->s, cs[k]->r);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = cs[k]->fast ? div_by_scale(x[k], cs[k]->s, cs[k]->r) : x[k] / cs[k]->s;
  }
}

__device__ __forceinline__ void unpack8(const U16x8& v, float x[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bits_f32(v.w[i] << 16);
    x[2 * i + 1] = bits_f32(v.w[i] & 0xFFFF0000u);
  }
}

// Encode 8 bf16 values with one scale into 8 codes (little-endian bytes).
__device__ __forceinline__ uint2 cast8(const U16x8& v, const CastScale& cs) {
  float x[8], y[8];
  unpack8(v, x);
  const CastScale* c[8] = {&cs, &cs, &cs, &cs, &cs, &cs, &cs, &cs};
  quotients8(x, c, y);
  return make_uint2(pack4(y, x), pack4(y + 4, x + 4));
}

// ---------------------------------------------------------------------------
// Rowwise: one wave per row, the row held in registers (NIT x 512 columns).
// ---------------------------------------------------------------------------
template <int NIT>
__global__ __launch_bounds__(256) void quant_rowwise_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    float eps, uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + row * ld_x;
  U16x8 v[NIT];
  uint32_t m = 0;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int64_t col = (int64_t(it) * 64 + lane) * 8;
    if (col < cols) {
      v[it] = load16(xr + col);
      m = max(m, absmax8(v[it]));
    }
  }
  m = wave_max(m);
  const float s = scale_from_amax(bf16_to_f32(uint16_t(m)), eps, true);
  const CastScale cs = make_cast_scale(s);
  if (lane == 0) scale[row] = s;
  uint8_t* qr = q + row * ld_q;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int64_t col = (int64_t(it) * 64 + lane) * 8;
    if (col < cols) *reinterpret_cast<uint2*>(qr + col) = cast8(v[it], cs);
  }
}

// Rows too long for registers: amax pass, then a second (L2-resident) pass.
__global__ __launch_bounds__(256) void quant_rowwise_long_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    float eps, uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + row * ld_x;
  uint32_t m = 0;
  for (int64_t col = int64_t(lane) * 8; col < cols; col += 512) m = max(m, absmax8(load16(xr + col)));
  m = wave_max(m);
  const float s = scale_from_amax(bf16_to_f32(uint16_t(m)), eps, true);
  const CastScale cs = make_cast_scale(s);
  if (lane == 0) scale[row] = s;
  uint8_t* qr = q + row * ld_q;
  for (int64_t col = int64_t(lane) * 8; col < cols; col += 512)
    *reinterpret_cast<uint2*>(qr + col) = cast8(load16(xr + col), cs);
}

// ---------------------------------------------------------------------------
// Blockwise (1, 128): one wave per row, 16 lanes per 128-column group, so a
// wave's load covers 512 contiguous columns (4 groups).  Workgroups of 4
// rows keep the grid fine-grained (every CU gets nearly the same number of
// rows).  Groups of U such 512-column strips are cast from one buffer while
// the next buffer's loads are in flight.  Scales go to scale[kb * rows + row].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_1x128_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;   // whole waves leave together
  const int sub = lane & 15;
  const int grp = lane >> 4;                     // which of the 4 groups of a strip
  const int64_t nkb = cols / 128;
  uint8_t* qr = q + row * ld_q + lane * 8;
  auto cast_group = [&](const U16x8& v, int64_t strip) {
    const int64_t kb = strip * 4 + grp;
    const uint32_t m = group16_max(absmax8(v));
    const float s = scale_from_amax(bf16_to_f32(uint16_t(m)), 0.0f, false);
    const CastScale cs = make_cast_scale(s);
    if (kb < nkb) {
      if (sub == 0) scale[kb * rows + row] = s;
      *reinterpret_cast<uint2*>(qr + strip * 512) = cast8(v, cs);
    }
  };
  const int64_t nstrip = (nkb + 3) / 4;           // the last strip may hold 1..4 groups
  constexpr int U = 4;
  const int64_t nfull = nstrip / U * U;
  // Loads past the end of a row (the last strip's missing groups, or the
  // re-read of strip nstrip - 1 that keeps loads out of branches) are clamped
  // into the row: they read valid columns whose results are unused.
  auto load_strip = [&](int64_t strip) {
    const int64_t st = min(strip, nstrip - 1);
    const int64_t col = min(st * 512 + lane * 8, (nkb - 1) * 128 + sub * 8);
    return load16(x + row * ld_x + col);
  };
  U16x8 va[U], vb[U];
  if (nfull > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) va[u] = load_strip(u);
  }
  for (int64_t st = 0; st < nfull; st += 2 * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) vb[u] = load_strip(st + U + u);
#pragma unroll
    for (int u = 0; u < U; ++u) cast_group(va[u], st + u);
#pragma unroll
    for (int u = 0; u < U; ++u) va[u] = load_strip(st + 2 * U + u);
    if (st + U < nfull) {
#pragma unroll
      for (int u = 0; u < U; ++u) cast_group(vb[u], st + U + u);
    }
  }
  for (int64_t st = nfull; st < nstrip; ++st) cast_group(load_strip(st), st);
}

// ---------------------------------------------------------------------------
// Blockwise (128, 128): one workgroup per block.  Thread t covers columns
// (t % 16) * 8 .. +8 of rows t/16 + 16 i, i < 8.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_128x128_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale) {
  __shared__ uint32_t wmax[4];
  const int t = threadIdx.x;
  const int64_t r0 = int64_t(blockIdx.y) * 128 + (t >> 4);
  const int64_t c0 = int64_t(blockIdx.x) * 128 + (t & 15) * 8;
  U16x8 v[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = load16(x + (r0 + 16 * i) * ld_x + c0);
    m = max(m, absmax8(v[i]));
  }
  m = wave_max(m);
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float s = scale_from_amax(bf16_to_f32(uint16_t(m)), 0.0f, false);
  const CastScale cs = make_cast_scale(s);
  if (t == 0) scale[int64_t(blockIdx.y) * (cols / 128) + blockIdx.x] = s;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint2*>(q + (r0 + 16 * i) * ld_q + c0) = cast8(v[i], cs);
}

// ---------------------------------------------------------------------------
// Blockwise (128, 1): a workgroup owns 128 rows x 128 columns; thread t holds
// columns (t % 16) * 8 .. +8 of the 8 consecutive rows (t / 16) * 8 .. +8.
// Column maxima: packed u16 max over the thread's rows, then across the 4
// row groups of a wave (lane xor 16, 32), then across the 4 waves in LDS.
// TRANSPOSE writes the codes as q[col, row]: each thread owns an 8x8 byte
// block and stores, per column, its 8 consecutive row codes as one 8-byte
// word.
// ---------------------------------------------------------------------------
//
// DUAL (with TRANSPOSE) also emits the 1x128 quantization of the same tile
// from the same registers: row maxima over the 16 lanes that hold a row's
// 128 columns, row scales scale_row[kb * rows + row] (kb = the tile's column
// block), row codes q_row[row, col].  One read of x gives both operands of a
// linear layer's backward that come from grad_output.
//
// GROUPED (with TRANSPOSE): the grouped weight gradient's runs.  Workgroup x
// takes run blockIdx.x counted over all experts (expert e owns rows
// [offs[e-1], offs[e])): the run's rows (fewer than 128 at an expert's end,
// the missing rows read as zeros, i.e. zero codes), its codes at columns
// [128 run, 128 run + 128) of q and its scales at row `run`.  It walks CT
// column tiles (from blockIdx.y CT), loading tile j + 1 while it reduces and
// writes tile j, so that the run lookup is paid once per CT tiles.
// Workgroups past the last run exit.
// Column tiles per workgroup of the grouped runs.  One: walking several
// tiles per workgroup (the next tile loaded during this one's work) paid for
// the run lookup once, but cut the workgroups fourfold and doubled the
// registers; measured slower (0.087 against 0.053 ms for the E = 64, 16384
// token pair of grad_output [.., 1408] and input [.., 2048]).
constexpr int kGroupedColTiles = 1;

template <bool TRANSPOSE, bool DUAL, bool GROUPED>
__global__ __launch_bounds__(256) void quant_128x1_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale,
    uint8_t* __restrict__ q_row, int64_t ld_q_row, float* __restrict__ scale_row,
    const int32_t* __restrict__ offsets, int64_t E) {
  static_assert(!GROUPED || TRANSPOSE, "grouped runs: transposed codes only");
  constexpr int CT = GROUPED ? kGroupedColTiles : 1;
  __shared__ U16x8 colmax[4][16];
  __shared__ float col_s[128];
  __shared__ float col_r[128];
  const int t = threadIdx.x;
  const int cc = t & 15;
  const int rg = t >> 4;
  const int wave = t >> 6;
  int64_t rb = blockIdx.y;                 // scale row and output block
  int64_t tile0 = blockIdx.x;              // first column tile
  int64_t row_first = rb * 128;            // first row of x in the group
  int rows_here = 128;                     // rows of x in the group
  if constexpr (GROUPED) {
    rb = blockIdx.x;
    tile0 = int64_t(blockIdx.y) * CT;
    int e = 0;
    int64_t row_end = 0;
    if (!grp::find_run(offsets, E, rows, 128, int(blockIdx.x), e, row_first, row_end)) return;
    rows_here = int(min<int64_t>(128, row_end - row_first));
  }
  const int64_t ntiles = (cols + 127) / 128;
  const int64_t r0 = rb * 128 + rg * 8;   // output row (TRANSPOSE: output column) of the thread's first row
  const int64_t xr0 = row_first + rg * 8; // its row of x
  // 8 rows x 8 columns of column tile `tile` (zeros past the run or the
  // columns; cols % 8 == 0, so a thread's 8 columns are all in or all out)
  auto load_tile = [&](int64_t tile, U16x8 (&dst)[8]) {
    const int64_t c0 = tile * 128 + cc * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (c0 < cols && rg * 8 + i < rows_here) {
        dst[i] = load16(x + (xr0 + i) * ld_x + c0);
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) dst[i].w[w] = 0u;
      }
    }
  };
  U16x8 v[8], vn[8];
  load_tile(tile0, v);
  for (int jt = 0; jt < CT; ++jt) {
    const int64_t tile = tile0 + jt;
    if (tile >= ntiles) break;                 // uniform over the workgroup
    if (jt + 1 < CT && tile + 1 < ntiles) load_tile(tile + 1, vn);
    const int64_t cbase = tile * 128;
    const int64_t c0 = cbase + cc * 8;
    const bool active = c0 < cols;
    U16x8 m;
#pragma unroll
    for (int i = 0; i < 4; ++i) m.w[i] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) absmax_accum(m, v[i]);
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      U16x8 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o.w[i] = (uint32_t)__shfl_xor((int)m.w[i], off, 64);
      absmax_accum(m, o);   // values are already magnitudes
    }
    // colmax of the previous tile was last read before that tile's second
    // barrier, col_s / col_r after it but before this tile's first barrier
    if ((t & 63) < 16) colmax[wave][cc] = m;
    __syncthreads();
    if (t < 128) {
      const int c = t;                       // column within the tile
      const int chunk = c >> 3, e = c & 7;
      uint32_t mm = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t word = colmax[w][chunk].w[e >> 1];
        mm = max(mm, (e & 1) ? (word >> 16) : (word & 0xFFFFu));
      }
      const float s = scale_from_amax(bf16_to_f32(uint16_t(mm)), 0.0f, false);
      col_s[c] = s;
      col_r[c] = 1.0f / s;
      if (cbase + c < cols) scale[rb * cols + cbase + c] = s;
    }
    __syncthreads();
    if (active) {
      if constexpr (DUAL) {
        // 1x128 of the tile's rows: each row's 128 columns are held by the 16
        // consecutive lanes of one row group (cols % 128 == 0: every tile
        // full); grouped, only the run's rows of x (a row group is all in or
        // all out, so the 16-lane reduction stays whole)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (GROUPED && rg * 8 + i >= rows_here) continue;
          const uint32_t mr = group16_max(absmax8(v[i]));
          const float sr = scale_from_amax(bf16_to_f32(uint16_t(mr)), 0.0f, false);
          if (cc == 0) scale_row[tile * rows + xr0 + i] = sr;
          *reinterpret_cast<uint2*>(q_row + (xr0 + i) * ld_q_row + c0) = cast8(v[i], make_cast_scale(sr));
        }
      }
      CastScale cs[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        cs[j].s = col_s[cc * 8 + j];
        cs[j].r = col_r[cc * 8 + j];
        cs[j].fast = cs[j].s >= kFastDivMinScale;
      }
      if (!TRANSPOSE) {
        // row by row: the 8 values of row r0 + i, one column scale each
        const CastScale* c[8] = {&cs[0], &cs[1], &cs[2], &cs[3], &cs[4], &cs[5], &cs[6], &cs[7]};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float xs[8], y[8];
          unpack8(v[i], xs);
          quotients8(xs, c, y);
          *reinterpret_cast<uint2*>(q + (r0 + i) * ld_q + c0) = make_uint2(pack4(y, xs), pack4(y + 4, xs + 4));
        }
      } else {
        // column by column: the 8 row values of column c0 + j, its scale,
        // stored as 8 consecutive bytes of q[c0 + j, ..] (only one column's
        // values and quotients are live at a time)
        bool fast = true;
#pragma unroll
        for (int j = 0; j < 8; ++j) fast = fast && cs[j].fast;
        const bool all_fast = __all(fast);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float xc[8], yc[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t w = v[i].w[j >> 1];
            xc[i] = bits_f32((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
          }
          if (all_fast) {
#pragma unroll
            for (int i = 0; i < 8; ++i) yc[i] = div_by_scale(xc[i], cs[j].s, cs[j].r);
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
              yc[i] = cs[j].fast ? div_by_scale(xc[i], cs[j].s, cs[j].r) : xc[i] / cs[j].s;
          }
          *reinterpret_cast<uint2*>(q + (c0 + j) * ld_q + r0) = make_uint2(pack4(yc, xc), pack4(yc + 4, xc + 4));
        }
      }
    }
    if (jt + 1 < CT) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = vn[i];
    }
  }
}

// ---------------------------------------------------------------------------
// Tensorwise (beyond the single-workgroup size below): clear -> amax (atomic
// max of the float bit pattern, valid because amax >= 0) -> cast -> finalize.  The scale slot holds amax until
// the finalize kernel replaces it with the scale.
// ---------------------------------------------------------------------------
__global__ void tensor_clear_kernel(float* slot) { *reinterpret_cast<uint32_t*>(slot) = 0u; }

__global__ __launch_bounds__(256) void tensor_amax_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x, float* slot) {
  const int64_t chunks_per_row = cols / 8;
  const int64_t total = rows * chunks_per_row;
  uint32_t m = 0;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = i / chunks_per_row;
    const int64_t c = (i - r * chunks_per_row) * 8;
    m = max(m, absmax8(load16(x + r * ld_x + c)));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0 && m != 0)
    atomicMax(reinterpret_cast<unsigned int*>(slot), f32_bits(bf16_to_f32(uint16_t(m))));
}

__global__ __launch_bounds__(256) void tensor_cast_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, const float* slot) {
  const float s = scale_from_amax(*slot, 0.0f, false);
  const CastScale cs = make_cast_scale(s);
  const int64_t chunks_per_row = cols / 8;
  const int64_t total = rows * chunks_per_row;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = i / chunks_per_row;
    const int64_t c = (i - r * chunks_per_row) * 8;
    *reinterpret_cast<uint2*>(q + r * ld_q + c) = cast8(load16(x + r * ld_x + c), cs);
  }
}

__global__ void tensor_finalize_kernel(float* slot) { *slot = scale_from_amax(*slot, 0.0f, false); }

// Small tensors (up to 1024 x 8 chunks of 8 elements): one workgroup of 1024
// threads holds the whole tensor in registers and does amax, scale and cast
// in a single launch.
constexpr int kTensorSmallIt = 8;
__global__ __launch_bounds__(1024) void tensor_small_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale) {
  __shared__ uint32_t wmax[16];
  const int t = threadIdx.x;
  const int64_t chunks_per_row = cols / 8;
  const int64_t total = rows * chunks_per_row;
  U16x8 v[kTensorSmallIt];
  uint32_t m = 0;
#pragma unroll
  for (int it = 0; it < kTensorSmallIt; ++it) {
    const int64_t i = t + int64_t(it) * 1024;
    if (i < total) {
      const int64_t r = i / chunks_per_row;
      v[it] = load16(x + r * ld_x + (i - r * chunks_per_row) * 8);
      m = max(m, absmax8(v[it]));
    }
  }
  m = wave_max(m);
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  m = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) m = max(m, wmax[w]);
  const float s = scale_from_amax(bf16_to_f32(uint16_t(m)), 0.0f, false);
  const CastScale cs = make_cast_scale(s);
  if (t == 0) *scale = s;
#pragma unroll
  for (int it = 0; it < kTensorSmallIt; ++it) {
    const int64_t i = t + int64_t(it) * 1024;
    if (i < total) {
      const int64_t r = i / chunks_per_row;
      *reinterpret_cast<uint2*>(q + r * ld_q + (i - r * chunks_per_row) * 8) = cast8(v[it], cs);
    }
  }
}

int grid_for(int64_t work_items, int per_block, int cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return int(g > cap ? cap : g);
}

}  // namespace

hipError_t launch_quant_tensorwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   uint8_t* q, int64_t ld_q, float* scale, hipStream_t st) {
  const int64_t chunks = rows * (cols / 8);
  if (chunks > 0 && chunks <= 1024 * kTensorSmallIt) {
    hipLaunchKernelGGL(tensor_small_kernel, dim3(1), dim3(1024), 0, st, x, rows, cols, ld_x, q, ld_q, scale);
    return hipGetLastError();
  }
  const int g = grid_for(chunks, 256 * 8, 2048);
  hipLaunchKernelGGL(tensor_clear_kernel, dim3(1), dim3(1), 0, st, scale);
  if (chunks > 0) {
    hipLaunchKernelGGL(tensor_amax_kernel, dim3(g), dim3(256), 0, st, x, rows, cols, ld_x, scale);
    hipLaunchKernelGGL(tensor_cast_kernel, dim3(g), dim3(256), 0, st, x, rows, cols, ld_x, q, ld_q,
                       (const float*)scale);
  }
  hipLaunchKernelGGL(tensor_finalize_kernel, dim3(1), dim3(1), 0, st, scale);
  return hipGetLastError();
}

hipError_t launch_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, float eps,
                                uint8_t* q, int64_t ld_q, float* scale, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const dim3 grid(unsigned((rows + 3) / 4)), block(256);
  const int64_t nit = (cols + 511) / 512;
  if (nit <= 1)
    hipLaunchKernelGGL(quant_rowwise_kernel<1>, grid, block, 0, st, x, rows, cols, ld_x, eps, q, ld_q, scale);
  else if (nit <= 2)
    hipLaunchKernelGGL(quant_rowwise_kernel<2>, grid, block, 0, st, x, rows, cols, ld_x, eps, q, ld_q, scale);
  else if (nit <= 4)
    hipLaunchKernelGGL(quant_rowwise_kernel<4>, grid, block, 0, st, x, rows, cols, ld_x, eps, q, ld_q, scale);
  else if (nit <= 8)
    hipLaunchKernelGGL(quant_rowwise_kernel<8>, grid, block, 0, st, x, rows, cols, ld_x, eps, q, ld_q, scale);
  else if (nit <= 16)
    hipLaunchKernelGGL(quant_rowwise_kernel<16>, grid, block, 0, st, x, rows, cols, ld_x, eps, q, ld_q, scale);
  else
    hipLaunchKernelGGL(quant_rowwise_long_kernel, grid, block, 0, st, x, rows, cols, ld_x, eps, q, ld_q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_blockwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                  int block_rows, int block_cols, int transpose_out, uint8_t* q,
                                  int64_t ld_q, float* scale, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (block_rows == 1 && block_cols == 128) {
    hipLaunchKernelGGL(quant_1x128_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, st, x, rows,
                       cols, ld_x, q, ld_q, scale);
  } else if (block_rows == 128 && block_cols == 128) {
    hipLaunchKernelGGL(quant_128x128_kernel, dim3(unsigned(cols / 128), unsigned(rows / 128)), dim3(256), 0,
                       st, x, rows, cols, ld_x, q, ld_q, scale);
  } else {
    const dim3 grid(unsigned((cols + 127) / 128), unsigned(rows / 128));
    if (transpose_out)
      hipLaunchKernelGGL((quant_128x1_kernel<true, false, false>), grid, dim3(256), 0, st, x, rows, cols, ld_x, q,
                         ld_q, scale, nullptr, int64_t(0), nullptr, nullptr, int64_t(0));
    else
      hipLaunchKernelGGL((quant_128x1_kernel<false, false, false>), grid, dim3(256), 0, st, x, rows, cols, ld_x, q,
                         ld_q, scale, nullptr, int64_t(0), nullptr, nullptr, int64_t(0));
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MXFP8 (OCP Microscaling with E4M3 elements): blocks of 32 consecutive
// elements along a row share the E8M0 byte max(exponent field of the bf16
// amax - 8, 0), i.e. the exponent E = floor(log2 amax) - 8 clamped at -127
// (an amax below 2^-119, a subnormal or zero block all clamp there); codes
// are the nearest-even saturating E4M3 of x * 2^-E, an exact power-of-two
// multiply.  Thread t handles 8 elements; four consecutive lanes are a block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_mx_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, uint8_t* __restrict__ scale) {
  const int64_t chunks_per_row = cols / 8;      // a multiple of 4 (cols % 32 == 0)
  const int64_t total = rows * chunks_per_row;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;   // a multiple of 4
  // the 4 lanes of a block enter and leave the loop together: total, stride
  // and the start of every 4-lane group are multiples of 4
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t r = i / chunks_per_row;
    const int64_t c = (i - r * chunks_per_row) * 8;
    const U16x8 v = load16(x + r * ld_x + c);
    uint32_t m = absmax8(v);
    m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
    const int eb = int(m >> 7);                            // bf16 exponent field of amax
    const int byte = eb > 8 ? eb - 8 : 0;                  // E + 127
    const float mult = bits_f32(uint32_t(254 - byte) << 23);   // 2^-E
    float xs[8], y[8];
    unpack8(v, xs);
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = xs[k] * mult;
    *reinterpret_cast<uint2*>(q + r * ld_q + c) = make_uint2(pack4(y, xs), pack4(y + 4, xs + 4));
    if ((threadIdx.x & 3) == 0) scale[r * (cols / 32) + c / 32] = uint8_t(byte);
  }
}

hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                           uint8_t* scale, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int g = grid_for(rows * (cols / 8), 256 * 8, 4096);
  hipLaunchKernelGGL(quant_mx_kernel, dim3(g), dim3(256), 0, st, x, rows, cols, ld_x, q, ld_q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_blockwise_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                       uint8_t* q_row, int64_t ld_q_row, float* scale_row, uint8_t* q_col_t,
                                       int64_t ld_q_col, float* scale_col, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid(unsigned(cols / 128), unsigned(rows / 128));
  hipLaunchKernelGGL((quant_128x1_kernel<true, true, false>), grid, dim3(256), 0, st, x, rows, cols, ld_x, q_col_t,
                     ld_q_col, scale_col, q_row, ld_q_row, scale_row, nullptr, int64_t(0));
  return hipGetLastError();
}

hipError_t launch_quant_grouped_128x1(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                      const int32_t* offsets, int64_t E, uint8_t* q_t, int64_t ld_q, float* scale,
                                      uint8_t* q_row, int64_t ld_q_row, float* scale_row, hipStream_t st) {
  if (rows == 0 || cols == 0 || E == 0) return hipSuccess;
  // an upper bound on the run count: each expert adds at most one short run
  const int64_t runs_max = rows / 128 + E;
  const int64_t tiles = (cols + 127) / 128;
  const dim3 grid(unsigned(runs_max), unsigned((tiles + kGroupedColTiles - 1) / kGroupedColTiles));
  if (q_row)
    hipLaunchKernelGGL((quant_128x1_kernel<true, true, true>), grid, dim3(256), 0, st, x, rows, cols, ld_x, q_t, ld_q,
                       scale, q_row, ld_q_row, scale_row, offsets, E);
  else
    hipLaunchKernelGGL((quant_128x1_kernel<true, false, true>), grid, dim3(256), 0, st, x, rows, cols, ld_x, q_t,
                       ld_q, scale, nullptr, int64_t(0), nullptr, offsets, E);
  return hipGetLastError();
}

}  // namespace fp8mm
