// Helpers shared by the FP8 GEMM kernels (gfx950): MFMA wrapper, swizzled
// LDS tile addressing, buffer descriptors, direct-to-LDS loads, tile order.
#pragma once

#include <stdint.h>

#include "grouped.hpp"
#include "launch.hpp"

namespace fp8mm {
namespace gk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BK = 128;

__device__ __forceinline__ v4f mfma_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
  // Zero scale operands select the unscaled FP8 x FP8 instruction
  // (cbsz = blgp = 0: both operands E4M3).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The block-scaled form.  The instruction's K order: lane group q (lanes
// 16q .. 16q + 15) holds K [16q, 16q + 16) in bytes 0-15 and K [64 + 16q,
// 64 + 16q + 16) in bytes 16-31 of its 32 (the fragment order of these
// kernels, chunks q and q + 4 of a 128-byte row).  The E8M0 byte (bits 0-7)
// that lane group g passes for its row (A) or column (B) scales K [32g,
// 32g + 32), i.e. chunks 2g and 2g + 1.  (Probed on the device byte by byte.)
__device__ __forceinline__ v4f mfma_16x16x128_mx(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// LDS tile rows are 128 bytes; 16-byte chunk c of row r is stored at slot
// c ^ ((r >> 1) & 7).  A 16x16 fragment read has 16 lanes of 16 bytes in
// flight per LDS cycle, one per row of a 16-row group: the swizzle gives the
// 16 rows distinct (row parity, slot) pairs, i.e. distinct bank groups of the
// 64-bank LDS.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer descriptor as four wave-uniform dwords (base, stride 0, size in
// bytes, gfx9 raw-buffer flags); loads at offsets >= size return zeros.
typedef int Rsrc __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Rsrc make_rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return Rsrc{__builtin_amdgcn_readfirstlane(int(uint32_t(a))), __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32))),
              __builtin_amdgcn_readfirstlane(int(bytes)), 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(__builtin_amdgcn_readfirstlane(
      int(uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p)))));
}

// Global -> LDS DMA of 16 (or 4) bytes per lane: lane l writes LDS bytes
// [lds + 16 l, +16) (or [lds + 4 l, +4)).  Written as inline asm so that the
// compiler does not attach its own conservative LDS-DMA waits to every LDS
// read; the kernel tracks these loads itself with s_waitcnt vmcnt.  The
// instructions have no register results: their operands are consumed at
// issue.
__device__ __forceinline__ void dma_b128(Rsrc r, uint32_t lds, uint32_t voff, uint32_t soff) {
  soff = uint32_t(__builtin_amdgcn_readfirstlane(int(soff)));
  lds = uint32_t(__builtin_amdgcn_readfirstlane(int(lds)));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(r),
               "s"(soff)
               : "memory", "m0");
}

// Four 16-byte-per-lane loads with one M0 write: load q (0..3) reads byte
// offset voff_q + soff + 1024 q and writes LDS bytes [lds + 1024 q + 16 l,
// +16) (the instruction offset moves both addresses).
__device__ __forceinline__ void dma_b128x4(Rsrc r, uint32_t lds, uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                           uint32_t soff) {
  soff = uint32_t(__builtin_amdgcn_readfirstlane(int(soff)));
  lds = uint32_t(__builtin_amdgcn_readfirstlane(int(lds)));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
      "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds" ::"s"(lds),
      "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(r), "s"(soff)
      : "memory", "m0");
}

__device__ __forceinline__ void dma_b32(Rsrc r, uint32_t lds, uint32_t voff) {
  lds = uint32_t(__builtin_amdgcn_readfirstlane(int(lds)));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}

// The same descriptor with no valid bytes: every lane's load returns zero.
__device__ __forceinline__ Rsrc dead(Rsrc r) { return Rsrc{r.x, r.y, 0, r.w}; }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

struct TileInfo {
  int64_t row0;       // first output / A row of the tile
  int rows_valid;     // rows of the tile inside the problem (<= BM)
  int64_t n0;
  int cols_valid;
  const uint8_t* A;   // A + row0 * lda
  const uint8_t* B;   // tile origin of B (n0 applied)
  const float* sb;    // scale_b of this problem (expert applied)
  const uint16_t* bias;
  const float* sa;    // scale_a of this problem (grouped weight gradient: expert applied)
  int K;              // contraction length of the tile
  int64_t out_off;    // element offset of the tile's problem in the output
};

constexpr int epi_passes(int nw, int tm, int tn, int outb, int stage) {
  // smallest number of column passes whose staging (nw/2 waves per stage
  // array, TM rows each, padded pitch) fits in one stage array
  for (int pz = 1; pz <= 4; pz *= 2)
    if ((nw / 2) * tm * ((tn / pz) * outb + 16) <= stage) return pz;
  return 8;
}

// Non-grouped tile order: the launcher pads the grid to a multiple of 8 and
// workgroup ids are remapped so that each of the 8 XCDs (one L2 each) owns a
// contiguous range of tiles; within it tiles are walked in groups of GROUP_M
// tile rows, so that the workgroups running together share A and B strips.
// Returns false for padding workgroups.
__device__ __forceinline__ bool tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_xcd = gridDim.x / 8;
  const int lin = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (lin >= tiles_m * tiles_n) return false;
  constexpr int GROUP_M = 8;
  const int span = GROUP_M * tiles_n;
  const int first_m = (lin / span) * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  tm = first_m + (lin % span) % gsize;
  tn = (lin % span) / gsize;
  return true;
}

// Grouped problems: m-tile g, counted over all experts in expert order
// (expert e has ceil(rows_e / bm) of them), -> expert, first row, end row.
// Returns false when g is past the last m-tile.
__device__ inline bool grouped_mtile(const GemmProblem& p, int bm, int g, int& e_out, int64_t& row0,
                                     int64_t& row_end) {
  return grp::find_run(p.offsets, p.E, p.M, bm, g, e_out, row0, row_end);
}

}  // namespace gk
}  // namespace fp8mm
