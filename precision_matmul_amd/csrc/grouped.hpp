// Expert ranges of grouped (MoE) problems, read from device offsets by the
// grouped GEMMs and the grouped quantizer.
//
// Expert e owns rows [offs[e-1], offs[e]) (offs[-1] = 0) of the token axis
// (the grouped form of pytorch/ao PR #4390, "Add _grouped_mm dispatch handler
// to Float8Tensor", "Design"); each offset is clamped to [0, rows] and a
// decreasing pair is an empty group.  Counts of runs of bm rows per expert
// (ceil(rows_e / bm)) place the experts' runs one after another: the m-tiles
// of the grouped GEMM, and the 128-token runs of the padded token axis of the
// grouped weight gradient.  Every function is called by a whole wave, which
// scans 64 experts at a time; all lanes get the same answer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mm {
namespace grp {

__device__ __forceinline__ int64_t clamp_offset(int32_t v, int64_t rows) {
  const int64_t x = v < 0 ? 0 : int64_t(v);
  return x > rows ? rows : x;
}

// Both offsets are loaded before either is used, so their latencies overlap.
__device__ __forceinline__ void expert_range(const int32_t* offs, int64_t rows, int64_t e, int64_t& start,
                                             int64_t& end) {
  const int32_t hi = offs[e];
  const int32_t lo = offs[e > 0 ? e - 1 : 0];
  end = clamp_offset(hi, rows);
  start = e == 0 ? 0 : clamp_offset(lo, rows);
}

// A value every lane holds, in scalar registers (so that the code that
// depends on it branches and addresses with scalar instructions).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  return int64_t((uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(v >> 32)))) << 32) |
                 uint32_t(__builtin_amdgcn_readfirstlane(int(v))));
}

__device__ __forceinline__ int runs_of(int64_t start, int64_t end, int bm) {
  return end > start ? int((end - start + bm - 1) / bm) : 0;
}

// Run g, counted over all experts in expert order -> expert, first row, end
// row of the expert.  Returns false when g is past the last run.
__device__ inline bool find_run(const int32_t* offs, int64_t E, int64_t rows, int bm, int g, int& e_out,
                                int64_t& row0, int64_t& row_end) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  int64_t carry = 0;    // clamped end offset of expert e0 - 1
  for (int64_t e0 = 0; e0 < E; e0 += 64) {
    const int64_t e = e0 + lane;
    // one offset per lane; an expert's start is the previous lane's end
    const int64_t end = e < E ? clamp_offset(offs[e], rows) : 0;
    const int64_t prev = __shfl_up(end, 1, 64);
    const int64_t start = lane == 0 ? carry : prev;
    const int cnt = e < E ? runs_of(start, end, bm) : 0;
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    const bool hit = (base + incl > g) && (base + incl - cnt <= g) && cnt > 0;
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      const int src = __builtin_ctzll(mask);
      const int excl = __shfl(incl - cnt, src, 64);
      // in scalar registers: the tile's addressing and branches depend on them
      e_out = __builtin_amdgcn_readfirstlane(int(e0) + src);
      row0 = uniform64(__shfl(start, src, 64) + int64_t(g - base - excl) * bm);
      row_end = uniform64(__shfl(end, src, 64));
      return true;
    }
    base += __shfl(incl, 63, 64);
    carry = __shfl(end, 63, 64);
  }
  return false;
}

// The m-tiles of the grouped GEMM (256 rows) in a load-balancing order: the
// experts' tiles with more than 128 rows come first (expert order), then
// their tiles with at most 128 rows (an expert's last tile when its row count
// leaves a remainder of at most 128), so that the short tiles fill the end of
// the launch.  Tile g -> expert, first row, end row of the expert; false past
// the last tile.
__device__ inline bool find_mtile_long_first(const int32_t* offs, int64_t E, int64_t rows, int g, int& e_out,
                                             int64_t& row0, int64_t& row_end) {
  constexpr int BM = 256;
  const int lane = threadIdx.x & 63;
  // long tiles of expert e: the full ones plus a remainder of more than 128 rows
  auto counts = [&](int64_t start, int64_t end, int& nlong, int& nshort) {
    const int64_t m = end > start ? end - start : 0;
    const int64_t rem = m % BM;
    nlong = int(m / BM) + (rem > BM / 2 ? 1 : 0);
    nshort = (rem > 0 && rem <= BM / 2) ? 1 : 0;
  };
  int total_long = 0;
  for (int64_t e0 = 0; e0 < E; e0 += 64) {
    const int64_t e = e0 + lane;
    int nl = 0, ns = 0;
    if (e < E) {
      int64_t start, end;
      expert_range(offs, rows, e, start, end);
      counts(start, end, nl, ns);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) nl += __shfl_xor(nl, off, 64);
    total_long += nl;
  }
  const bool want_long = g < total_long;
  const int gg = want_long ? g : g - total_long;
  int base = 0;
  for (int64_t e0 = 0; e0 < E; e0 += 64) {
    const int64_t e = e0 + lane;
    int64_t start = 0, end = 0;
    int nl = 0, ns = 0;
    if (e < E) {
      expert_range(offs, rows, e, start, end);
      counts(start, end, nl, ns);
    }
    const int cnt = want_long ? nl : ns;
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    const bool hit = (base + incl > gg) && (base + incl - cnt <= gg) && cnt > 0;
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      const int src = __builtin_ctzll(mask);
      const int excl = __shfl(incl - cnt, src, 64);
      e_out = __builtin_amdgcn_readfirstlane(int(e0) + src);
      const int64_t s = uniform64(__shfl(start, src, 64));
      const int64_t en = uniform64(__shfl(end, src, 64));
      // a long tile j starts at 256 j; the short tile after the full ones
      row0 = want_long ? s + int64_t(gg - base - excl) * BM : s + (en - s) / BM * BM;
      row_end = en;
      return true;
    }
    base += __shfl(incl, 63, 64);
  }
  return false;
}

// Runs of bm rows of the experts before e (first) and of expert e (count).
__device__ inline void runs_before(const int32_t* offs, int64_t rows, int bm, int64_t e, int64_t& first,
                                   int& count) {
  const int lane = threadIdx.x & 63;
  int64_t acc = 0;
  for (int64_t e0 = 0; e0 < e; e0 += 64) {
    const int64_t ee = e0 + lane;
    if (ee < e) {
      int64_t start, end;
      expert_range(offs, rows, ee, start, end);
      acc += runs_of(start, end, bm);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  // every lane holds the sum: make it visibly wave-uniform (scalar registers)
  first = uniform64(acc);
  int64_t start, end;
  expert_range(offs, rows, e, start, end);
  count = __builtin_amdgcn_readfirstlane(runs_of(start, end, bm));
}

}  // namespace grp
}  // namespace fp8mm
