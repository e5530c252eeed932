// FP8 (E4M3) scaled GEMM kernels for gfx950 (CDNA4) matrix cores.
//
//   out[i, j] = sum_k A[i,k] sA(i,k) * B(j,k) sB(j,k)  (+ bias[j])
//
// The formulation is the fused scaled-mm call of ColossalAI PR #6419 ("Fix:
// Handle LowLevelZeroPlugin with use_fp8=True", "Forward pass"); the recipes
// are those of pytorch PR #164141 ("Add _scaled_mm_v2 API") and pytorch/ao PR
// #2784 ("improve fp8 blockwise gemm perf"); the grouped form is that of
// pytorch/ao PR #4390 ("Add _grouped_mm dispatch handler to Float8Tensor").
//
// Design (MI355X first):
//  * One workgroup of 4 waves computes a BM x BN output tile; each wave a
//    TM x TN sub-tile made of 16x16 fragments.  The K loop walks 128-byte
//    steps: one v_mfma_f32_16x16x128_f8f6f4 consumes exactly one 128-wide K
//    block, which is also the scaling block of the blockwise recipes.
//  * A and B (B stored [N, K]) are staged global -> LDS with direct-to-LDS
//    buffer loads (no VGPR round trip), double buffered, one barrier per K
//    step.  LDS rows are 128 bytes; 16-byte chunk c of row r sits at slot
//    c ^ (r & 7) so that fragment reads of 8 consecutive rows hit 8 distinct
//    bank groups.  Buffer descriptors clip the ragged M / N / K edges to zero.
//  * B stored [K, N] (grad_input's weight) is loaded to registers and
//    byte-transposed with v_perm_b32 on its way into the same [N][128] LDS
//    layout.
//  * Tensorwise / rowwise: the MFMA accumulates straight into the fp32
//    accumulator; scales and bias are applied once in the epilogue.
//    Blockwise: each 128-K block's MFMA result is promoted into the fp32
//    accumulator with acc += P * sA * sB (the per-block scales are staged in
//    LDS next to the tiles).
//  * Workgroup ids are remapped so that each of the 8 XCDs (each with its own
//    L2) owns a contiguous range of tiles, walked in groups of 8 tile rows.
//  * Grouped (MoE): the tile space is (expert m-tiles) x (N tiles); every
//    workgroup finds its expert from the device-resident offsets with a
//    64-lane prefix scan, so no host synchronization is needed.
#include "launch.hpp"

namespace fp8mm {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int BK = 128;

__device__ __forceinline__ v4f mfma_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
  // Zero scale operands select the unscaled FP8 x FP8 instruction
  // (cbsz = blgp = 0: both operands E4M3).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// 4x4 byte transpose: rows r[0..3] hold 4 consecutive k for 4 n (byte n of
// r[k]); the result c[n] holds byte k = r[k].byte(n).
__device__ __forceinline__ void transpose4x4(const uint32_t r[4], uint32_t c[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
  const uint32_t t2 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);
  const uint32_t t3 = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
  c[0] = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
  c[1] = __builtin_amdgcn_perm(t1, t0, 0x07060302u);
  c[2] = __builtin_amdgcn_perm(t3, t2, 0x05040100u);
  c[3] = __builtin_amdgcn_perm(t3, t2, 0x07060302u);
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
};

template <int BM, int BN, int WM, Epi EPI, bool B_KN, bool OUT_BF16, bool BIAS, bool GROUPED>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmProblem p, int tiles_m, int tiles_n) {
  constexpr int WN = 4 / WM;
  constexpr int TM = BM / WM;
  constexpr int TN = BN / WN;
  constexpr int FM = TM / 16;
  constexpr int FN = TN / 16;
  constexpr bool BLOCKWISE = EPI == Epi::Block128x128 || EPI == Epi::Block128x1;
  constexpr int A_BYTES = BM * BK;
  constexpr int B_BYTES = BN * BK;
  constexpr int SA_BYTES = BLOCKWISE ? BM * 4 : 0;
  constexpr int SB_BYTES = EPI == Epi::Block128x1 ? BN * 4 : 0;
  constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile shape");
  static_assert(!BLOCKWISE || TN <= 128, "a wave's columns must sit in one 128-column scale block");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---------------- tile selection ----------------
  const int nblk = gridDim.x;
  const int per_xcd = nblk / 8;   // the launcher pads the grid to a multiple of 8
  const int lin = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  TileInfo ti;
  if constexpr (!GROUPED) {
    if (lin >= tiles_m * tiles_n) return;
    constexpr int GROUP_M = 8;
    const int span = GROUP_M * tiles_n;
    const int first_m = (lin / span) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (lin % span) % gsize;
    const int tn = (lin % span) / gsize;
    ti.row0 = int64_t(tm) * BM;
    ti.rows_valid = int(min<int64_t>(BM, p.M - ti.row0));
    ti.n0 = int64_t(tn) * BN;
    ti.cols_valid = int(min<int64_t>(BN, p.N - ti.n0));
    ti.A = p.A + ti.row0 * p.lda;
    ti.B = B_KN ? p.B + ti.n0 : p.B + ti.n0 * p.ldb;
    ti.sb = p.sb;
    ti.bias = p.bias;
  } else {
    // lin = tn * tiles_m + g: the m-tiles of one expert are adjacent.
    const int tn = lin / tiles_m;
    const int g = lin % tiles_m;
    if (tn >= tiles_n) return;
    // Find expert e with prefix[e] <= g < prefix[e] + count[e].
    int base = 0;
    int e_found = -1, mt = 0;
    int64_t start_found = 0, end_found = 0;
    for (int64_t e0 = 0; e0 < p.E && e_found < 0; e0 += 64) {
      const int64_t e = e0 + lane;
      int64_t start = 0, end = 0;
      if (e < p.E) {
        end = min<int64_t>(max<int64_t>(p.offsets[e], 0), p.M);
        start = e == 0 ? 0 : min<int64_t>(max<int64_t>(p.offsets[e - 1], 0), p.M);
      }
      const int cnt = end > start ? int((end - start + BM - 1) / BM) : 0;
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
        e_found = int(e0) + src;
        const int excl = __shfl(incl - cnt, src, 64);
        mt = g - base - excl;
        start_found = __shfl(start, src, 64);
        end_found = __shfl(end, src, 64);
      }
      base += __shfl(incl, 63, 64);
    }
    if (e_found < 0) return;
    ti.row0 = start_found + int64_t(mt) * BM;
    ti.rows_valid = int(min<int64_t>(BM, end_found - ti.row0));
    ti.n0 = int64_t(tn) * BN;
    ti.cols_valid = int(min<int64_t>(BN, p.N - ti.n0));
    ti.A = p.A + ti.row0 * p.lda;
    ti.B = p.B + int64_t(e_found) * p.N * p.K + ti.n0 * p.ldb;
    ti.sb = p.sb + int64_t(e_found) * p.N;
    ti.bias = BIAS ? p.bias + int64_t(e_found) * p.N : nullptr;
  }

  const int K = int(p.K);
  const int nk = (K + BK - 1) / BK;

  // ---------------- loaders ----------------
  // Direct-to-LDS loads: instruction i of wave w fills tile rows
  // [(i*4 + w) * 8, +8); lane l writes LDS bytes [16 l, 16 l + 16) of that
  // 1 KiB span, i.e. row l/8, slot l%8, which holds chunk (l%8) ^ (l/8).
  const int ld_row = lane >> 3;
  const int ld_chunk = (lane & 7) ^ ld_row;
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(ti.A, uint32_t(ti.rows_valid) * uint32_t(p.lda));
  __amdgpu_buffer_rsrc_t rsB;
  if constexpr (!B_KN) rsB = make_rsrc(ti.B, uint32_t(ti.cols_valid) * uint32_t(p.ldb));
  else rsB = make_rsrc(ti.B, uint32_t(K) * uint32_t(p.ldb) - uint32_t(ti.n0));

  auto issue_direct = [&](int stage, int kt) {
    uint8_t* st = smem + stage * STAGE;
    const int k0 = kt * BK;
    const bool kin = k0 + ld_chunk * 16 < K;
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
      const int r = (i * 4 + wave) * 8 + ld_row;
      const uint32_t off = kin ? uint32_t(r) * uint32_t(p.lda) + uint32_t(k0 + ld_chunk * 16) : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_ptr)(st + (i * 4 + wave) * 1024), 16, off, 0, 0, 0);
    }
    if constexpr (!B_KN) {
#pragma unroll
      for (int i = 0; i < BN / 32; ++i) {
        const int r = (i * 4 + wave) * 8 + ld_row;
        const uint32_t off = kin ? uint32_t(r) * uint32_t(p.ldb) + uint32_t(k0 + ld_chunk * 16) : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_ptr)(st + A_BYTES + (i * 4 + wave) * 1024), 16, off,
                                                 0, 0, 0);
      }
    }
    if constexpr (BLOCKWISE) {
      // sA[kb, row0 .. row0 + BM) -> LDS, one float per lane (scale rows are
      // only 4-byte aligned).  The descriptor spans to the end of the scale
      // array, so no load is partly out of range; rows past the tile edge
      // read neighbouring scales that only reach rows which are never stored.
      if (wave * 64 < BM) {
        const int64_t off = int64_t(kt) * p.M + ti.row0 + wave * 64;
        const int64_t rem = int64_t(nk) * p.M - off;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.sa + (rem > 0 ? off : 0), uint32_t(rem > 0 ? rem * 4 : 0));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(st + A_BYTES + B_BYTES + wave * 256), 4,
                                                 uint32_t(lane) * 4u, 0, 0, 0);
      }
      if constexpr (EPI == Epi::Block128x1) {
        if (wave * 64 < BN) {
          const int64_t off = int64_t(kt) * p.N + ti.n0 + wave * 64;
          const int64_t rem = int64_t(nk) * p.N - off;
          const __amdgpu_buffer_rsrc_t rs = make_rsrc(ti.sb + (rem > 0 ? off : 0), uint32_t(rem > 0 ? rem * 4 : 0));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(st + A_BYTES + B_BYTES + SA_BYTES + wave * 256),
                                                   4, uint32_t(lane) * 4u, 0, 0, 0);
        }
      }
    }
  };

  // B stored [K, N]: thread t loads KR consecutive k rows x 16 n bytes and
  // writes them transposed (n rows of the [N][128] tile).
  constexpr int NCH = BN / 16;              // 16-byte chunks per k row
  constexpr int KR = BK * NCH / 256;       // k rows per thread
  static_assert(!B_KN || KR == 4 || KR == 8, "KN loader shape");
  const int kn_nc = tid % NCH;
  const int kn_kg = tid / NCH;
  v4i kn_regs[B_KN ? KR : 1];
  auto kn_load = [&](int kt) {
    if constexpr (B_KN) {
      const int k0 = kt * BK + kn_kg * KR;
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        const bool in = (k0 + r < K) && (kn_nc * 16 < ti.cols_valid);
        const uint32_t off = in ? uint32_t(k0 + r) * uint32_t(p.ldb) + uint32_t(kn_nc * 16) : 0x80000000u;
        kn_regs[r] = __builtin_amdgcn_raw_buffer_load_b128(rsB, off, 0, 0);
      }
    }
  };
  auto kn_store = [&](int stage) {
    if constexpr (B_KN) {
      uint8_t* bt = smem + stage * STAGE + A_BYTES;
#pragma unroll
      for (int q = 0; q < 4; ++q) {          // 4-byte column group within the 16-byte chunk
        uint32_t cols[KR / 4][4];
#pragma unroll
        for (int h = 0; h < KR / 4; ++h) {
          uint32_t rr[4] = {uint32_t(kn_regs[h * 4 + 0][q]), uint32_t(kn_regs[h * 4 + 1][q]),
                            uint32_t(kn_regs[h * 4 + 2][q]), uint32_t(kn_regs[h * 4 + 3][q])};
          transpose4x4(rr, cols[h]);
        }
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) {
          const int n = kn_nc * 16 + q * 4 + jn;
          const int kl = kn_kg * KR;            // first k byte within the 128-byte row
          uint8_t* dst = bt + lds_off(n, kl >> 4) + (kl & 15);
          if constexpr (KR == 8) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(cols[0][jn], cols[1][jn]);
          } else {
            *reinterpret_cast<uint32_t*>(dst) = cols[0][jn];
          }
        }
      }
    }
  };

  // ---------------- accumulators ----------------
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int row_base = wm * TM;
  const int col_base = wn * TN;
  const int frow = lane & 15;   // fragment row (A) / column (B) of this lane
  const int fq = lane >> 4;     // which 32-byte quarter of the 128-byte K block
  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int stage, int kt) {
    const uint8_t* As = smem + stage * STAGE;
    const uint8_t* Bs = As + A_BYTES;
    v8i b[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = col_base + j * 16 + frow;
      const v4i lo = *reinterpret_cast<const v4i*>(Bs + lds_off(r, 2 * fq));
      const v4i hi = *reinterpret_cast<const v4i*>(Bs + lds_off(r, 2 * fq + 1));
      b[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    [[maybe_unused]] float sbk = 0.f;
    [[maybe_unused]] float sbv[FN];
    if constexpr (EPI == Epi::Block128x128) {
      const int64_t nb = (ti.n0 + col_base) / 128;
      sbk = B_KN ? ti.sb[int64_t(kt) * (p.N / 128) + nb] : ti.sb[nb * (K / BK) + kt];
    }
    if constexpr (EPI == Epi::Block128x1) {
      const float* sbs = reinterpret_cast<const float*>(As + A_BYTES + B_BYTES + SA_BYTES);
#pragma unroll
      for (int j = 0; j < FN; ++j) sbv[j] = sbs[col_base + j * 16 + frow];
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = row_base + i * 16 + frow;
      const v4i lo = *reinterpret_cast<const v4i*>(As + lds_off(r, 2 * fq));
      const v4i hi = *reinterpret_cast<const v4i*>(As + lds_off(r, 2 * fq + 1));
      const v8i a = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if constexpr (!BLOCKWISE) {
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_16x16x128(a, b[j], acc[i][j]);
      } else {
        const float* sas = reinterpret_cast<const float*>(As + A_BYTES + B_BYTES);
        v4f fa = *reinterpret_cast<const v4f*>(sas + row_base + i * 16 + fq * 4);
        if constexpr (EPI == Epi::Block128x128) fa = fa * sbk;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v4f t = mfma_16x16x128(a, b[j], v4f{0.f, 0.f, 0.f, 0.f});
          if constexpr (EPI == Epi::Block128x128) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(t[e], fa[e], acc[i][j][e]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(t[e] * sbv[j], fa[e], acc[i][j][e]);
          }
        }
      }
    }
  };

  // ---------------- main loop ----------------
  if (nk > 0) {
    issue_direct(0, 0);
    kn_load(0);
    kn_store(0);
    wait_vmem();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int s = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        issue_direct(s ^ 1, kt + 1);
        kn_load(kt + 1);
      }
      compute(s, kt);
      if (more) kn_store(s ^ 1);
      wait_vmem();
      __syncthreads();
    }
  }

  // ---------------- epilogue ----------------
  [[maybe_unused]] float s_tensor = 0.f;
  if constexpr (EPI == Epi::Tensor) s_tensor = p.sa[0] * p.sb[0];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int rl = row_base + i * 16 + fq * 4;   // local row of element 0
    [[maybe_unused]] float sar[4];
    if constexpr (EPI == Epi::Row) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sar[e] = (rl + e < ti.rows_valid) ? p.sa[ti.row0 + rl + e] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int cl = col_base + j * 16 + frow;
      if (cl >= ti.cols_valid) continue;
      const int64_t col = ti.n0 + cl;
      [[maybe_unused]] float sbc = 0.f;
      if constexpr (EPI == Epi::Row) sbc = ti.sb[col];
      float bias_v = 0.f;
      if constexpr (BIAS) bias_v = __uint_as_float(uint32_t(ti.bias[col]) << 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (rl + e >= ti.rows_valid) continue;
        float v = acc[i][j][e];
        if constexpr (EPI == Epi::Tensor) v = v * s_tensor;
        if constexpr (EPI == Epi::Row) v = (v * sar[e]) * sbc;
        if constexpr (BIAS) v = v + bias_v;
        const int64_t row = ti.row0 + rl + e;
        if constexpr (OUT_BF16)
          reinterpret_cast<uint16_t*>(p.out)[row * p.ldo + col] = f32_to_bf16_rne(v);
        else
          reinterpret_cast<float*>(p.out)[row * p.ldo + col] = v;
      }
    }
  }
}

template <int BM, int BN, int WM, Epi EPI, bool B_KN, bool OUT_BF16, bool BIAS, bool GROUPED>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t st) {
  int tiles_m, tiles_n = int((p.N + BN - 1) / BN);
  if (GROUPED)
    tiles_m = int((p.M + BM - 1) / BM + p.E);   // upper bound on expert m-tiles
  else
    tiles_m = int((p.M + BM - 1) / BM);
  const int64_t tiles = int64_t(tiles_m) * tiles_n;
  if (tiles == 0) return hipSuccess;
  const int grid = int((tiles + 7) / 8 * 8);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, EPI, B_KN, OUT_BF16, BIAS, GROUPED>), dim3(grid), dim3(256), 0, st, p,
                     tiles_m, tiles_n);
  return hipGetLastError();
}

template <Epi EPI, bool B_KN, bool OUT_BF16, bool BIAS, bool GROUPED>
hipError_t launch_epi(const GemmProblem& p, hipStream_t st) {
  if constexpr (GROUPED)
    return launch_cfg<128, 128, 2, EPI, false, OUT_BF16, BIAS, true>(p, st);
  else if constexpr (EPI == Epi::Block128x128 || EPI == Epi::Block128x1)
    return launch_cfg<256, 128, 2, EPI, B_KN, OUT_BF16, BIAS, false>(p, st);
  else
    return launch_cfg<256, 256, 2, EPI, B_KN, OUT_BF16, BIAS, false>(p, st);
}

template <Epi EPI, bool B_KN, bool GROUPED>
hipError_t launch_out(const GemmProblem& p, hipStream_t st) {
  const bool bias = p.bias != nullptr;
  if (p.out_bf16)
    return bias ? launch_epi<EPI, B_KN, true, true, GROUPED>(p, st) : launch_epi<EPI, B_KN, true, false, GROUPED>(p, st);
  return bias ? launch_epi<EPI, B_KN, false, true, GROUPED>(p, st) : launch_epi<EPI, B_KN, false, false, GROUPED>(p, st);
}

}  // namespace

hipError_t launch_gemm(const GemmProblem& p, hipStream_t st) {
  if (p.offsets) return launch_out<Epi::Row, false, true>(p, st);
  switch (p.epi) {
    case Epi::Tensor:
      return p.b_kn ? launch_out<Epi::Tensor, true, false>(p, st) : launch_out<Epi::Tensor, false, false>(p, st);
    case Epi::Row:
      return p.b_kn ? launch_out<Epi::Row, true, false>(p, st) : launch_out<Epi::Row, false, false>(p, st);
    case Epi::Block128x128:
      return p.b_kn ? launch_out<Epi::Block128x128, true, false>(p, st)
                    : launch_out<Epi::Block128x128, false, false>(p, st);
    case Epi::Block128x1:
      return p.b_kn ? launch_out<Epi::Block128x1, true, false>(p, st)
                    : launch_out<Epi::Block128x1, false, false>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fp8mm
