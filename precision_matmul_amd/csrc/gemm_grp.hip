// Grouped (MoE) FP8 (E4M3) scaled GEMM for gfx950 in the weight-streaming
// regime.
//
//   out[rows_e, :] = (A[rows_e] sA) @ (W[e] sB[e])^T  (+ bias)
//
// The grouped form of pytorch/ao PR #4390 ("Add _grouped_mm dispatch handler
// to Float8Tensor", "Design"): expert e owns rows [offs[e-1], offs[e]) of A
// and multiplies them by its own weights W[e], stored [N, K] (K contiguous).
// Rowwise x rowwise (per-token and per-output-row scales), as on that page,
// and the 1x128 x 128x128 recipe of pytorch/ao PR #2784 ("improve fp8
// blockwise gemm perf") applied per expert.
//
// When the experts own a few hundred rows each, the call streams the expert
// weights from HBM and does little arithmetic per weight byte: at E = 64,
// 16384 routed rows, N = 1408, K = 2048 it moves 185 MB of weights for 94.5
// GFLOP, under the machine balance of the chip.  The layout serves that:
//  * An m-block holds up to 320 rows of one expert, so an expert with at
//    most 320 rows reads each of its weight slices once (tiles of 256 rows
//    stream the slice a second time for the expert's remainder rows).
//  * An n-block has bn <= 192 columns; the launcher picks bn so that N splits
//    into equal blocks (1408 = 8 x 176), which at the MoE shape gives 512
//    tiles of equal weight traffic: two full rounds of the 256 CUs.
//  * Weight tiles go through a three-deep LDS ring, A rows (shared by the
//    n-blocks of an m-block through L2) through a two-deep one.  Each K step
//    waits only for the tiles it is about to use: the weight tiles of the
//    step after it stay in flight across the barrier.
//  * The n-blocks of one m-block run on one XCD, whose L2 then holds the
//    m-block's A rows; m-blocks are dealt to the XCDs round-robin.
//
// Waves.  8 waves, wave w: column group cg = w >> 2, row group rg = (w +
// cg) & 3.  Row fragment i (i < 5) of the wave is tile rows 16 (rg + 4 i) ..
// +15, so the valid rows of a short m-block spread over all four SIMDs (SIMD
// = w & 3), and the two waves of a SIMD have different row groups: a fifth
// row fragment that only one row group has (an m-block of 257 to 272 rows)
// falls on two SIMDs, not twice on one.  Column fragment j (j < 6) is tile
// columns 96 cg + 16 j .. +15.  Each
// fragment is a v_mfma_f32_16x16x128_f8f6f4 block computed transposed (the
// weight fragment as the first operand), so a lane holds one output row and
// four adjacent columns: one row scale per lane and fragment, 8- or 16-byte
// stores.
#include <type_traits>

#include "gemm_common.hpp"

namespace fp8mm {
namespace {

using namespace gk;

constexpr int GW_MB = 320;                 // rows of an m-block
constexpr int GW_BN = 192;                 // columns of the LDS weight tile (bn <= 192 valid)
constexpr int GW_NW = 8;
constexpr int GW_RF = 5;                   // row fragments per wave
constexpr int GW_CF = 6;                   // column fragments per wave
constexpr int GW_A = GW_MB * BK;           // A codes of one K step (40 KiB)
constexpr int GW_SA = GW_MB * 4;           // 1x128 row scales of one K step
constexpr int GW_SB = 256;                 // 128x128 block scales of one K step (up to 3 used)
constexpr int GW_ASTAGE = GW_A + GW_SA + GW_SB;
constexpr int GW_ASTAGE_PAD = (GW_ASTAGE + 1023) / 1024 * 1024;
constexpr int GW_B = GW_BN * BK;           // weight codes of one K step (24 KiB)
constexpr int GW_LA = GW_MB / 8 / GW_NW;   // 1 KiB A loads per wave per step (5)
constexpr int GW_LB = GW_BN / 8 / GW_NW;   // 1 KiB weight loads per wave per step (3)
static_assert(2 * GW_ASTAGE_PAD + 3 * GW_B <= 160 * 1024, "LDS budget");
static_assert(GW_LA * 8 * GW_NW == GW_MB && GW_LB * 8 * GW_NW == GW_BN, "loads per wave");

template <Epi EPI, bool OUT_BF16, bool BIAS, bool K_ALIGNED>
__global__ __launch_bounds__(GW_NW * 64, 1) void gemm_grouped_wide_kernel(GemmProblem p, int n_blocks, int bn,
                                                                         int vec_out) {
  constexpr bool BLOCKWISE = EPI == Epi::Block128x128;
  static_assert(EPI == Epi::Row || EPI == Epi::Block128x128, "grouped: rowwise or 1x128 x 128x128");
  constexpr int OUTB = OUT_BF16 ? 2 : 4;

  // One LDS array: the A and weight rings during the K loop, the output
  // staging area after it.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * GW_ASTAGE_PAD + 3 * GW_B];
  uint8_t* const a_ring = smem;
  uint8_t* const b_ring = smem + 2 * GW_ASTAGE_PAD;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---------------- tile ----------------
  // Workgroup b runs on XCD x = b % 8 (workgroups are dealt to the XCDs
  // round-robin); slot r = b / 8 of that XCD takes n-block r % n_blocks of
  // the XCD's m-block r / n_blocks, which is m-block g = (r / n_blocks) * 8
  // + x over all experts.  The grid is sized for the most m-blocks the
  // offsets can give; the real ones are a prefix in g, so workgroups past it
  // exit at once.
  const int x = blockIdx.x % 8;
  const int r = blockIdx.x / 8;
  const int g = (r / n_blocks) * 8 + x;
  const int nb = r % n_blocks;
  int e = 0;
  int64_t row0 = 0, rend = 0;
  if (!grp::find_run(p.offsets, p.E, p.M, GW_MB, g, e, row0, rend)) return;
  const int rows_valid = int(min<int64_t>(GW_MB, rend - row0));
  const int64_t n0 = int64_t(nb) * bn;
  const int cols_valid = int(min<int64_t>(bn, p.N - n0));
  if (cols_valid <= 0 || rows_valid <= 0) return;
  const int K = int(p.K);
  const int nk = (K + BK - 1) / BK;
  const uint8_t* We = p.B + int64_t(e) * p.N * p.K;
  const float* sbe = p.sb + int64_t(e) * (BLOCKWISE ? (p.N / 128) * (p.K / 128) : p.N);
  [[maybe_unused]] const uint16_t* biase = BIAS ? p.bias + int64_t(e) * p.bias_stride_e : nullptr;

  // ---------------- loaders ----------------
  // A: wave w fills tile rows [40 w, 40 w + 40), five 1 KiB loads of 8 rows;
  // weights: rows (output columns) [24 w, 24 w + 24), three loads.  Lane l of
  // a load writes LDS bytes [16 l, +16) of its 1 KiB: row l / 8 of the load,
  // slot l % 8, which holds chunk (l % 8) ^ swz(row).  The descriptors end at
  // the m-block's last row and the n-block's last column, so rows and
  // columns past them read zeros; chunks past a ragged K end likewise.
  const Rsrc rsA = make_rsrc4(p.A + row0 * p.lda, uint32_t(rows_valid) * uint32_t(p.lda));
  const Rsrc rsB = make_rsrc4(We + n0 * p.ldb, uint32_t(cols_valid) * uint32_t(p.ldb));
  // Load q of a wave starts at a row 8 q + a multiple of 8 whose swz() parity
  // (bit 2) is that of q + w: 40 w and 24 w are multiples of 8 with 40 w / 2
  // and 24 w / 2 = 4 w (mod 8), so swz(row) = (l >> 4) | (((q + w) & 1) << 2)
  // for lane l, and the chunk of lane l is (l & 7) ^ swz(row).
  const int ch_even = (lane & 7) ^ (lane >> 4);          // q + w even
  const int ch_odd = (lane & 7) ^ (4 | (lane >> 4));     // q + w odd
  const uint32_t rowA = uint32_t(wave * 40 + (lane >> 3)) * uint32_t(p.lda);
  const uint32_t rowB = uint32_t(wave * 24 + (lane >> 3)) * uint32_t(p.ldb);
  const uint32_t ldsA = lds_addr(a_ring), ldsB = lds_addr(b_ring);

  // Blockwise scales of K step kt, loaded with the A rows: waves 0..4 the
  // 1x128 row scales sA[kt, row0 + 64 w .. +64) (the descriptor spans to the
  // end of the array, so rows past the m-block read neighbouring scales that
  // reach no stored output), wave 5 the 128x128 scales of the weight blocks
  // n0 / 128 + l (l < 3 used) of expert e.
  [[maybe_unused]] const int64_t nkb = p.K / 128;
  [[maybe_unused]] const int64_t blk0 = n0 / 128;
  // A load q (q < 5) of K step kt into A slot kt % 2: tile rows 40 w + 8 q
  // .. +7.  Rows wholly past the m-block are not loaded: their LDS rows feed
  // only accumulators that are never stored.  The last load of a step also
  // brings its blockwise scales.
  auto load_a = [&](int kt, int q) {
    const int s = kt & 1;
    const bool live = kt < nk;
    const uint32_t k0 = uint32_t(kt) * BK;
    if (wave * 40 + q * 8 < rows_valid) {
      const Rsrc ra = live ? rsA : dead(rsA);
      const int ch = ((q + wave) & 1) ? ch_odd : ch_even;
      uint32_t vo = rowA + uint32_t(q * 8) * uint32_t(p.lda) + uint32_t(ch * 16);
      if (!K_ALIGNED && int(k0) + ch * 16 >= K) vo = 0x80000000u;
      dma_b128(ra, ldsA + s * GW_ASTAGE_PAD + (wave * 40 + q * 8) * 128, vo, k0);
    }
    if (BLOCKWISE && q == GW_LA - 1) {
      const uint32_t sc = ldsA + s * GW_ASTAGE_PAD + GW_A;
      if (wave < 5) {
        const int64_t off = int64_t(kt) * p.M + row0 + wave * 64;
        const int64_t rem = int64_t(nk) * p.M - off;
        const Rsrc r2 = make_rsrc4(p.sa + (rem > 0 ? off : 0), uint32_t(live && rem > 0 ? rem * 4 : 0));
        dma_b32(r2, sc + wave * 256, uint32_t(lane) * 4u);
      } else if (wave == 5) {
        const int64_t nblk = p.N / 128;
        const Rsrc r2 = make_rsrc4(sbe, uint32_t(live ? nblk * nkb * 4 : 0));
        dma_b32(r2, sc + GW_SA, uint32_t((blk0 + lane) * nkb + kt) * 4u);
      }
    }
  };
  // Weight load q (q < 3) of K step kt into ring slot kt % 3: n-block
  // columns 24 w + 8 q .. +7.  Past the last step the loads go through a
  // descriptor with no valid bytes (zeros into a slot nobody reads), so that
  // every step issues the same three loads last and one vmcnt immediate
  // tracks the ring.
  auto load_b = [&](int kt, int q) {
    const int s = kt % 3;
    const uint32_t k0 = uint32_t(kt) * BK;
    const Rsrc rb = kt < nk ? rsB : dead(rsB);
    const int ch = ((q + wave) & 1) ? ch_odd : ch_even;
    uint32_t vo = rowB + uint32_t(q * 8) * uint32_t(p.ldb) + uint32_t(ch * 16);
    if (!K_ALIGNED && int(k0) + ch * 16 >= K) vo = 0x80000000u;
    dma_b128(rb, ldsB + s * GW_B + (wave * 24 + q * 8) * 128, vo, k0);
  };
  auto issue_a = [&](int kt) {
#pragma unroll
    for (int q = 0; q < GW_LA; ++q) load_a(kt, q);
  };
  auto issue_b = [&](int kt) {
#pragma unroll
    for (int q = 0; q < GW_LB; ++q) load_b(kt, q);
  };
  // The loads that K step kt issues (A of kt + 1, then the weights of kt +
  // 2), spread over its six column slots so that the load instructions queue
  // between MFMAs instead of holding them back at the top of the step.
  auto issue_slot = [&](int kt, int j) {
    if (j == 0) { load_a(kt + 1, 0); load_a(kt + 1, 1); }
    if (j == 1) { load_a(kt + 1, 2); load_a(kt + 1, 3); }
    if (j == 2) load_a(kt + 1, 4);
    if (j >= 3) load_b(kt + 2, j - 3);
  };

  // ---------------- registers ----------------
  const int cg = wave >> 2;
  const int rg = (wave + cg) & 3;
  const int frow = lane & 15;
  const int fq = lane >> 4;
  const int col_base = cg * 96;
  // whether this wave's fifth row fragment (tile rows 16 (rg + 16) ..) holds
  // any of the m-block's rows
  const bool five = 16 * (rg + 16) < rows_valid;
  const bool cact = col_base < cols_valid;
  v4f acc[GW_RF][GW_CF];
#pragma unroll
  for (int i = 0; i < GW_RF; ++i)
#pragma unroll
    for (int j = 0; j < GW_CF; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Fragment reads.  Every fragment row the wave reads is a multiple of 16
  // plus frow, so swz(row) = (frow >> 1) & 7 for all of them: the lane's two
  // chunk offsets are fixed, and fragment f of a tile sits 2048 f bytes on.
  const int off_lo = frow * 128 + ((fq ^ swz(frow)) << 4);
  const int off_hi = frow * 128 + (((fq + 4) ^ swz(frow)) << 4);
  auto read_frag16 = [&](const uint8_t* tile, int f) {
    const v4i lo = *reinterpret_cast<const v4i*>(tile + off_lo + f * 2048);
    const v4i hi = *reinterpret_cast<const v4i*>(tile + off_hi + f * 2048);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  // One K step.  The weight fragment of column j + 1 is read while column
  // j's MFMAs run.  Rowwise: the fifth row fragment only where the m-block
  // reaches it (an m-block of at most 256 rows has four per wave), and no
  // column fragment past the n-block's columns (176 of 192 at N = 1408): a
  // wave-uniform branch per column.  Blockwise: each MFMA's 128-K partial is
  // promoted into the accumulator one MFMA later (acc += P sA(row)
  // sB(block)), so the FMAs never wait for the MFMA that produces their
  // input; that pipeline runs NV row and NC column fragments: a fifth row
  // fragment past the m-block (every wave's, for an m-block of at most 256
  // rows) and a last column wholly past the n-block (the second column
  // group's at bn = 176) are left out, with one form of the K loop per
  // count.  Every wave holds all five row fragments' accumulators either
  // way: a branch per MFMA, or accumulators only for the fragments a form
  // runs, makes the compiler keep more fragments live than the 256 registers
  // hold.
  auto compute = [&](int kt, auto nv, auto nc) {
    constexpr int NV = BLOCKWISE ? decltype(nv)::value : GW_RF;
    constexpr int NC = BLOCKWISE ? decltype(nc)::value : GW_CF;
    const uint8_t* As = a_ring + (kt & 1) * GW_ASTAGE_PAD;
    const uint8_t* Bs = b_ring + (kt % 3) * GW_B;
    v8i a[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (BLOCKWISE || i < NV - 1 || five) a[i] = read_frag16(As, rg + 4 * i);

    [[maybe_unused]] float fa[NV];
    [[maybe_unused]] const float* sbs = reinterpret_cast<const float*>(As + GW_A + GW_SA);
    if constexpr (BLOCKWISE) {
      const float* sas = reinterpret_cast<const float*>(As + GW_A);
#pragma unroll
      for (int i = 0; i < NV; ++i) fa[i] = sas[16 * (rg + 4 * i) + frow];
    }
    [[maybe_unused]] v4f t_prev = v4f{0.f, 0.f, 0.f, 0.f};
    [[maybe_unused]] float f_prev = 0.f;
    v8i b = read_frag16(Bs, col_base / 16);
#pragma unroll
    for (int j = 0; j < GW_CF; ++j) {
      issue_slot(kt, j);
      const bool col_j = BLOCKWISE ? j < NC : col_base + 16 * j < cols_valid;
      v8i bnext = b;
      if (j + 1 < GW_CF && (BLOCKWISE ? j + 1 < NC : col_base + 16 * (j + 1) < cols_valid))
        bnext = read_frag16(Bs, col_base / 16 + j + 1);
      [[maybe_unused]] float sbj = 0.f;
      if constexpr (BLOCKWISE) sbj = sbs[(n0 + col_base + 16 * j) / 128 - blk0];
      if (col_j) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          if (!BLOCKWISE && i == NV - 1 && !five) continue;
          if constexpr (BLOCKWISE) {
            const v4f t = mfma_16x16x128(b, a[i], v4f{0.f, 0.f, 0.f, 0.f});
            if (i > 0 || j > 0) {
              const int ip = i > 0 ? i - 1 : NV - 1;
              const int jp = i > 0 ? j : j - 1;
#pragma unroll
              for (int c = 0; c < 4; ++c) acc[ip][jp][c] = __builtin_fmaf(t_prev[c], f_prev, acc[ip][jp][c]);
            }
            t_prev = t;
            f_prev = fa[i] * sbj;
          } else {
            acc[i][j] = mfma_16x16x128(b, a[i], acc[i][j]);
          }
        }
      }
      b = bnext;
      // one column at a time: otherwise the scheduler lifts every weight
      // fragment read to the top of the step and runs out of registers
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (BLOCKWISE) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[NV - 1][NC - 1][c] = __builtin_fmaf(t_prev[c], f_prev, acc[NV - 1][NC - 1][c]);
    }
  };

  // ---------------- K loop ----------------
  // During step kt, A (and scales) of kt+1 go to A slot (kt+1) % 2 and the
  // weights of kt+2 to B slot (kt+2) % 3, both last read by step kt-1, which
  // every wave finished before the previous barrier.  After step kt each
  // wave waits for all but its newest three loads (the weights of kt+2), so
  // A of kt+1 and the weights of kt+1 (issued a step earlier) have landed,
  // and the barrier makes them visible to every wave.
  // Rowwise: the epilogue's scales go to LDS now, long before they are
  // needed, into the A stages' blockwise scale regions (unused by this
  // recipe): the column scales sB[e, n0 .. n0 + bn) into stage 0's (waves
  // 0-2, 64 floats each), the row scales sA[row0 .. row0 + 320) into stage
  // 1's (waves 3-7).  Entries past the tile's rows or columns read zeros.
  if constexpr (EPI == Epi::Row) {
    if (wave < 3) {
      const Rsrc r2 = make_rsrc4(sbe + n0, uint32_t(cols_valid) * 4u);
      dma_b32(r2, ldsA + GW_A + wave * 256, uint32_t(wave * 64 + lane) * 4u);
    } else {
      const Rsrc r2 = make_rsrc4(p.sa + row0, uint32_t(rows_valid) * 4u);
      dma_b32(r2, ldsA + GW_ASTAGE_PAD + GW_A + (wave - 3) * 256, uint32_t((wave - 3) * 64 + lane) * 4u);
    }
  }
  issue_a(0);
  issue_b(0);
  issue_b(1);
  asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  auto k_loop = [&](auto nv, auto nc) {
    for (int kt = 0; kt < nk; ++kt) {
      if (cact) {
        compute(kt, nv, nc);
      } else {
#pragma unroll
        for (int j = 0; j < GW_CF; ++j) issue_slot(kt, j);
      }
      asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // blockwise: the fifth row fragment and the last column fragment only
  // where they hold any of the tile's rows or columns
  using all_rows = std::integral_constant<int, GW_RF>;
  using all_cols = std::integral_constant<int, GW_CF>;
  using four_rows = std::integral_constant<int, GW_RF - 1>;
  using five_cols = std::integral_constant<int, GW_CF - 1>;
  const bool six = col_base + 16 * (GW_CF - 1) < cols_valid;
  if (!BLOCKWISE || (five && six))
    k_loop(all_rows(), all_cols());
  else if (five)
    k_loop(all_rows(), five_cols());
  else if (six)
    k_loop(four_rows(), all_cols());
  else
    k_loop(four_rows(), five_cols());
  // the dead loads of the last two steps (zeros into unread slots)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---------------- epilogue: scales, bias, one rounding, staged stores ----------------
  // The tile's outputs go through LDS (free after the K loop) so that whole
  // rows leave in 16-byte stores from consecutive lanes: full 128-byte lines
  // per 8 lanes.  (Non-temporal stores straight from the fragment layout, 32
  // bytes per row per instruction, wrote about twice the output's bytes.)
  // bf16: the whole 320 x 192 tile in one pass; fp32: one pass per column
  // group (96 columns).
  constexpr int PASSES = OUT_BF16 ? 1 : 2;
  constexpr int PW = GW_BN / PASSES;                  // columns per pass
  constexpr int PITCH = PW * OUTB + 16;               // padded staging row (bytes)
  static_assert(GW_MB * PITCH <= 2 * GW_ASTAGE_PAD + 3 * GW_B, "staging fits the LDS");
  constexpr int CPR_MAX = PW * OUTB / 16;             // 16-byte chunks per staged row
  // Rowwise scales from LDS (loaded in the prologue), into registers before
  // the staging area overwrites them.
  [[maybe_unused]] float sr[GW_RF];
  [[maybe_unused]] float scol[GW_CF][4];
  if constexpr (EPI == Epi::Row) {
    const float* lsb = reinterpret_cast<const float*>(smem + GW_A);
    const float* lsa = reinterpret_cast<const float*>(smem + GW_ASTAGE_PAD + GW_A);
#pragma unroll
    for (int i = 0; i < GW_RF; ++i) sr[i] = lsa[16 * (rg + 4 * i) + frow];
#pragma unroll
    for (int j = 0; j < GW_CF; ++j)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) scol[j][cc] = lsb[col_base + 16 * j + 4 * fq + cc];
  }
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    __syncthreads();    // the K loop's last LDS reads, or the previous pass's copy-out, are done
    if (cact && (PASSES == 1 || cg == pass)) {
#pragma unroll
      for (int j = 0; j < GW_CF; ++j) {
        const int c = col_base + 16 * j + 4 * fq;     // tile column of the lane's first value
        float sc[4] = {1.f, 1.f, 1.f, 1.f};
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          if constexpr (EPI == Epi::Row) sc[cc] = scol[j][cc];
          if constexpr (BIAS) {
            if (c + cc < cols_valid) bv[cc] = __uint_as_float(uint32_t(biase[n0 + c + cc]) << 16);
          }
        }
#pragma unroll
        for (int i = 0; i < GW_RF; ++i) {
          const int rt = 16 * (rg + 4 * i) + frow;
          float v[4];
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            v[cc] = acc[i][j][cc];
            if constexpr (EPI == Epi::Row) v[cc] = (v[cc] * sr[i]) * sc[cc];
            if constexpr (BIAS) v[cc] = v[cc] + bv[cc];
          }
          uint8_t* dst = smem + rt * PITCH + (c - pass * PW) * OUTB;
          if constexpr (OUT_BF16) {
            *reinterpret_cast<uint2*>(dst) =
                uint2{uint32_t(f32_to_bf16_rne(v[0])) | (uint32_t(f32_to_bf16_rne(v[1])) << 16),
                      uint32_t(f32_to_bf16_rne(v[2])) | (uint32_t(f32_to_bf16_rne(v[3])) << 16)};
          } else {
            *reinterpret_cast<v4f*>(dst) = v4f{v[0], v[1], v[2], v[3]};
          }
        }
      }
    }
    __syncthreads();
    // copy-out: staged rows [0, rows_valid), the pass's valid columns
    const int pc0 = pass * PW;                              // first tile column of the pass
    const int pcols = min(PW, cols_valid - pc0);            // valid columns in the pass
    const int cpr = (pcols * OUTB + 15) / 16;
    if (pcols > 0 && vec_out && (pcols * OUTB) % 16 == 0) {
      // whole 16-byte chunks only: each thread has four LDS reads in flight
      // before their stores (one at a time, every copy waited out the LDS
      // latency)
      constexpr int NT = GW_NW * 64;
      const int total = rows_valid * CPR_MAX;
      uint8_t* const obase = reinterpret_cast<uint8_t*>(p.out) + (row0 * p.ldo + n0 + pc0) * OUTB;
      for (int base = int(threadIdx.x); base < total; base += 4 * NT) {
        v4i val[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int idx = base + u * NT;
          const int rt = idx / CPR_MAX, ch = idx % CPR_MAX;
          if (idx < total && ch < cpr) val[u] = *reinterpret_cast<const v4i*>(smem + rt * PITCH + ch * 16);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int idx = base + u * NT;
          const int rt = idx / CPR_MAX, ch = idx % CPR_MAX;
          // plain stores: L2 merges the partial lines at the n-block edges
          // (non-temporal ones wrote 51 MB for the 46 MB MoE output)
          if (idx < total && ch < cpr) *reinterpret_cast<v4i*>(obase + int64_t(rt) * p.ldo * OUTB + ch * 16) = val[u];
        }
      }
    } else if (pcols > 0) {
      for (int idx = int(threadIdx.x); idx < rows_valid * CPR_MAX; idx += GW_NW * 64) {
        const int rt = idx / CPR_MAX;
        const int ch = idx % CPR_MAX;
        if (ch >= cpr) continue;
        const uint8_t* src = smem + rt * PITCH + ch * 16;
        uint8_t* dst = reinterpret_cast<uint8_t*>(p.out) + ((row0 + rt) * p.ldo + n0 + pc0) * OUTB + ch * 16;
        const int nvals = min(16 / OUTB, pcols - ch * (16 / OUTB));
        if (vec_out && nvals == 16 / OUTB) {
          *reinterpret_cast<v4i*>(dst) = *reinterpret_cast<const v4i*>(src);
        } else {
          for (int e2 = 0; e2 < nvals; ++e2) {
            if constexpr (OUT_BF16)
              reinterpret_cast<uint16_t*>(dst)[e2] = reinterpret_cast<const uint16_t*>(src)[e2];
            else
              reinterpret_cast<float*>(dst)[e2] = reinterpret_cast<const float*>(src)[e2];
          }
        }
      }
    }
  }
}

template <Epi EPI, bool OUT_BF16, bool BIAS>
hipError_t launch_wide(const GemmProblem& p, hipStream_t st) {
  // n-blocks: the fewest blocks of at most 192 columns, equal widths rounded
  // up to 16
  const int64_t n_blocks = (p.N + GW_BN - 1) / GW_BN;
  const int64_t bn = ((p.N + n_blocks - 1) / n_blocks + 15) / 16 * 16;
  // at most ceil(M / 320) + E m-blocks (each expert adds at most one partial
  // block), dealt to the 8 XCDs in whole rounds
  const int64_t mblocks = (p.M + GW_MB - 1) / GW_MB + p.E;
  const int64_t grid = (mblocks + 7) / 8 * 8 * n_blocks;
  if (grid == 0) return hipSuccess;
  if (grid > int64_t(INT32_MAX)) return hipErrorInvalidValue;
  const int outb = OUT_BF16 ? 2 : 4;
  const int vec_out = ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0) && ((p.ldo * outb) % 16 == 0);
  // blockwise problems have K % 128 == 0 (checked by the caller)
  if (EPI == Epi::Block128x128 || p.K % BK == 0)
    hipLaunchKernelGGL((gemm_grouped_wide_kernel<EPI, OUT_BF16, BIAS, true>), dim3(unsigned(grid)), dim3(GW_NW * 64),
                       0, st, p, int(n_blocks), int(bn), vec_out);
  else if constexpr (EPI == Epi::Row)
    hipLaunchKernelGGL((gemm_grouped_wide_kernel<EPI, OUT_BF16, BIAS, false>), dim3(unsigned(grid)),
                       dim3(GW_NW * 64), 0, st, p, int(n_blocks), int(bn), vec_out);
  return hipGetLastError();
}

template <Epi EPI>
hipError_t launch_wide_out(const GemmProblem& p, hipStream_t st) {
  const bool bias = p.bias != nullptr;
  if (p.out_bf16) return bias ? launch_wide<EPI, true, true>(p, st) : launch_wide<EPI, true, false>(p, st);
  return bias ? launch_wide<EPI, false, true>(p, st) : launch_wide<EPI, false, false>(p, st);
}

}  // namespace

bool grouped_wide_applies(const GemmProblem& p) {
  // Weights stored [N, K], leading dimensions that the 128-byte row loads
  // need, and experts of at most 384 rows on average: below that the 320-row
  // m-blocks read each weight slice about once, above it the 256 x 256
  // streaming tiles (more arithmetic per loaded byte) are the better fit.
  return p.offsets && !p.group_k && !p.b_kn && (p.epi == Epi::Row || p.epi == Epi::Block128x128) &&
         p.lda >= 128 && p.ldb >= 128 && p.E > 0 && p.M <= 384 * p.E;
}

hipError_t launch_gemm_grouped_wide(const GemmProblem& p, hipStream_t st) {
  if (p.epi == Epi::Row) return launch_wide_out<Epi::Row>(p, st);
  if (p.epi == Epi::Block128x128) return launch_wide_out<Epi::Block128x128>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace fp8mm
