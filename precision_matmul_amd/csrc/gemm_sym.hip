// Streaming FP8 (E4M3) scaled GEMM for gfx950, B stored [N, K].
//
//   out[i, j] = sum_k A[i,k] sA(i,k) * B(j,k) sB(j,k)  (+ bias[j])
//
// Serves the forward (input @ weight.t()), input-gradient (B stored [K, N])
// and weight-gradient (grad_output.t() @ input, both operands stored
// token-contiguous) call forms of ColossalAI PR #6419 ("Fix: Handle
// LowLevelZeroPlugin with use_fp8=True", "Forward pass" / "Backward pass"),
// for the tensorwise, rowwise, 1x128 x 128x128 and 1x128 x 128x1 recipes of
// pytorch PR #164141 ("Add _scaled_mm_v2 API") and pytorch/ao PR #2784
// ("improve fp8 blockwise gemm perf"), and MXFP8 on the block-scaled MFMA.
// GROUPED runs the MoE form of pytorch/ao PR #4390 ("Add _grouped_mm
// dispatch handler to Float8Tensor": expert e's rows times its own weights),
// GROUPED_K the per-expert weight gradient (expert e's tokens as the
// contraction); both store their outputs non-temporally.
//
// Schedule.  A workgroup of 8 waves (two per SIMD) computes a 256 x 256
// output tile, each wave a 64 x 128 sub-tile: 4 x 8 fragments of
// v_mfma_f32_16x16x128_f8f6f4 (one instruction consumes one 128-wide K
// block, which is also the scaling block of the blockwise recipes).  Both
// waves of a SIMD issue matrix instructions all the time; a single wave
// cannot keep the matrix pipe busy on its own.  Within a K step a wave walks
// its 8 fragment columns; the 4 A fragments stay in registers and the B
// fragments stream through a two-entry ring, each read one column ahead.
// LDS reads, global -> LDS loads and the blockwise promotion are spread
// between the MFMAs, so no wave ever has a burst of them.
//
// Data movement.  A and B tiles go global -> LDS with direct-to-LDS buffer
// loads into a two-stage ring (2 x 66 KiB).  One workgroup barrier per K
// step, before fragment column 7: every wave has then finished reading the
// current stage (its last B fragment is read in column 6) and waited for its
// own loads of the next stage, so after the barrier the next stage is
// readable and the current one may be refilled.  The loads of step k+1 are
// issued as early as that allows, so they have most of a step to land: the A
// tile in column 7 of step k-1, the B tile and the scales in columns 0 and 1
// of step k.  Each wave loads 32 rows of A and 32 of B with one group of
// four 1 KiB loads (one M0 write per group).
//
// Grouped short tiles.  An expert's last m-tile of at most 128 rows keeps
// the loads, stages and barriers above but spreads its outputs over all 8
// waves (64 x 32 or 64 x 64 blocks, transposed operand order), since the
// 64 x 128 sub-tiles would leave most waves without rows.
//
// Fragment K order.  Lane l of an MFMA operand supplies 32 bytes that the
// instruction treats as k in [32 q, 32 q + 32), q = l / 16.  A and B only
// need the same k order, so each lane supplies the 16-byte chunks q and
// q + 4 of the 128-byte row; with chunk c of row r stored at slot
// c ^ ((r >> 1) & 7) these reads are close to conflict-free.
#include <type_traits>

#include "gemm_common.hpp"

namespace fp8mm {
namespace {

using namespace gk;

constexpr int SY_BM = 256;
constexpr int SY_BN = 256;
constexpr int SY_NW = 8;
constexpr int SY_A = SY_BM * BK;            // A codes of one stage
constexpr int SY_B = SY_BN * BK;            // B codes of one stage
constexpr int SY_SCALE = 1024;              // 256 fp32 scales (sA), or up to 256 (sB)
constexpr int SY_STAGE = SY_A + SY_B + 2 * SY_SCALE;
constexpr int SY_GCH = 4;                   // grouped: m-tiles per XCD chunk
constexpr int SY_TM = 64;                   // wave sub-tile
constexpr int SY_TN = 128;
constexpr int SY_FM = SY_TM / 16;
constexpr int SY_FN = SY_TN / 16;

__device__ __forceinline__ void sy_fence() { __builtin_amdgcn_sched_barrier(0); }

typedef int v2i __attribute__((ext_vector_type(2)));

// B stored [K, N]: LDS tile of 128 k-rows x 256 bytes; 16-byte chunk c of
// row k at slot c ^ kswz(k).  The eight rows of one transposing read (k,
// k + 1, .., k + 7 with the same 16-byte chunk) land in eight different
// slots, and rows 16 apart (another lane group) in different slot sets.
__device__ __forceinline__ float fac(float f, int) { return f; }
__device__ __forceinline__ float fac(const v4f& f, int e) { return f[e]; }

__device__ __forceinline__ int kswz(int k) { return (k & 7) | (((k >> 4) & 1) << 3); }
__device__ __forceinline__ int kn_off(int k, int n) { return k * 256 + (((n >> 4) ^ kswz(k)) << 4) + (n & 15); }

// GROUPED_K: the grouped weight gradient, E problems of M x N that contract
// over the experts' runs of 128 tokens (offsets along K).
template <Epi EPI, bool OUT_BF16, bool BIAS, bool K_ALIGNED, bool B_KN, bool GROUPED, bool GROUPED_K = false>
__global__ __launch_bounds__(SY_NW * 64, 1) void gemm_sym_kernel(GemmProblem p, int tiles_m, int tiles_n,
                                                                   int vec_out) {
  constexpr bool BLOCKWISE = EPI == Epi::Block128x128 || EPI == Epi::Block128x1;
  // Operand order of the MFMA: each 16 x 16 output block is computed
  // transposed (B fragment as the instruction's first operand), so a lane
  // holds one output row and four adjacent columns: one promotion factor per
  // lane and row fragment for a 128x128 B, and one row factor times four
  // column factors for a 128x1 B.
  // MXFP8: the MFMA applies the E8M0 byte of lane group g (for the lane's
  // row or column) to K [32 g, 32 g + 32) of the step, i.e. to chunks 2g and
  // 2g + 1, in the fragment order below.
  constexpr bool MX = EPI == Epi::MX;
  static_assert(!MX || (!B_KN && !GROUPED), "MXFP8: plain GEMMs with B stored [N, K]");
  static_assert(!GROUPED || EPI == Epi::Row || EPI == Epi::Block128x128, "grouped: rowwise or 1x128 x 128x128");
  static_assert(!GROUPED_K || (EPI == Epi::Block128x1 && !B_KN && !GROUPED && !BIAS), "grouped weight gradient");
  // promotion factor of one MFMA result: per lane (128x128) or per element (128x1)
  using Fac = std::conditional_t<EPI == Epi::Block128x1, v4f, float>;
  constexpr int OUTB = OUT_BF16 ? 2 : 4;
  constexpr int EPI_PASSES = epi_passes(SY_NW, SY_TM, SY_TN, OUTB, SY_STAGE);
  constexpr int EPI_COLS = SY_TN / EPI_PASSES;
  constexpr int EPI_PITCH = EPI_COLS * OUTB + 16;
  static_assert(EPI_PASSES <= 4 && SY_TN % EPI_PASSES == 0, "epilogue staging");
  static_assert(2 * SY_STAGE <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(1024))) uint8_t stage0[SY_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[SY_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---------------- tile ----------------
  // Grouped (MoE) problems: m-tiles g of all experts (in the order chosen
  // below) go to the 8 XCDs (workgroups are dealt to them round-robin, XCD =
  // b % 8) in chunks of SY_GCH consecutive m-tiles, chunk c to XCD c % 8; an
  // XCD walks its m-tiles in order, all n-tiles tn of one m-tile together.
  // So the n-tiles of one m-tile share its A rows in one XCD's L2, the
  // m-tiles of one expert (consecutive g) mostly share its B tiles there too,
  // and the real m-tiles (a prefix of the upper bound the grid is sized for)
  // are spread over all XCDs.
  // Expert e's B is [N, K] (or [K, N]) at B + e N K, its bias the [N] row
  // at bias + e bias_stride_e (one shared row, or row e of [E, N]), its
  // scales row e of [E, N] (rowwise) or grid e of [E, N/128 x K/128]
  // (128x128).
  int tn;
  int64_t row0;
  int rows_valid;
  const uint8_t* Ag = p.A;
  const uint8_t* Bg = p.B;
  const float* sag = p.sa;
  const float* sbg = p.sb;
  [[maybe_unused]] const uint16_t* biasg = p.bias;
  int K = int(p.K);
  int64_t out_off = 0;
  if constexpr (GROUPED_K) {
    // Expert e = lin / (tiles_m tiles_n): one expert's tiles are consecutive
    // in one XCD, whose L2 then holds that expert's operand columns: columns
    // [128 first, 128 (first + runs)) of the padded token axis, scale rows
    // [first, first + runs) of [runs, M] and [runs, N]; output problem e of
    // [E, M, N].
    const int64_t per_xcd = gridDim.x / 8;   // the launcher pads the grid to a multiple of 8
    const int64_t lin = int64_t(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const int64_t tiles = int64_t(tiles_m) * tiles_n;
    const int64_t e = lin / tiles;
    if (e >= p.E) return;
    const int t = int(lin - e * tiles);
    tn = t % tiles_n;
    int64_t first = 0;
    int runs = 0;
    grp::runs_before(p.offsets, p.tokens, 128, e, first, runs);
    // the operands and scales hold lda / 128 runs; offsets that are not
    // non-decreasing could ask for more, which are dropped
    const int64_t cap = p.lda / 128;
    first = min(first, cap);
    runs = int(min<int64_t>(runs, cap - first));
    row0 = int64_t(t / tiles_n) * SY_BM;
    rows_valid = int(min<int64_t>(SY_BM, p.M - row0));
    Ag = p.A + first * 128;
    Bg = p.B + first * 128;
    sag = p.sa + first * p.M;
    sbg = p.sb + first * p.N;
    K = runs * 128;
    out_off = e * p.M * p.ldo;
  } else if constexpr (GROUPED) {
    const int r = blockIdx.x / 8;              // slot within the XCD
    const int mt = r / tiles_n;                // the XCD's m-tile ordinal
    const int g = ((mt / SY_GCH) * 8 + int(blockIdx.x % 8)) * SY_GCH + mt % SY_GCH;
    tn = r % tiles_n;
    if (g >= tiles_m) return;
    int e = 0;
    int64_t rend = 0;
    // B stored [N, K]: m-tiles with more than 128 rows first, the short ones
    // last (grouped.hpp).  B stored [K, N]: expert order, so an expert's
    // short last m-tile runs beside its full ones and finds their B tiles
    // in L2 (measured 7 % faster there; the [N, K] form gains from the order
    // instead).
    if constexpr (B_KN) {
      if (!grp::find_run(p.offsets, p.E, p.M, SY_BM, g, e, row0, rend)) return;
    } else {
      if (!grp::find_mtile_long_first(p.offsets, p.E, p.M, g, e, row0, rend)) return;
    }
    rows_valid = int(min<int64_t>(SY_BM, rend - row0));
    Bg = p.B + int64_t(e) * p.N * p.K;
    sbg = p.sb + int64_t(e) * (EPI == Epi::Block128x128 ? (p.N / 128) * (p.K / 128) : p.N);
    if constexpr (BIAS) biasg = p.bias + int64_t(e) * p.bias_stride_e;
  } else {
    int tm;
    if (!tile_coords(tiles_m, tiles_n, tm, tn)) return;
    row0 = p.row_begin + int64_t(tm) * SY_BM;
    rows_valid = int(min<int64_t>(SY_BM, p.M - row0));
  }
  const int64_t n0 = int64_t(tn) * SY_BN;
  const int cols_valid = int(min<int64_t>(SY_BN, p.N - n0));
  const int nk = (K + BK - 1) / BK;

  // ---------------- loaders ----------------
  // Wave w fills tile rows [32 w, 32 w + 32) of A and of B with one group of
  // four loads each: load q covers rows 32 w + 8 q + l / 8 (lane l, 16 bytes
  // at slot l % 8, which holds chunk (l % 8) ^ swz(row) = (l % 8) ^
  // (((q & 1) << 2) | (l >> 4))), at LDS 1 KiB block 4 w + q.  The group's
  // instruction offsets add 1024 q to both addresses, so the per-lane offset
  // of load q is its row offset minus 1024 q (non-negative as ld >= 128).
  const int ld_row = lane >> 3;
  const int ch_even = (lane & 7) ^ (lane >> 4);
  const int ch_odd = (lane & 7) ^ (4 | (lane >> 4));
  const Rsrc rsA = make_rsrc4(Ag + row0 * p.lda, uint32_t(rows_valid) * uint32_t(p.lda));
  [[maybe_unused]] const Rsrc rsB = make_rsrc4(Bg + n0 * p.ldb, uint32_t(cols_valid) * uint32_t(p.ldb));
  const uint32_t rowA = uint32_t(wave * 32 + ld_row) * uint32_t(p.lda);
  const uint32_t rowB = uint32_t(wave * 32 + ld_row) * uint32_t(p.ldb);
  const uint32_t stepA = 8u * uint32_t(p.lda) - 1024u;   // per-q change of the per-lane offset
  const uint32_t stepB = 8u * uint32_t(p.ldb) - 1024u;
  const uint32_t lds0 = lds_addr(stage0), lds1 = lds_addr(stage1);

  // The group of A (or B) loads of K step kt into the stage at LDS address st;
  // steps past the end issue nothing.
  // B stored [K, N]: the B tile is 128 k-rows of 256 bytes (n); 16-byte chunk
  // c of row k sits at slot c ^ kswz(k).  Wave w fills rows [16 w, 16 w + 16):
  // load q rows 16 w + 4 q + l / 16, lane l slot l % 16 (one 1 KiB block, at
  // LDS block 4 w + q as for the [N, K] layout).  The per-step descriptor
  // starts at row k0 of the tile's columns and ends with the matrix, so rows
  // past K read zeros; columns past N read bytes of the next row (or zeros),
  // which only reach output columns that are never stored.
  [[maybe_unused]] const int kn_row = lane >> 4;
  [[maybe_unused]] const int kn_slot = lane & 15;
  auto load_group_kn = [&](int kt, uint32_t st) {
    if (kt >= nk) return;
    const int64_t k0 = int64_t(kt) * BK;
    const int64_t rem = (p.K - k0) * p.ldb - n0;
    const Rsrc r = make_rsrc4(Bg + k0 * p.ldb + n0, uint32_t(rem));
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = wave * 16 + q * 4 + kn_row;
      v[q] = uint32_t(row) * uint32_t(p.ldb) + uint32_t((kn_slot ^ kswz(row)) * 16) - uint32_t(q) * 1024u;
    }
    dma_b128x4(r, st + SY_A + wave * 4096, v[0], v[1], v[2], v[3], 0u);
  };
  auto load_group = [&](bool is_b, int kt, uint32_t st) {
    if constexpr (B_KN) {
      if (is_b) {
        load_group_kn(kt, st);
        return;
      }
    }
    if (kt >= nk) return;
    const uint32_t k0 = uint32_t(kt) * BK;
    const uint32_t rowv = is_b ? rowB : rowA;
    const uint32_t stp = is_b ? stepB : stepA;
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = (q & 1) ? ch_odd : ch_even;
      const bool in = K_ALIGNED || int(k0) + ch * 16 < K;
      v[q] = in ? rowv + uint32_t(ch * 16) + uint32_t(q) * stp : 0x80000000u;
    }
    dma_b128x4(is_b ? rsB : rsA, st + (is_b ? SY_A : 0) + wave * 4096, v[0], v[1], v[2], v[3], k0);
  };
  // Blockwise: scale chunk `wave` of K step kt (256 bytes, filled by this
  // wave's 64 lanes; lanes whose offset is out of range write zeros).  Waves
  // 0..3: sA[kt, row0 + 64 wave .. +64); waves 4..7 (128x1): sB[kt, n0 +
  // 64 (wave - 4) .. +64); waves 4, 5 (128x128): sB[n0/128 + wave - 4,
  // kt .. ] of which only the first element is used.  Each descriptor spans
  // to the end of the scale array, so rows or columns past the tile edge read
  // neighbouring scales that only reach outputs never stored, and no load is
  // partly out of range.
  [[maybe_unused]] const float* sc_base = nullptr;
  [[maybe_unused]] int64_t sc_count = 0;     // elements from sc_base to the array end
  [[maybe_unused]] int64_t sc_stride = 0;    // elements per K step
  if constexpr (BLOCKWISE) {
    if (wave < 4) {
      sc_base = sag + row0 + wave * 64;
      sc_count = int64_t(nk) * p.M - row0 - wave * 64;
      sc_stride = p.M;
    } else if constexpr (EPI == Epi::Block128x1) {
      sc_base = sbg + n0 + (wave - 4) * 64;
      sc_count = int64_t(nk) * p.N - n0 - (wave - 4) * 64;
      sc_stride = p.N;
    } else {
      // 128x128: sB[n0/128 + wave - 4, kt] (grid [N/128, K/128] for B stored
      // [N, K], [K/128, N/128] for B stored [K, N])
      const int64_t nb = n0 / 128 + (wave - 4);
      const bool in = wave < 6 && nb < p.N / 128;
      if constexpr (B_KN) {
        sc_base = sbg + (in ? nb : 0);
        sc_count = in ? int64_t(nk) * (p.N / 128) - nb : 0;
        sc_stride = p.N / 128;
      } else {
        sc_base = sbg + (in ? nb * nk : 0);
        sc_count = in ? nk : 0;
        sc_stride = 1;
      }
    }
  }
  [[maybe_unused]] auto load_scales = [&](int kt, uint32_t st) {
    if (kt >= nk) return;
    if constexpr (MX) {
      // E8M0 bytes of K step kt (4 per row / column): waves 0..3 rows
      // row0 + 64 wave + lane of A, waves 4..7 columns n0 + 64 (wave - 4) +
      // lane of B; lane l's 4 bytes land at 4 l of its wave's 256 bytes.
      // Rows / columns past the tile edge read zeros.
      const int64_t nkb = K / 32;                                 // bytes per row
      const int w4 = wave & 3;
      const int64_t first = (wave < 4 ? row0 : n0) + 64 * w4;
      const int valid = wave < 4 ? rows_valid : cols_valid;
      const int here = min(max(valid - 64 * w4, 0), 64);
      const uint8_t* base = (wave < 4 ? reinterpret_cast<const uint8_t*>(sag) : reinterpret_cast<const uint8_t*>(sbg)) +
                            (here > 0 ? first * nkb : 0);
      const Rsrc r = make_rsrc4(base, uint32_t(here) * uint32_t(nkb));
      dma_b32(r, st + SY_A + SY_B + (wave < 4 ? 0 : SY_SCALE) + w4 * 256,
              uint32_t(lane) * uint32_t(nkb) + uint32_t(kt) * 4u);
      return;
    }
    const int64_t off = int64_t(kt) * sc_stride;
    const int64_t rem = sc_count - off;
    const Rsrc r = make_rsrc4(sc_base + (rem > 0 ? off : 0), uint32_t(rem > 0 ? rem * 4 : 0));
    dma_b32(r, st + SY_A + SY_B + (wave < 4 ? wave * 256 : SY_SCALE + (wave - 4) * 256), uint32_t(lane) * 4u);
  };

  // ---------------- registers ----------------
  // Wave w < 4 takes rows [64 w, +64) of columns [0, 128); wave w >= 4 rows
  // [64 ((w + 2) & 3), +64) of columns [128, 256).  The SIMD of wave w is
  // w % 4, so the two waves of a SIMD share neither rows nor columns: a tile
  // with only its first 64 rows valid keeps two SIMDs busy (waves 0 and 6),
  // one with only its first 128 rows valid all four with one wave each
  // (waves 0, 1, 6, 7), one with only its first 128 columns valid all four
  // (waves 0-3).
  const int wm = wave < 4 ? wave : (wave + 2) & 3;
  const int wn = wave >> 2;
  const int row_base = wm * SY_TM;               // sub-tile origin within the tile
  const int col_base = wn * SY_TN;
  const bool active = row_base < rows_valid && col_base < cols_valid;   // wave-uniform
  const int frow = lane & 15;                    // fragment row (A) / column (B) of this lane
  const int fq = lane >> 4;                      // K quarter of this lane
  v4f acc[SY_FM][SY_FN];
#pragma unroll
  for (int i = 0; i < SY_FM; ++i)
#pragma unroll
    for (int j = 0; j < SY_FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto read_frag = [&](const uint8_t* tile, int r) {
    const v4i lo = *reinterpret_cast<const v4i*>(tile + lds_off(r, fq));
    const v4i hi = *reinterpret_cast<const v4i*>(tile + lds_off(r, fq + 4));
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // B stored [K, N]: the 16 x 128 fragment of columns [n0, n0 + 16) from four
  // transposing reads.  In each 16-lane group, lane 2 j + h points at the 8
  // bytes of row kb + j, columns n0 + 8 h .. +8; the read hands lane i the
  // bytes of column n0 + i in rows kb .. kb + 7 (lanes 0..7 from the even
  // lanes' rows, 8..15 from the odd lanes').  The four reads give lane l
  // (group q = l / 16) rows 16 q .. 16 q + 15 and 64 + 16 q .. +15: the same
  // chunks q and q + 4 that read_frag takes from an [N, K] tile.
  // The four rows of a lane differ by multiples of 8 in bits 3 and 6 only, so
  // they share kswz and sit at fixed distances; with nc a multiple of 16
  // below 256 the offset of (k, nc + 8 h) is kn_off(k, 8 h) ^ nc.
  [[maybe_unused]] const int kn_base = kn_off(fq * 16 + (frow >> 1), (frow & 1) * 8);
  [[maybe_unused]] auto read_frag_kn = [&](const uint8_t* tile, int nc) {
    const uint8_t* b = tile + (kn_base ^ nc);
    v2i r[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      r[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i*)(b + ((t >> 1) * 64 + (t & 1) * 8) * 256));
    return v8i{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
  };
  auto read_b = [&](const uint8_t* tile, int nc) {
    if constexpr (B_KN) return read_frag_kn(tile, nc);
    else return read_frag(tile, nc + frow);
  };
  auto stage_ptr = [&](int s) -> const uint8_t* { return s == 0 ? stage0 : stage1; };
  // Blockwise: per-lane scales of the 4 row fragments (sA of the lane's row
  // in each) and, for 128x128, the B block scale (folded into the row
  // factors in column 0 of the step that uses them).
  auto read_fa = [&](const uint8_t* st, float* fa_out, float* sbv_out) {
    const float* sas = reinterpret_cast<const float*>(st + SY_A + SY_B);
    const float* sbs = sas + SY_SCALE / 4;
#pragma unroll
    for (int i = 0; i < SY_FM; ++i) {
      fa_out[i] = sas[row_base + i * 16 + frow];
    }
    if constexpr (EPI == Epi::Block128x128) sbv_out[0] = sbs[(col_base / 128) * 64];
  };
  // 128x1: the four column factors of the lane's columns in fragment column
  // j of a stage
  [[maybe_unused]] auto read_colf = [&](const uint8_t* st, int j) {
    const float* sbs = reinterpret_cast<const float*>(st + SY_A + SY_B) + SY_SCALE / 4;
    return *reinterpret_cast<const v4f*>(sbs + col_base + j * 16 + fq * 4);
  };

  v8i a[SY_FM];
  v8i bring[2];
  // MXFP8: the lane's E8M0 byte for each A fragment (its row, K range
  // 32 fq) and for the B fragments of the ring (its column).
  [[maybe_unused]] int mxa[SY_FM];
  [[maybe_unused]] int mxb[2];
  [[maybe_unused]] auto mx_byte = [&](const uint8_t* stage, int region, int idx) {
    return int(stage[SY_A + SY_B + region + idx * 4 + fq]);
  };
  // Promotion factors of the current / next step.  128x1 keeps one set of
  // row factors: the next step's value of each replaces the current one
  // right after its last use in column 7; its column factors are read one
  // fragment column ahead into a ring of two (colf).
  constexpr int FSETS = EPI == Epi::Block128x1 ? 1 : 2;
  [[maybe_unused]] float fa[FSETS][SY_FM];
  [[maybe_unused]] float sbv[FSETS][1];
  [[maybe_unused]] v4f colf[2];
  // Blockwise promotion runs two MFMAs behind: pending results and where they go.
  [[maybe_unused]] v4f pend_t[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
  [[maybe_unused]] Fac pend_f[2] = {Fac{}, Fac{}};

  // ---------------- one K step ----------------
  // F selects the promotion-factor buffer of this step (steps alternate).
  auto step = [&](auto stage_c, auto fsel_c, int kt) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int F = decltype(fsel_c)::value;
    const uint8_t* As = stage_ptr(S);
    const uint8_t* Bs = As + SY_A;
    const uint8_t* An = stage_ptr(S ^ 1);
    const uint32_t this_st = S == 0 ? lds0 : lds1;
    const uint32_t next_st = S == 0 ? lds1 : lds0;
#pragma unroll
    for (int j = 0; j < SY_FN; ++j) {
      if (j == SY_FN - 1) {
        // Barrier: every wave has read the last B fragment of this stage (in
        // column 6) and its own loads of the next stage have landed.
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        sy_fence();
        asm volatile("s_barrier" ::: "memory");
        sy_fence();
      }
#pragma unroll
      for (int i = 0; i < SY_FM; ++i) {
        const int m = j * SY_FM + i;     // slot in the step
        const v8i& bf = bring[j & 1];
        if constexpr (MX) {
          acc[i][j] = mfma_16x16x128_mx(bf, a[i], acc[i][j], mxb[j & 1], mxa[i]);
          // Without this pin the compiler gathers the step's block-scaled
          // MFMAs and moves the fragment reads around them, keeping all
          // eight B fragments live (and spilling).
          asm volatile("" : "+v"(acc[i][j]));
        } else if constexpr (!BLOCKWISE) {
          acc[i][j] = mfma_16x16x128(bf, a[i], acc[i][j]);
        } else {
          const v4f t = mfma_16x16x128(bf, a[i], v4f{0.f, 0.f, 0.f, 0.f});
          // promote the result of slot m - 2 (possibly of the previous step)
          {
            const int mp = m - 2;
            const int ip = (mp + 32) % 32 % SY_FM;
            const int jp = (mp + 32) % 32 / SY_FM;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[ip][jp][e] = __builtin_fmaf(pend_t[m & 1][e], fac(pend_f[m & 1], e), acc[ip][jp][e]);
            asm volatile("" ::"v"(acc[ip][jp]));
          }
          pend_t[m & 1] = t;
          if constexpr (EPI == Epi::Block128x128) {
            if (j == 0) fa[F % FSETS][i] = fa[F % FSETS][i] * sbv[F % FSETS][0];
            pend_f[m & 1] = fa[F % FSETS][i];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) pend_f[m & 1][e] = fa[F % FSETS][i] * colf[j & 1][e];
          }
        }
        if constexpr (BLOCKWISE) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
        sy_fence();
        // ---- work between MFMAs ----
        // B fragment of the next column (column 7: column 0 of the next step)
        if (i == 0) {
          if (j + 1 < SY_FN) {
            bring[(j + 1) & 1] = read_b(Bs, col_base + (j + 1) * 16);
            if constexpr (MX) mxb[(j + 1) & 1] = mx_byte(As, SY_SCALE, col_base + (j + 1) * 16 + frow);
            if constexpr (EPI == Epi::Block128x1) colf[(j + 1) & 1] = read_colf(As, j + 1);
          } else {
            bring[0] = read_b(An + SY_A, col_base);
            if constexpr (MX) mxb[0] = mx_byte(An, SY_SCALE, col_base + frow);
            if constexpr (EPI == Epi::Block128x1) colf[0] = read_colf(An, 0);
          }
        }
        // next step's A fragment i, right after its last use
        if (j == SY_FN - 1) {
          a[i] = read_frag(An, row_base + i * 16 + frow);
          if constexpr (MX) mxa[i] = mx_byte(An, 0, row_base + i * 16 + frow);
        }
        // next step's promotion factors
        if constexpr (BLOCKWISE) {
          if constexpr (FSETS == 2) {
            if (j == SY_FN - 1 && i == 1) read_fa(An, fa[F ^ 1], sbv[F ^ 1]);
          } else if (j == SY_FN - 1) {
            // 128x1, one set: row factor i after its last use (slot 7, i)
            fa[0][i] = reinterpret_cast<const float*>(An + SY_A + SY_B)[row_base + i * 16 + frow];
          }
        }
        // loads: A of step kt+2 into this stage (free after the barrier) in
        // column 7; B and the scales of step kt+1 into the other stage in
        // columns 0 and 1
        if (j == SY_FN - 1 && i == 0) load_group(false, kt + 2, this_st);
        if (j == 0 && i == 1) load_group(true, kt + 1, next_st);
        if constexpr (BLOCKWISE || MX) {
          if (j == 1 && i == 1) load_scales(kt + 1, next_st);
        }
        sy_fence();
      }
    }
  };

  // Grouped short tile: K loop and stores, entered with stage 0 complete and
  // visible.  FNS = 2 (at most 64 rows): wave w takes the 64 x 32 block at
  // rows [0, 64), columns [32 w, 32 w + 32).  FNS = 4 (at most 128 rows):
  // the 64 x 64 block at rows [64 (w & 1), +64), columns [64 (w >> 1), +64),
  // so the two waves of a SIMD (w, w + 4) share rows but not columns.
  [[maybe_unused]] auto short_tile = [&](auto fns_c) {
    constexpr int FNS = decltype(fns_c)::value;
    const int rb = FNS == 2 ? 0 : (wave & 1) * 64;           // the wave's first row in the tile
    const int cb = FNS == 2 ? wave * 32 : (wave >> 1) * 64;  // its first column
    const bool cact = rb < rows_valid && cb < cols_valid;    // wave-uniform
    v4f sacc[SY_FM][FNS];
#pragma unroll
    for (int i = 0; i < SY_FM; ++i)
#pragma unroll
      for (int j = 0; j < FNS; ++j) sacc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    load_group(false, 1, lds1);
    for (int kt = 0; kt < nk; ++kt) {
      const uint32_t this_st = (kt & 1) ? lds1 : lds0;
      const uint32_t next_st = (kt & 1) ? lds0 : lds1;
      const uint8_t* St = (kt & 1) ? stage1 : stage0;
      load_group(true, kt + 1, next_st);
      if constexpr (BLOCKWISE) load_scales(kt + 1, next_st);
      if (cact) {
        v8i fa_s[SY_FM], fb_s[FNS];
#pragma unroll
        for (int i = 0; i < SY_FM; ++i) fa_s[i] = read_frag(St, rb + i * 16 + frow);
#pragma unroll
        for (int j = 0; j < FNS; ++j) fb_s[j] = read_b(St + SY_A, cb + j * 16);
        if constexpr (BLOCKWISE) {
          // 1x128 x 128x128: the step's partial times sA(row) sB(block)
          const float* sas = reinterpret_cast<const float*>(St + SY_A + SY_B);
          const float sbk = sas[SY_SCALE / 4 + (cb / 128) * 64];
#pragma unroll
          for (int i = 0; i < SY_FM; ++i) {
            const float f = sas[rb + i * 16 + frow] * sbk;
#pragma unroll
            for (int j = 0; j < FNS; ++j) {
              const v4f t = mfma_16x16x128(fb_s[j], fa_s[i], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int e = 0; e < 4; ++e) sacc[i][j][e] = __builtin_fmaf(t[e], f, sacc[i][j][e]);
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < SY_FM; ++i)
#pragma unroll
            for (int j = 0; j < FNS; ++j) sacc[i][j] = mfma_16x16x128(fb_s[j], fa_s[i], sacc[i][j]);
        }
      }
      // every wave has read this stage and its loads of the next have landed
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      sy_fence();
      asm volatile("s_barrier" ::: "memory");
      sy_fence();
      load_group(false, kt + 2, this_st);
    }
    if (!cact) return;
    // stores: 4 adjacent columns per lane and fragment, one 8- or 16-byte
    // non-temporal store where they are all inside the tile
#pragma unroll
    for (int i = 0; i < SY_FM; ++i) {
      const int r = rb + i * 16 + frow;
      if (r >= rows_valid) continue;
      [[maybe_unused]] float sr = 1.f;
      if constexpr (EPI == Epi::Row) sr = p.sa[row0 + r];
      uint8_t* orow = reinterpret_cast<uint8_t*>(p.out) + (out_off + (row0 + r) * p.ldo + n0) * OUTB;
#pragma unroll
      for (int j = 0; j < FNS; ++j) {
        const int c = cb + j * 16 + fq * 4;
        if (c >= cols_valid) continue;
        const int n = min(4, cols_valid - c);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = sacc[i][j][e];
          if (e < n) {
            if constexpr (EPI == Epi::Row) v[e] = (v[e] * sr) * sbg[n0 + c + e];
            if constexpr (BIAS) v[e] = v[e] + __uint_as_float(uint32_t(biasg[n0 + c + e]) << 16);
          }
        }
        uint8_t* dst = orow + c * OUTB;
        if (vec_out && n == 4) {
          if constexpr (OUT_BF16) {
            const v2i w{int(uint32_t(f32_to_bf16_rne(v[0])) | (uint32_t(f32_to_bf16_rne(v[1])) << 16)),
                        int(uint32_t(f32_to_bf16_rne(v[2])) | (uint32_t(f32_to_bf16_rne(v[3])) << 16))};
            __builtin_nontemporal_store(w, reinterpret_cast<v2i*>(dst));
          } else {
            __builtin_nontemporal_store(v4f{v[0], v[1], v[2], v[3]}, reinterpret_cast<v4f*>(dst));
          }
        } else {
          for (int e = 0; e < n; ++e) {
            if constexpr (OUT_BF16)
              reinterpret_cast<uint16_t*>(dst)[e] = f32_to_bf16_rne(v[e]);
            else
              reinterpret_cast<float*>(dst)[e] = v[e];
          }
        }
      }
    }
  };

  if (nk > 0) {
    // Prologue: stage 0 complete and visible; the fragments and factors of
    // step 0 in registers; the first loads of step 1 in flight.
    load_group(false, 0, lds0);
    load_group(true, 0, lds0);
    if constexpr (BLOCKWISE || MX) load_scales(0, lds0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if constexpr (GROUPED) {
      // An expert's last m-tile with at most 128 rows (the remainder past its
      // full tiles).  In the layout above at most four waves would have rows
      // to compute, two of them on one SIMD; here all 8 do, in the
      // transposed operand order (lane: row 16 i + frow, columns 16 j + 4 fq
      // + e).  Loads, stages and the one barrier per K step are those of the
      // full tile.
      const int rv = __builtin_amdgcn_readfirstlane(rows_valid);
      if (rv <= SY_TM) {
        short_tile(std::integral_constant<int, 2>{});
        return;
      }
      if (rv <= 2 * SY_TM) {
        short_tile(std::integral_constant<int, 4>{});
        return;
      }
    }
    if (active) {
#pragma unroll
      for (int i = 0; i < SY_FM; ++i) a[i] = read_frag(stage0, row_base + i * 16 + frow);
      bring[0] = read_b(stage0 + SY_A, col_base);
      if constexpr (BLOCKWISE) read_fa(stage0, fa[0], sbv[0]);
      if constexpr (EPI == Epi::Block128x1) colf[0] = read_colf(stage0, 0);
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < SY_FM; ++i) mxa[i] = mx_byte(stage0, 0, row_base + i * 16 + frow);
        mxb[0] = mx_byte(stage0, SY_SCALE, col_base + frow);
      }
      load_group(false, 1, lds1);
      for (int kt = 0; kt < nk; kt += 2) {
        step(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, kt);
        if (kt + 1 < nk) step(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}, kt + 1);
      }
    } else {
      // Every row or every column of this wave's sub-tile is past the tile's
      // valid ones (an expert's last m-tile, the M or N edge): no fragments
      // and no MFMAs, only this wave's share of the loads, in the same order
      // and under the same one barrier per K step as the computing waves.
      load_group(false, 1, lds1);
      for (int kt = 0; kt < nk; ++kt) {
        const uint32_t this_st = (kt & 1) ? lds1 : lds0;
        const uint32_t next_st = (kt & 1) ? lds0 : lds1;
        load_group(true, kt + 1, next_st);
        if constexpr (BLOCKWISE || MX) load_scales(kt + 1, next_st);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        sy_fence();
        asm volatile("s_barrier" ::: "memory");
        sy_fence();
        load_group(false, kt + 2, this_st);
      }
    }
    if (BLOCKWISE && active) {
      // the last two results of the last step
#pragma unroll
      for (int mm = 30; mm < 32; ++mm) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[mm % SY_FM][mm / SY_FM][e] = __builtin_fmaf(pend_t[mm & 1][e], fac(pend_f[mm & 1], e), acc[mm % SY_FM][mm / SY_FM][e]);
      }
    }
  }

  // ---------------- epilogue: scale, round, stage in LDS, 16-byte stores ----------------
  // The epilogue's scale and bias loads are all issued first, so their
  // latency overlaps the wait for the last loads and each other.
  [[maybe_unused]] float s_tensor = 0.f;
  if constexpr (EPI == Epi::Tensor) s_tensor = p.sa[0] * p.sb[0];
  // Row scale of the lane's row in each row fragment (i * 16 + frow).
  [[maybe_unused]] float sar[SY_FM];
  if constexpr (EPI == Epi::Row) {
#pragma unroll
    for (int i = 0; i < SY_FM; ++i) {
      const int rt = row_base + i * 16 + frow;
      sar[i] = rt < rows_valid ? p.sa[row0 + rt] : 0.f;
    }
  }
  // Column scales and bias of the lane's four adjacent output columns per
  // column fragment j (4 fq + e): one 16-byte scale load and one 8-byte bias
  // load per column fragment where alignment and the N edge allow.
  [[maybe_unused]] float sbc[SY_FN][4];
  [[maybe_unused]] float bias_v[SY_FN][4];
  [[maybe_unused]] const bool sb_vec = (reinterpret_cast<uintptr_t>(sbg) & 15) == 0;
  [[maybe_unused]] const bool bias_vec = (reinterpret_cast<uintptr_t>(biasg) & 7) == 0;
#pragma unroll
  for (int j = 0; j < SY_FN; ++j) {
    const int c0 = col_base + j * 16 + fq * 4;
    const bool whole = c0 + 4 <= cols_valid;
    if constexpr (EPI == Epi::Row) {
      if (sb_vec && whole) {
        const v4f t = *reinterpret_cast<const v4f*>(sbg + n0 + c0);
#pragma unroll
        for (int e = 0; e < 4; ++e) sbc[j][e] = t[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) sbc[j][e] = c0 + e < cols_valid ? sbg[n0 + c0 + e] : 0.f;
      }
    }
    if constexpr (BIAS) {
      if (bias_vec && whole) {
        const uint2 t = *reinterpret_cast<const uint2*>(biasg + n0 + c0);
        bias_v[j][0] = __uint_as_float(t.x << 16);
        bias_v[j][1] = __uint_as_float(t.x & 0xFFFF0000u);
        bias_v[j][2] = __uint_as_float(t.y << 16);
        bias_v[j][3] = __uint_as_float(t.y & 0xFFFF0000u);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bias_v[j][e] = c0 + e < cols_valid ? __uint_as_float(uint32_t(biasg[n0 + c0 + e]) << 16) : 0.f;
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  uint8_t* ep = (wave < SY_NW / 2 ? stage0 : stage1) + (wave % (SY_NW / 2)) * SY_TM * EPI_PITCH;
#pragma unroll
  for (int pass = 0; pass < EPI_PASSES; ++pass) {
    constexpr int FNP = SY_FN / EPI_PASSES;
#pragma unroll
    for (int jj = 0; jj < FNP; ++jj) {
      const int j = pass * FNP + jj;
#pragma unroll
      for (int i = 0; i < SY_FM; ++i) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[i][j][e];
          if constexpr (EPI == Epi::Tensor) v[e] = v[e] * s_tensor;
          if constexpr (EPI == Epi::Row) v[e] = (v[e] * sar[i]) * sbc[j][e];
          if constexpr (BIAS) v[e] = v[e] + bias_v[j][e];
        }
        uint8_t* dst = ep + (i * 16 + frow) * EPI_PITCH + (jj * 16 + fq * 4) * OUTB;
        if constexpr (OUT_BF16) {
          const uint32_t lo = uint32_t(f32_to_bf16_rne(v[0])) | (uint32_t(f32_to_bf16_rne(v[1])) << 16);
          const uint32_t hi = uint32_t(f32_to_bf16_rne(v[2])) | (uint32_t(f32_to_bf16_rne(v[3])) << 16);
          *reinterpret_cast<uint2*>(dst) = uint2{lo, hi};
        } else {
          *reinterpret_cast<v4f*>(dst) = v4f{v[0], v[1], v[2], v[3]};
        }
      }
    }
    __syncthreads();
    constexpr int CPR = EPI_COLS * OUTB / 16;
    constexpr int EPR = 16 / OUTB;
    constexpr int ITER = SY_TM * CPR / 64;    // 16-byte copies per lane and pass
    static_assert(ITER % 4 == 0, "copy-out batches");
    if (vec_out && row_base + SY_TM <= rows_valid && col_base + SY_TN <= cols_valid) {
      // The wave's whole sub-tile is inside the output: no per-chunk
      // conditions, so each lane has four LDS reads in flight before their
      // stores (one at a time, every copy waited out the LDS latency).
      uint8_t* const obase = reinterpret_cast<uint8_t*>(p.out) +
                             (out_off + (row0 + row_base) * p.ldo + n0 + col_base + pass * EPI_COLS) * OUTB;
#pragma unroll
      for (int u0 = 0; u0 < ITER; u0 += 4) {
        v4i val[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int idx = lane + (u0 + u) * 64;
          val[u] = *reinterpret_cast<const v4i*>(ep + (idx / CPR) * EPI_PITCH + (idx % CPR) * 16);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int idx = lane + (u0 + u) * 64;
          uint8_t* dst = obase + int64_t(idx / CPR) * p.ldo * OUTB + (idx % CPR) * 16;
          if constexpr (GROUPED || GROUPED_K)
            __builtin_nontemporal_store(val[u], reinterpret_cast<v4i*>(dst));
          else
            *reinterpret_cast<v4i*>(dst) = val[u];
        }
      }
      if (pass + 1 < EPI_PASSES) __syncthreads();
      continue;
    }
#pragma unroll 4
    for (int idx = lane; idx < SY_TM * CPR; idx += 64) {
      const int rl = idx / CPR;
      const int ch = idx % CPR;
      const int rt = row_base + rl;
      const int ct = col_base + pass * EPI_COLS + ch * EPR;
      if (rt >= rows_valid || ct >= cols_valid) continue;
      const uint8_t* src = ep + rl * EPI_PITCH + ch * 16;
      uint8_t* dst = reinterpret_cast<uint8_t*>(p.out) + (out_off + (row0 + rt) * p.ldo + n0 + ct) * OUTB;
      if (vec_out && ct + EPR <= cols_valid) {
        // Grouped outputs: non-temporal stores, measured 3-15 % faster there
        // (no gain measured on the dense GEMMs, which keep plain stores)
        if constexpr (GROUPED || GROUPED_K)
          __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(src), reinterpret_cast<v4i*>(dst));
        else
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        const int n = min(EPR, cols_valid - ct);
        for (int e = 0; e < n; ++e) {
          if constexpr (OUT_BF16)
            reinterpret_cast<uint16_t*>(dst)[e] = reinterpret_cast<const uint16_t*>(src)[e];
          else
            reinterpret_cast<float*>(dst)[e] = reinterpret_cast<const float*>(src)[e];
        }
      }
    }
    if (pass + 1 < EPI_PASSES) __syncthreads();
  }
}

template <Epi EPI, bool OUT_BF16, bool BIAS, bool B_KN, bool GROUPED>
hipError_t launch_sym(const GemmProblem& p, hipStream_t st) {
  // grouped: an upper bound on the experts' m-tiles (each expert adds at most
  // one partial tile); workgroups past the last real tile exit at once
  const int tiles_m = GROUPED ? int((p.M + SY_BM - 1) / SY_BM + p.E)
                              : int((p.row_end - p.row_begin + SY_BM - 1) / SY_BM);
  const int tiles_n = int((p.N + SY_BN - 1) / SY_BN);
  const int64_t tiles = int64_t(tiles_m) * tiles_n;
  if (tiles == 0) return hipSuccess;
  // grouped: whole rounds of 8 chunks of SY_GCH m-tiles (see the tile order
  // in the kernel)
  const int grid = GROUPED ? int((tiles_m + 8 * SY_GCH - 1) / (8 * SY_GCH) * (8 * SY_GCH) * tiles_n)
                           : int((tiles + 7) / 8 * 8);
  const int outb = OUT_BF16 ? 2 : 4;
  const int vec_out = ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0) && ((p.ldo * outb) % 16 == 0);
  // blockwise and MXFP8 problems have K % 128 == 0 (checked by the caller)
  constexpr bool BLOCKWISE = EPI == Epi::Block128x128 || EPI == Epi::Block128x1 || EPI == Epi::MX;
  if (BLOCKWISE || p.K % BK == 0)
    hipLaunchKernelGGL((gemm_sym_kernel<EPI, OUT_BF16, BIAS, true, B_KN, GROUPED>), dim3(grid), dim3(SY_NW * 64), 0, st,
                       p, tiles_m, tiles_n, vec_out);
  else if constexpr (!BLOCKWISE)
    hipLaunchKernelGGL((gemm_sym_kernel<EPI, OUT_BF16, BIAS, false, B_KN, GROUPED>), dim3(grid), dim3(SY_NW * 64), 0,
                       st, p, tiles_m, tiles_n, vec_out);
  return hipGetLastError();
}

template <Epi EPI>
hipError_t launch_sym_out(const GemmProblem& p, hipStream_t st) {
  const bool bias = p.bias != nullptr;
  if constexpr (EPI == Epi::Row || EPI == Epi::Block128x128) {
    if (p.offsets) {
      if (p.b_kn) {
        if (p.out_bf16)
          return bias ? launch_sym<EPI, true, true, true, true>(p, st) : launch_sym<EPI, true, false, true, true>(p, st);
        return bias ? launch_sym<EPI, false, true, true, true>(p, st) : launch_sym<EPI, false, false, true, true>(p, st);
      }
      if (p.out_bf16)
        return bias ? launch_sym<EPI, true, true, false, true>(p, st) : launch_sym<EPI, true, false, false, true>(p, st);
      return bias ? launch_sym<EPI, false, true, false, true>(p, st) : launch_sym<EPI, false, false, false, true>(p, st);
    }
  }
  if (p.offsets) return hipErrorInvalidValue;
  if constexpr (EPI != Epi::MX) {
    if (p.b_kn) {
      if (p.out_bf16)
        return bias ? launch_sym<EPI, true, true, true, false>(p, st) : launch_sym<EPI, true, false, true, false>(p, st);
      return bias ? launch_sym<EPI, false, true, true, false>(p, st) : launch_sym<EPI, false, false, true, false>(p, st);
    }
  }
  if (p.out_bf16)
    return bias ? launch_sym<EPI, true, true, false, false>(p, st) : launch_sym<EPI, true, false, false, false>(p, st);
  return bias ? launch_sym<EPI, false, true, false, false>(p, st) : launch_sym<EPI, false, false, false, false>(p, st);
}

// The grouped weight gradient on 256 x 256 tiles: grid E x tiles, padded to
// a multiple of 8.
template <bool OUT_BF16>
hipError_t launch_sym_group_k(const GemmProblem& p, hipStream_t st) {
  const int tiles_m = int((p.M + SY_BM - 1) / SY_BM), tiles_n = int((p.N + SY_BN - 1) / SY_BN);
  const int64_t total = int64_t(tiles_m) * tiles_n * p.E;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 7) / 8 * 8;
  if (grid > int64_t(INT32_MAX)) return hipErrorInvalidValue;
  const int outb = OUT_BF16 ? 2 : 4;
  const int vec_out = ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0) && ((p.ldo * outb) % 16 == 0);
  hipLaunchKernelGGL((gemm_sym_kernel<Epi::Block128x1, OUT_BF16, false, true, false, false, true>),
                     dim3(unsigned(grid)), dim3(SY_NW * 64), 0, st, p, tiles_m, tiles_n, vec_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_group_k_streaming(const GemmProblem& p, hipStream_t st) {
  return p.out_bf16 ? launch_sym_group_k<true>(p, st) : launch_sym_group_k<false>(p, st);
}

// Streaming schedule: plain GEMMs (B stored [N, K] or [K, N]) and grouped
// rowwise or 1x128 x 128x128 GEMMs (expert weights [E, N, K] or [E, K, N]).
hipError_t launch_gemm_streaming(const GemmProblem& p, hipStream_t st) {
  switch (p.epi) {
    case Epi::Tensor: return launch_sym_out<Epi::Tensor>(p, st);
    case Epi::Row: return launch_sym_out<Epi::Row>(p, st);
    case Epi::Block128x128: return launch_sym_out<Epi::Block128x128>(p, st);
    case Epi::Block128x1: return launch_sym_out<Epi::Block128x1>(p, st);
    case Epi::MX: return p.b_kn ? hipErrorInvalidValue : launch_sym_out<Epi::MX>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fp8mm
