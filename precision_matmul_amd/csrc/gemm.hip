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
// This file holds the general tile kernel; it serves B stored [K, N]
// (grad_output @ weight), the grouped (MoE) GEMM and plain GEMMs whose
// leading dimensions are below 128 bytes.  Plain GEMMs with B stored [N, K]
// go to the streaming kernel of gemm_sym.hip.
//
// Design (MI355X first):
//  * A workgroup of WM x WN waves computes a BM x BN output tile; each wave a
//    TM x TN sub-tile made of 16x16 fragments.  The K loop walks 128-byte
//    steps: one v_mfma_f32_16x16x128_f8f6f4 consumes exactly one 128-wide K
//    block, which is also the scaling block of the blockwise recipes.
//  * A and B (B stored [N, K]) are staged global -> LDS with direct-to-LDS
//    buffer loads (no VGPR round trip) into a 2- or 3-stage ring, one barrier
//    per K step.  LDS rows are 128 bytes; 16-byte chunk c of row r sits at
//    slot c ^ ((r >> 1) & 7).  Buffer descriptors clip the ragged M / N / K
//    edges to zero.
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
#include <type_traits>

#include "gemm_common.hpp"

#include <algorithm>
#include <atomic>

namespace fp8mm {
namespace {

using namespace gk;


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

// GROUPED_K: the grouped weight gradient, E problems of M x N that contract
// over the experts' runs of 128 tokens (offsets along K); two workgroups per
// CU, so that one's epilogue overlaps the other's loads.
template <int BM, int BN, int WM, int WN, int STAGES, Epi EPI, bool B_KN, bool OUT_BF16, bool BIAS, bool GROUPED,
          bool K_ALIGNED, bool GROUPED_K = false>
__global__ __launch_bounds__(WM * WN * 64, GROUPED_K ? 2 : 1) void gemm_kernel(GemmProblem p, int tiles_m, int tiles_n,
                                                                              int vec_out) {
  constexpr int NW = WM * WN;            // waves: WM along M x WN along N
  constexpr int NT = NW * 64;
  constexpr int TM = BM / WM;
  constexpr int TN = BN / WN;
  constexpr int FM = TM / 16;
  constexpr int FN = TN / 16;
  constexpr int D = STAGES - 1;          // prefetch distance in K steps
  constexpr bool BLOCKWISE = EPI == Epi::Block128x128 || EPI == Epi::Block128x1;
  // MXFP8: E8M0 bytes per 32 K, 4 per row / column per K step, loaded like
  // the blockwise scales and applied by the block-scaled MFMA.
  constexpr bool MX = EPI == Epi::MX;
  static_assert(!MX || (!B_KN && !GROUPED), "MXFP8: plain GEMMs with B stored [N, K]");
  static_assert(!GROUPED || EPI == Epi::Row || EPI == Epi::Block128x128, "grouped: rowwise or 1x128 x 128x128");
  static_assert(!GROUPED_K || (EPI == Epi::Block128x1 && !B_KN && !GROUPED && !BIAS), "grouped weight gradient");
  constexpr int A_BYTES = BM * BK;
  constexpr int B_BYTES = BN * BK;
  // Scale regions (blockwise): 8 chunks of 256 bytes, 4 for sA (BM = 256
  // rows) and 4 for sB (128x1: up to 256 column scales; 128x128: one block
  // scale per 128 columns, at the start of its chunk).  Each chunk is filled
  // by one wave's 64 lanes: a lane whose DMA offset is out of range still
  // writes (zeros) to its LDS slot, so a wave must own its whole chunk.
  constexpr int SA_BYTES = BLOCKWISE || MX ? 1024 : 0;
  constexpr int SB_BYTES = BLOCKWISE || MX ? 1024 : 0;
  constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
  constexpr int OUTB = OUT_BF16 ? 2 : 4;
  constexpr int EPI_PASSES = epi_passes(NW, TM, TN, OUTB, STAGE);
  constexpr int EPI_COLS = TN / EPI_PASSES;
  constexpr int EPI_PITCH = EPI_COLS * OUTB + 16;    // padded row pitch
  // loads per wave per K step (identical for every wave, so that one vmcnt
  // immediate tracks the ring)
  constexpr int LA = BM / (8 * NW);
  constexpr int LB = B_KN ? 0 : BN / (8 * NW);
  constexpr int NCH = BN / 16;                       // KN loader: 16-byte chunks per k row
  constexpr int KR = B_KN ? BK * NCH / NT : 1;       // KN loader: k rows per thread
  constexpr int LKN = B_KN ? KR : 0;
  constexpr int LS = BLOCKWISE || MX ? 8 / NW : 0;
  constexpr int LPS = LA + LB + LKN + LS;
  static_assert((NW == 4 || NW == 8) && NW % 2 == 0, "4 or 8 waves");
  static_assert(STAGES == 2 || STAGES == 3, "2 or 3 stages");
  static_assert(TM % 16 == 0 && TN % 16 == 0 && LA >= 1 && (B_KN || LB >= 1), "tile shape");
  static_assert(!BLOCKWISE || ((BM == 128 || BM == 256) && BN % 128 == 0 && 128 % TN == 0), "blockwise tile shape");
  static_assert(!B_KN || KR == 4 || KR == 8, "KN loader shape");
  static_assert(STAGES * STAGE <= 160 * 1024, "LDS budget");
  static_assert(EPI_PASSES <= 4 && TN % EPI_PASSES == 0, "epilogue staging");
  // One LDS array per stage: with every stage index a compile-time constant,
  // reads of the current stage and DMA into the prefetch stage are visibly
  // distinct.
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[STAGES > 2 ? STAGE : 16];
  auto stage_ptr = [&](int s) -> uint8_t* { return s == 0 ? stage0 : (s == 1 ? stage1 : stage2); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---------------- tile selection ----------------
  TileInfo ti;
  ti.sa = p.sa;
  ti.K = int(p.K);
  ti.out_off = 0;
  if constexpr (GROUPED_K) {
    // Expert e = lin / (tiles_m tiles_n): one expert's tiles are consecutive
    // in one XCD, whose L2 then holds that expert's operand columns.  Its
    // operands are the columns [128 first, 128 (first + runs)) of the padded
    // token axis, its scales rows [first, first + runs) of [runs, M] and
    // [runs, N], its output problem e of [E, M, N].
    const int64_t per_xcd = gridDim.x / 8;   // the launcher pads the grid to a multiple of 8
    const int64_t lin = int64_t(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const int64_t tiles = int64_t(tiles_m) * tiles_n;
    const int64_t e = lin / tiles;
    if (e >= p.E) return;
    const int t = int(lin - e * tiles);
    const int tm = t / tiles_n, tn = t % tiles_n;
    int64_t first = 0;
    int runs = 0;
    grp::runs_before(p.offsets, p.tokens, 128, e, first, runs);
    // the operands and scales hold lda / 128 runs; offsets that are not
    // non-decreasing could ask for more, which are dropped
    const int64_t cap = p.lda / 128;
    first = min(first, cap);
    runs = int(min<int64_t>(runs, cap - first));
    ti.row0 = int64_t(tm) * BM;
    ti.rows_valid = int(min<int64_t>(BM, p.M - ti.row0));
    ti.n0 = int64_t(tn) * BN;
    ti.cols_valid = int(min<int64_t>(BN, p.N - ti.n0));
    ti.A = p.A + ti.row0 * p.lda + first * 128;
    ti.B = p.B + ti.n0 * p.ldb + first * 128;
    ti.sa = p.sa + first * p.M;
    ti.sb = p.sb + first * p.N;
    ti.bias = nullptr;
    ti.K = runs * 128;
    ti.out_off = e * p.M * p.ldo;
  } else if constexpr (!GROUPED) {
    int tm, tn;
    if (!tile_coords(tiles_m, tiles_n, tm, tn)) return;
    ti.row0 = p.row_begin + int64_t(tm) * BM;
    ti.rows_valid = int(min<int64_t>(BM, p.M - ti.row0));
    ti.n0 = int64_t(tn) * BN;
    ti.cols_valid = int(min<int64_t>(BN, p.N - ti.n0));
    ti.A = p.A + ti.row0 * p.lda;
    ti.B = B_KN ? p.B + ti.n0 : p.B + ti.n0 * p.ldb;
    ti.sb = p.sb;
    ti.bias = p.bias;
  } else {
    // lin = tn * tiles_m + g: the m-tiles of one expert are adjacent.
    const int per_xcd = gridDim.x / 8;   // the launcher pads the grid to a multiple of 8
    const int lin = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const int tn = lin / tiles_m;
    const int g = lin % tiles_m;
    if (tn >= tiles_n) return;
    int e_found = 0;
    int64_t end_found = 0;
    if (!grouped_mtile(p, BM, g, e_found, ti.row0, end_found)) return;
    ti.rows_valid = int(min<int64_t>(BM, end_found - ti.row0));
    ti.n0 = int64_t(tn) * BN;
    ti.cols_valid = int(min<int64_t>(BN, p.N - ti.n0));
    ti.A = p.A + ti.row0 * p.lda;
    // expert e: B [N, K] or [K, N] at B + e N K; scales row e of [E, N]
    // (rowwise) or grid e of [E, N/128 x K/128] (128x128)
    ti.B = p.B + int64_t(e_found) * p.N * p.K + (B_KN ? ti.n0 : ti.n0 * p.ldb);
    ti.sb = p.sb + int64_t(e_found) * (EPI == Epi::Block128x128 ? (p.N / 128) * (p.K / 128) : p.N);
    ti.bias = BIAS ? p.bias + int64_t(e_found) * p.bias_stride_e : nullptr;
  }

  const int K = ti.K;
  const int nk = (K + BK - 1) / BK;
  // Split K: grid row y covers K steps [kt_begin, kt_end) (all of K when the
  // grid has one row).
  const int kt_begin = int(int64_t(nk) * blockIdx.y / gridDim.y);
  const int kt_end = int(int64_t(nk) * (blockIdx.y + 1) / gridDim.y);

  // ---------------- loaders ----------------
  // Direct-to-LDS: load number q < LA of wave w fills tile rows
  // [(q*NW + w) * 8, +8); lane l writes LDS bytes [16 l, 16 l + 16) of that
  // 1 KiB span, i.e. row l/8 of the span, slot l%8, which holds chunk
  // (l%8) ^ swz(row).  The span starts at a multiple of 8 rows and NW is
  // even, so swz(row) = ((w & 1) << 2) | (l >> 4) for every q.
  const int ld_row = lane >> 3;
  const int ld_chunk = (lane & 7) ^ (((wave & 1) << 2) | (lane >> 4));
  const Rsrc rsA = make_rsrc4(ti.A, uint32_t(ti.rows_valid) * uint32_t(p.lda));
  __amdgpu_buffer_rsrc_t rsB;             // B stored [K, N]: register loads
  Rsrc rsB4;                              // B stored [N, K]: DMA
  if constexpr (!B_KN) rsB4 = make_rsrc4(ti.B, uint32_t(ti.cols_valid) * uint32_t(p.ldb));
  else rsB = make_rsrc(ti.B, uint32_t(K) * uint32_t(p.ldb) - uint32_t(ti.n0));
  // per-lane byte offsets of each load at k = 0; the K position is the
  // instruction's scalar offset
  uint32_t voffA[LA];
#pragma unroll
  for (int q = 0; q < LA; ++q) voffA[q] = uint32_t((q * NW + wave) * 8 + ld_row) * uint32_t(p.lda) + ld_chunk * 16;
  uint32_t voffB[LB > 0 ? LB : 1];
#pragma unroll
  for (int q = 0; q < LB; ++q) voffB[q] = uint32_t((q * NW + wave) * 8 + ld_row) * uint32_t(p.ldb) + ld_chunk * 16;
  const uint32_t lds0 = lds_addr(stage0), lds1 = lds_addr(stage1), lds2 = lds_addr(stage2);
  auto stage_lds = [&](int s) -> uint32_t { return s == 0 ? lds0 : (s == 1 ? lds1 : lds2); };
  constexpr bool k_ragged = !K_ALIGNED;   // K % 128 != 0 is possible

  // Issue load number q (0 <= q < LA + LB + LS) of K step kt into its stage.
  // Past the last K step the same instructions go through a descriptor with
  // no valid bytes: they write zeros into a stage nobody reads and keep the
  // per-step load count uniform for the vmcnt bookkeeping, without branches.
  auto issue_one = [&](int q, int stage, int kt, bool live) {
    const uint32_t st = stage_lds(stage);
    const uint32_t k0 = uint32_t(kt) * BK;
    const bool tail = k_ragged && (int(k0) + BK > K);   // K_ALIGNED: folds to false
    if (q < LA) {
      const Rsrc r = live ? rsA : dead(rsA);
      uint32_t vo = voffA[q];
      if (tail) vo = (int(k0) + ld_chunk * 16 < K) ? vo : 0x80000000u;
      dma_b128(r, st + (q * NW + wave) * 1024, vo, k0);
    } else if (q < LA + LB) {
      const int qb = q - LA;
      const Rsrc r = live ? rsB4 : dead(rsB4);
      uint32_t vo = voffB[qb];
      if (tail) vo = (int(k0) + ld_chunk * 16 < K) ? vo : 0x80000000u;
      dma_b128(r, st + A_BYTES + (qb * NW + wave) * 1024, vo, k0);
    } else if constexpr (MX) {
      // chunk c < 4: E8M0 bytes of A rows row0 + 64c + lane; c >= 4: of B
      // columns n0 + 64(c - 4) + lane; 4 bytes (K step kt) per lane at 4 lane
      const int c = (q - LA - LB) * NW + wave;
      const int64_t nkb = K / 32;
      const int w4 = c & 3;
      const int64_t first = (c < 4 ? ti.row0 : ti.n0) + 64 * w4;
      const int valid = c < 4 ? ti.rows_valid : ti.cols_valid;
      const int here = live ? min(max(valid - 64 * w4, 0), 64) : 0;
      const uint8_t* base = (c < 4 ? reinterpret_cast<const uint8_t*>(ti.sa) : reinterpret_cast<const uint8_t*>(ti.sb)) +
                            (here > 0 ? first * nkb : 0);
      const Rsrc r = make_rsrc4(base, uint32_t(here) * uint32_t(nkb));
      dma_b32(r, st + A_BYTES + B_BYTES + (c < 4 ? 0 : SA_BYTES) + w4 * 256,
              uint32_t(lane) * uint32_t(nkb) + uint32_t(kt) * 4u);
    } else if constexpr (BLOCKWISE) {
      const int c = (q - LA - LB) * NW + wave;        // scale chunk 0..7 of this wave
      if (c < 4) {
        // sA[kb, row0 + 64c .. +64).  The descriptor spans to the end of the
        // scale array, so no load is partly out of range; rows past the tile
        // edge read neighbouring scales that only reach rows never stored.
        const int64_t off = int64_t(kt) * p.M + ti.row0 + c * 64;
        const int64_t rem = int64_t(nk) * p.M - off;
        const Rsrc r = make_rsrc4(ti.sa + (rem > 0 ? off : 0), uint32_t(rem > 0 && live ? rem * 4 : 0));
        dma_b32(r, st + A_BYTES + B_BYTES + c * 256, uint32_t(lane) * 4u);
      } else {
        const int cc = c - 4;
        if constexpr (EPI == Epi::Block128x1) {
          // column scales sB[kb, n0 + 64cc .. +64)
          const bool in = live && cc * 64 < BN;
          const int64_t off = int64_t(kt) * p.N + ti.n0 + cc * 64;
          const int64_t rem = int64_t(nk) * p.N - off;
          const Rsrc r = make_rsrc4(ti.sb + (rem > 0 && in ? off : 0), uint32_t(rem > 0 && in ? rem * 4 : 0));
          dma_b32(r, st + A_BYTES + B_BYTES + SA_BYTES + cc * 256, uint32_t(lane) * 4u);
        } else {
          // the weight-block scale of (n-block n0/128 + cc, kb), fetched by lane 0
          const int64_t nb = ti.n0 / 128 + cc;
          const bool in = live && cc < BN / 128 && nb < p.N / 128;
          const int64_t idx = B_KN ? int64_t(kt) * (p.N / 128) + nb : nb * nk + kt;
          const Rsrc r = make_rsrc4(ti.sb + (in ? idx : 0), uint32_t(in ? 4 : 0));
          dma_b32(r, st + A_BYTES + B_BYTES + SA_BYTES + cc * 256, uint32_t(lane) * 4u);
        }
      }
    }
  };
  constexpr int LDIRECT = LA + LB + LS;

  // B stored [K, N]: thread t loads KR consecutive k rows x 16 n bytes and
  // writes them transposed into the [N][128] tile (v_perm_b32 4x4 transposes).
  const int kn_nc = tid % NCH;
  const int kn_kg = tid / NCH;
  v4i kn_regs[KR];
  auto kn_load = [&](int kt, bool live) {
    if constexpr (B_KN) {
      const int k0 = kt * BK + kn_kg * KR;
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        const bool in = live && (k0 + r < K) && (kn_nc * 16 < ti.cols_valid);
        const uint32_t off = in ? uint32_t(k0 + r) * uint32_t(p.ldb) + uint32_t(kn_nc * 16) : 0x80000000u;
        kn_regs[r] = __builtin_amdgcn_raw_buffer_load_b128(rsB, off, 0, 0);
      }
    }
  };
  auto kn_store = [&](int stage) {
    if constexpr (B_KN) {
      uint8_t* bt = stage_ptr(stage) + A_BYTES;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
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
          const int kl = kn_kg * KR;
          uint8_t* dst = bt + lds_off(n, kl >> 4) + (kl & 15);
          if constexpr (KR == 8)
            *reinterpret_cast<uint2*>(dst) = make_uint2(cols[0][jn], cols[1][jn]);
          else
            *reinterpret_cast<uint32_t*>(dst) = cols[0][jn];
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
  const int fq = lane >> 4;     // the lane's 16-byte chunks of the 128-byte K block: fq and fq + 4
  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Both operands take the same k order, so the contraction is unchanged;
  // chunks q and q + 4 (rather than 2q, 2q + 1) keep the 16-lane groups of
  // one read on distinct LDS banks.
  auto read_frag = [&](const uint8_t* tile, int r) {
    const v4i lo = *reinterpret_cast<const v4i*>(tile + lds_off(r, fq));
    const v4i hi = *reinterpret_cast<const v4i*>(tile + lds_off(r, fq + 4));
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  // One K step on stage S.  The loads of K step kt + D (zeros past the end)
  // are spread over the fragment rows, the A fragment of the next row is read
  // one row ahead, and sched_barrier fences pin the order (MFMA q, promotion
  // of MFMA q-1) so that every MFMA overlaps the VALU work of its
  // predecessor instead of waiting for it.
  auto compute = [&](auto stage_c, int kt, bool live_next) {
    constexpr int S = decltype(stage_c)::value;
    const uint8_t* As = stage_ptr(S);
    const uint8_t* Bs = As + A_BYTES;
    [[maybe_unused]] const float* sas = reinterpret_cast<const float*>(As + A_BYTES + B_BYTES);
    [[maybe_unused]] const float* sbs = reinterpret_cast<const float*>(As + A_BYTES + B_BYTES + SA_BYTES);
    v8i a_cur = read_frag(As, row_base + frow);
    v8i b[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j] = read_frag(Bs, col_base + j * 16 + frow);
    // MXFP8: the lane's E8M0 byte for its row / column and lane group fq
    [[maybe_unused]] const uint8_t* sab = As + A_BYTES + B_BYTES;
    [[maybe_unused]] int mxb[FN];
    [[maybe_unused]] int mxa_cur = 0;
    if constexpr (MX) {
#pragma unroll
      for (int j = 0; j < FN; ++j) mxb[j] = sab[SA_BYTES + (col_base + j * 16 + frow) * 4 + fq];
      mxa_cur = sab[(row_base + frow) * 4 + fq];
    }
    [[maybe_unused]] float sbk = 0.f;
    [[maybe_unused]] float sbv[FN];
    [[maybe_unused]] v4f fa_cur;
    if constexpr (BLOCKWISE) {
      fa_cur = *reinterpret_cast<const v4f*>(sas + row_base + fq * 4);
      if constexpr (EPI == Epi::Block128x128) sbk = sbs[(col_base / 128) * 64];
      if constexpr (EPI == Epi::Block128x1) {
#pragma unroll
        for (int j = 0; j < FN; ++j) sbv[j] = sbs[col_base + j * 16 + frow];
      }
    }
    [[maybe_unused]] v4f t_prev = v4f{0.f, 0.f, 0.f, 0.f};
    [[maybe_unused]] v4f f_prev = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int q = i * LDIRECT / FM; q < (i + 1) * LDIRECT / FM; ++q) issue_one(q, (S + D) % STAGES, kt + D, live_next);
      v8i a_next = a_cur;
      [[maybe_unused]] v4f fa_next;
      [[maybe_unused]] int mxa_next = mxa_cur;
      if (i + 1 < FM) {
        a_next = read_frag(As, row_base + (i + 1) * 16 + frow);
        if constexpr (MX) mxa_next = sab[(row_base + (i + 1) * 16 + frow) * 4 + fq];
        if constexpr (BLOCKWISE) fa_next = *reinterpret_cast<const v4f*>(sas + row_base + (i + 1) * 16 + fq * 4);
      }
      if constexpr (MX) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = mfma_16x16x128_mx(a_cur, b[j], acc[i][j], mxa_cur, mxb[j]);
          asm volatile("" : "+v"(acc[i][j]));   // keeps the compiler's order (see the streaming kernel)
          __builtin_amdgcn_sched_barrier(0);
        }
        mxa_cur = mxa_next;
      } else if constexpr (!BLOCKWISE) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = mfma_16x16x128(a_cur, b[j], acc[i][j]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        v4f fa = fa_cur;
        if constexpr (EPI == Epi::Block128x128) fa = fa * sbk;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v4f t = mfma_16x16x128(a_cur, b[j], v4f{0.f, 0.f, 0.f, 0.f});
          if (i > 0 || j > 0) {
            const int ip = j > 0 ? i : i - 1;
            const int jp = j > 0 ? j - 1 : FN - 1;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[ip][jp][e] = __builtin_fmaf(t_prev[e], f_prev[e], acc[ip][jp][e]);
          }
          t_prev = t;
          if constexpr (EPI == Epi::Block128x128) {
            f_prev = fa;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) f_prev[e] = fa[e] * sbv[j];
          }
          // within this region: the MFMA issues first, the VALU work after it
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        fa_cur = fa_next;
      }
      a_cur = a_next;
    }
    if constexpr (BLOCKWISE) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[FM - 1][FN - 1][e] = __builtin_fmaf(t_prev[e], f_prev[e], acc[FM - 1][FN - 1][e]);
    }
  };

  // ---------------- main loop: STAGES-deep ring, prefetch distance D ----------------
  auto step = [&](auto stage_c, int kt) {
    constexpr int S = decltype(stage_c)::value;
    // Stage kt is complete once only the newest D-1 steps' loads are in
    // flight.  A bare s_barrier (not __syncthreads, whose release fence would
    // drain every outstanding load): each wave first retires its own DMA for
    // this stage and its LDS reads / writes, so after the barrier the stage is
    // complete and the stage refilled next is no longer being read.
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((D - 1) * LPS) : "memory");
    const bool live = kt + D < kt_end;
    kn_load(kt + D, live);
    compute(stage_c, kt, live);
    kn_store((S + D) % STAGES);
  };
  if (kt_end > kt_begin) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kd = kt_begin + d;
#pragma unroll
      for (int q = 0; q < LDIRECT; ++q) issue_one(q, d, kd, kd < kt_end);
      kn_load(kd, kd < kt_end);
      kn_store(d);
    }
    for (int kt = kt_begin; kt < kt_end; kt += STAGES) {
      step(std::integral_constant<int, 0>{}, kt);
      if (kt + 1 < kt_end) step(std::integral_constant<int, 1>{}, kt + 1);
      if constexpr (STAGES > 2) {
        if (kt + 2 < kt_end) step(std::integral_constant<int, 2 % STAGES>{}, kt + 2);
      }
    }
  }

  // ---------------- epilogue: scale, round, stage in LDS, 16-byte stores ----------------
  // Every DMA of the ring (including the zero loads issued past the last K
  // step into spare stages) has landed before the stages are reused below.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();   // every wave is done with the ring
  uint8_t* ep = (wave < NW / 2 ? stage0 : stage1) + (wave % (NW / 2)) * TM * EPI_PITCH;
  [[maybe_unused]] float s_tensor = 0.f;
  if constexpr (EPI == Epi::Tensor) s_tensor = p.sa[0] * p.sb[0];
  [[maybe_unused]] float sar[FM][4];
  if constexpr (EPI == Epi::Row) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rt = row_base + i * 16 + fq * 4 + e;   // row within the block tile
        sar[i][e] = rt < ti.rows_valid ? p.sa[ti.row0 + rt] : 0.f;
      }
  }
#pragma unroll
  for (int pass = 0; pass < EPI_PASSES; ++pass) {
    constexpr int FNP = FN / EPI_PASSES;
#pragma unroll
    for (int jj = 0; jj < FNP; ++jj) {
      const int j = pass * FNP + jj;
      const int cl = jj * 16 + frow;                  // column within this pass
      const int ct = col_base + j * 16 + frow;        // column within the block tile
      const bool cin = ct < ti.cols_valid;
      [[maybe_unused]] float sbc = 0.f;
      if constexpr (EPI == Epi::Row) sbc = cin ? ti.sb[ti.n0 + ct] : 0.f;
      float bias_v = 0.f;
      if constexpr (BIAS) bias_v = cin ? __uint_as_float(uint32_t(ti.bias[ti.n0 + ct]) << 16) : 0.f;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = acc[i][j][e];
          if constexpr (EPI == Epi::Tensor) v = v * s_tensor;
          if constexpr (EPI == Epi::Row) v = (v * sar[i][e]) * sbc;
          if constexpr (BIAS) v = v + bias_v;
          uint8_t* dst = ep + (i * 16 + fq * 4 + e) * EPI_PITCH + cl * OUTB;
          if constexpr (OUT_BF16)
            *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16_rne(v);
          else
            *reinterpret_cast<float*>(dst) = v;
        }
      }
    }
    __syncthreads();
    constexpr int CPR = EPI_COLS * OUTB / 16;       // 16-byte chunks per staged row
    constexpr int EPR = 16 / OUTB;                  // elements per chunk
    constexpr int ITER = TM * CPR / 64;             // 16-byte copies per lane and pass
    constexpr int BATCH = ITER % 4 == 0 ? 4 : (ITER % 2 == 0 ? 2 : 1);
    static_assert((TM * CPR) % 64 == 0, "copy-out per lane");
    if (vec_out && row_base + TM <= ti.rows_valid && col_base + TN <= ti.cols_valid) {
      // The wave's whole sub-tile is inside the output: no per-chunk
      // conditions, so each lane has BATCH LDS reads in flight before their
      // stores (one at a time, every copy waited out the LDS latency).
      uint8_t* const obase = reinterpret_cast<uint8_t*>(p.out) +
                             ((ti.out_off + int64_t(blockIdx.y) * p.split_stride +
                               (ti.row0 - p.out_row0 + row_base) * p.ldo + ti.n0 + col_base + pass * EPI_COLS) * OUTB);
#pragma unroll
      for (int u0 = 0; u0 < ITER; u0 += BATCH) {
        v4i val[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int idx = lane + (u0 + u) * 64;
          val[u] = *reinterpret_cast<const v4i*>(ep + (idx / CPR) * EPI_PITCH + (idx % CPR) * 16);
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int idx = lane + (u0 + u) * 64;
          *reinterpret_cast<v4i*>(obase + int64_t(idx / CPR) * p.ldo * OUTB + (idx % CPR) * 16) = val[u];
        }
      }
      if (pass + 1 < EPI_PASSES) __syncthreads();
      continue;
    }
#pragma unroll 4
    for (int idx = lane; idx < TM * CPR; idx += 64) {
      const int rl = idx / CPR;
      const int ch = idx % CPR;
      const int rt = row_base + rl;
      const int ct = col_base + pass * EPI_COLS + ch * EPR;
      if (rt >= ti.rows_valid || ct >= ti.cols_valid) continue;
      const uint8_t* src = ep + rl * EPI_PITCH + ch * 16;
      uint8_t* dst = reinterpret_cast<uint8_t*>(p.out) +
                     ((ti.out_off + int64_t(blockIdx.y) * p.split_stride + (ti.row0 - p.out_row0 + rt) * p.ldo +
                       ti.n0 + ct) * OUTB);
      if (vec_out && ct + EPR <= ti.cols_valid) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        const int n = min(EPR, ti.cols_valid - ct);
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

template <int BM, int BN, int WM, int WN, int STAGES, Epi EPI, bool B_KN, bool OUT_BF16, bool BIAS, bool GROUPED>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t st) {
  int tiles_m, tiles_n = int((p.N + BN - 1) / BN);
  if (GROUPED)
    tiles_m = int((p.M + BM - 1) / BM + p.E);   // upper bound on expert m-tiles
  else
    tiles_m = int((p.row_end - p.row_begin + BM - 1) / BM);
  const int64_t tiles = int64_t(tiles_m) * tiles_n;
  if (tiles == 0) return hipSuccess;
  const int grid = int((tiles + 7) / 8 * 8);
  const int outb = p.out_bf16 ? 2 : 4;
  const int vec_out = ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0) && ((p.ldo * outb) % 16 == 0);
  // blockwise and MXFP8 problems have K % 128 == 0 (checked by the caller)
  constexpr bool BLOCKWISE = EPI == Epi::Block128x128 || EPI == Epi::Block128x1 || EPI == Epi::MX;
  if (BLOCKWISE || p.K % BK == 0)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, STAGES, EPI, B_KN, OUT_BF16, BIAS, GROUPED, true>),
                       dim3(grid, max(1, p.splits)), dim3(WM * WN * 64), 0, st, p, tiles_m, tiles_n, vec_out);
  else if constexpr (!BLOCKWISE)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, STAGES, EPI, B_KN, OUT_BF16, BIAS, GROUPED, false>),
                       dim3(grid, max(1, p.splits)), dim3(WM * WN * 64), 0, st, p, tiles_m, tiles_n, vec_out);
  return hipGetLastError();
}

template <Epi EPI, bool B_KN, bool OUT_BF16, bool BIAS, bool GROUPED>
hipError_t launch_epi(const GemmProblem& p, hipStream_t st) {
  // tensorwise / rowwise: 256 x 256 tiles, 8 waves (2 per SIMD), 2 stages;
  // blockwise: the promotion's registers do not fit two waves per SIMD, so
  // 256 x 128 tiles, 4 waves, 3 stages; grouped: 128 x 128 tiles, 3 stages.
  constexpr bool BLOCKWISE = EPI == Epi::Block128x128 || EPI == Epi::Block128x1;
  if constexpr (GROUPED)
    return launch_cfg<128, 128, 2, 2, 3, EPI, B_KN, OUT_BF16, BIAS, true>(p, st);
  else if constexpr (BLOCKWISE && B_KN)
    return launch_cfg<256, 128, 2, 2, 3, EPI, true, OUT_BF16, BIAS, false>(p, st);   // cfg:kn_block
  else if constexpr (B_KN)
    return launch_cfg<256, 256, 2, 4, 2, EPI, true, OUT_BF16, BIAS, false>(p, st);   // cfg:kn_row
  else if constexpr (BLOCKWISE)
    return launch_cfg<256, 128, 2, 2, 3, EPI, false, OUT_BF16, BIAS, false>(p, st);  // cfg:block
  else
    return launch_cfg<256, 256, 2, 4, 2, EPI, false, OUT_BF16, BIAS, false>(p, st);  // cfg:row
}

template <Epi EPI, bool B_KN, bool GROUPED>
hipError_t launch_out(const GemmProblem& p, hipStream_t st) {
  const bool bias = p.bias != nullptr;
  if (p.out_bf16)
    return bias ? launch_epi<EPI, B_KN, true, true, GROUPED>(p, st) : launch_epi<EPI, B_KN, true, false, GROUPED>(p, st);
  return bias ? launch_epi<EPI, B_KN, false, true, GROUPED>(p, st) : launch_epi<EPI, B_KN, false, false, GROUPED>(p, st);
}

// The grouped weight gradient: 128 x 128 tiles of E problems, 2 stages (two
// workgroups per CU), grid E x tiles padded to a multiple of 8.
template <bool OUT_BF16>
hipError_t launch_group_k(const GemmProblem& p, hipStream_t st) {
  constexpr int BM = 128, BN = 128;
  const int tiles_m = int((p.M + BM - 1) / BM), tiles_n = int((p.N + BN - 1) / BN);
  const int64_t total = int64_t(tiles_m) * tiles_n * p.E;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 7) / 8 * 8;
  if (grid > int64_t(INT32_MAX)) return hipErrorInvalidValue;
  const int outb = OUT_BF16 ? 2 : 4;
  const int vec_out = ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0) && ((p.ldo * outb) % 16 == 0);
  hipLaunchKernelGGL(
      (gemm_kernel<BM, BN, 2, 2, 2, Epi::Block128x1, false, OUT_BF16, false, false, true, true>),
      dim3(unsigned(grid)), dim3(256), 0, st, p, tiles_m, tiles_n, vec_out);
  return hipGetLastError();
}

// Compute units of the device the stream belongs to, cached per device.
// Calls from several host threads may fill an entry at once; they store the
// same value, through atomics.
static int device_cus(hipStream_t st) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipStreamGetDevice(st, &dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The tail rows of a plain GEMM.  A short tail (its 128 x 128 tiles fit in
// half the compute units) uses 128 x 128 tiles on 4 waves, four workgroups
// per 256 x 256 tile; a longer one 256 x 128 tiles on 8 waves (B stored
// [K, N]: 4 waves), which run closer to the streaming kernel's rate.
template <Epi EPI, bool OUT_BF16, bool BIAS>
hipError_t launch_tail(const GemmProblem& p, bool small, hipStream_t st) {
  if constexpr (EPI != Epi::MX) {
    if (p.b_kn) {
      if (small) return launch_cfg<128, 128, 2, 2, 3, EPI, true, OUT_BF16, BIAS, false>(p, st);
      return launch_cfg<256, 128, 2, 2, 3, EPI, true, OUT_BF16, BIAS, false>(p, st);
    }
  }
  if (small) return launch_cfg<128, 128, 2, 2, 3, EPI, false, OUT_BF16, BIAS, false>(p, st);
  return launch_cfg<256, 128, 4, 2, 3, EPI, false, OUT_BF16, BIAS, false>(p, st);
}

template <Epi EPI>
hipError_t launch_tail_out(const GemmProblem& p, bool small, hipStream_t st) {
  const bool bias = p.bias != nullptr;
  if (p.out_bf16)
    return bias ? launch_tail<EPI, true, true>(p, small, st) : launch_tail<EPI, true, false>(p, small, st);
  return bias ? launch_tail<EPI, false, true>(p, small, st) : launch_tail<EPI, false, false>(p, small, st);
}

hipError_t launch_gemm_tail(const GemmProblem& p, bool small, hipStream_t st) {
  switch (p.epi) {
    case Epi::Tensor: return launch_tail_out<Epi::Tensor>(p, small, st);
    case Epi::Row: return launch_tail_out<Epi::Row>(p, small, st);
    case Epi::Block128x128: return launch_tail_out<Epi::Block128x128>(p, small, st);
    case Epi::Block128x1: return launch_tail_out<Epi::Block128x1>(p, small, st);
    case Epi::MX: return p.b_kn ? hipErrorInvalidValue : launch_tail_out<Epi::MX>(p, small, st);
  }
  return hipErrorInvalidValue;
}

// Sum of the split-K partials: out[row_begin + r, c] = round(sum_y part[y][r][c]
// (+ bias[c])), the slices added in order y = 0, 1, ...  One thread per four
// adjacent columns of one row.
template <bool OUT_BF16, bool BIAS>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* part, int splits, int64_t slice,
                                                            int64_t rows, int64_t N, const uint16_t* bias,
                                                            void* out, int64_t ldo, int64_t row_begin) {
  const int64_t n4 = (N + 3) / 4;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= rows * n4) return;
  const int64_t r = idx / n4;
  const int64_t c = (idx % n4) * 4;
  const int nc = int(min<int64_t>(4, N - c));
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int y = 0; y < splits; ++y) {
    const float* src = part + y * slice + r * N + c;
    if (nc == 4 && (N & 3) == 0) {
      const v4f t = *reinterpret_cast<const v4f*>(src);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += t[e];
    } else {
      for (int e = 0; e < nc; ++e) v[e] += src[e];
    }
  }
  if constexpr (BIAS) {
    for (int e = 0; e < nc; ++e) v[e] += __uint_as_float(uint32_t(bias[c + e]) << 16);
  }
  const int64_t o = (row_begin + r) * ldo + c;
  if constexpr (OUT_BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(out) + o;
    for (int e = 0; e < nc; ++e) dst[e] = f32_to_bf16_rne(v[e]);
  } else {
    float* dst = reinterpret_cast<float*>(out) + o;
    for (int e = 0; e < nc; ++e) dst[e] = v[e];
  }
}

// The short tail split along K: the tail's tiles (128 x 128, or with `small`
// false the generic kernel's 256 x 128) x `splits` K ranges write fp32
// partials to `scratch` (splits x rows x N floats, 16-byte aligned), then one
// pass sums them in order, adds the bias and rounds once into the tail rows
// of the output.
hipError_t launch_tail_splitk(const GemmProblem& p, int splits, float* scratch, hipStream_t st, bool small) {
  const int64_t rows = p.row_end - p.row_begin;
  const int64_t slice = rows * p.N;
  GemmProblem q = p;
  q.out = scratch;
  q.ldo = p.N;
  q.out_bf16 = false;
  q.bias = nullptr;
  q.out_row0 = p.row_begin;
  q.split_stride = slice;
  q.splits = splits;
  hipError_t e = launch_gemm_tail(q, small, st);
  if (e != hipSuccess) return e;
  const int64_t threads = rows * ((p.N + 3) / 4);
  const dim3 grid(unsigned((threads + 255) / 256));
  if (p.out_bf16) {
    if (p.bias)
      hipLaunchKernelGGL((splitk_reduce_kernel<true, true>), grid, dim3(256), 0, st, scratch, splits, slice, rows, p.N,
                         p.bias, p.out, p.ldo, p.row_begin);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<true, false>), grid, dim3(256), 0, st, scratch, splits, slice, rows,
                         p.N, p.bias, p.out, p.ldo, p.row_begin);
  } else {
    if (p.bias)
      hipLaunchKernelGGL((splitk_reduce_kernel<false, true>), grid, dim3(256), 0, st, scratch, splits, slice, rows,
                         p.N, p.bias, p.out, p.ldo, p.row_begin);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<false, false>), grid, dim3(256), 0, st, scratch, splits, slice, rows,
                         p.N, p.bias, p.out, p.ldo, p.row_begin);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmProblem& p, hipStream_t st) {
  if (p.group_k) {
    if (p.epi != Epi::Block128x1 || p.b_kn || p.bias || !p.offsets) return hipErrorInvalidValue;
    if (p.lda >= 128 && p.ldb >= 128) return launch_gemm_group_k_streaming(p, st);
    return p.out_bf16 ? launch_group_k<true>(p, st) : launch_group_k<false>(p, st);
  }
  if (p.offsets) {
    // grouped: experts of a few hundred rows with weights stored [N, K] on
    // the weight-streaming kernel; otherwise the streaming kernel when its
    // grouped loads fit the leading dimensions (as below), else 128 x 128
    // tiles
    if (grouped_wide_applies(p)) return launch_gemm_grouped_wide(p, st);
    if (p.lda >= 128 && (p.b_kn ? p.ldb >= 256 : p.ldb >= 128)) return launch_gemm_streaming(p, st);
    if (p.epi == Epi::Row)
      return p.b_kn ? launch_out<Epi::Row, true, true>(p, st) : launch_out<Epi::Row, false, true>(p, st);
    if (p.epi == Epi::Block128x128)
      return p.b_kn ? launch_out<Epi::Block128x128, true, true>(p, st)
                    : launch_out<Epi::Block128x128, false, true>(p, st);
    return hipErrorInvalidValue;
  }
  // The streaming kernel's grouped loads need leading dimensions of at least
  // 128 bytes (256 for B stored [K, N]).  Its 256 x 256 tiles are handed out in rounds of one per CU;
  // when the last round would be less than half full, the streaming kernel
  // takes the rows of tiles that fill whole rounds and the rest of the rows
  // (the tail) run with 128 x 128 tiles, four times as many workgroups.
  const int64_t tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
  const int64_t tiles = tiles_m * tiles_n, cus = device_cus(st);
  // Small problems (even 128 x 128 tiles fill at most half the device): four
  // times as many workgroups on 128 x 128 tiles finish sooner.
  if (4 * tiles <= cus / 2) return launch_gemm_tail(p, true, st);
  if (p.lda >= 128 && (p.b_kn ? p.ldb >= 256 : p.ldb >= 128)) {
    const int64_t rem = tiles % cus;
    const int64_t tm_main = tiles > cus && rem > 0 && rem <= cus / 2 ? (tiles / cus * cus) / tiles_n : tiles_m;
    if (tm_main >= tiles_m || tm_main == 0) return launch_gemm_streaming(p, st);
    GemmProblem head = p, tail = p;
    head.row_end = tm_main * 256;
    tail.row_begin = tm_main * 256;
    const int64_t tail_tiles = (tiles_m - tm_main) * tiles_n;
    const bool small = 4 * tail_tiles <= cus / 2;
    // A short tail leaves most compute units idle: split its K range so that
    // its tiles times the splits cover the device, each split keeping at
    // least 8 K steps.  Tiles of 128 x 128, or with B stored [K, N] 256 x
    // 128 (twice the K ranges per tile: measured 11 us faster on the
    // 16640 x 8192 x 5120 input gradient, no faster with B stored [N, K]).
    // The fp32 partials are staged in the head rows of the output
    // (contiguous rows only), which the streaming kernel overwrites
    // afterwards on the same stream; so the tail runs first.
    const int64_t nk = (p.K + 127) / 128;
    const int64_t per_tile = p.b_kn ? 2 : 4;   // split tiles per 256 x 256 tile
    const int64_t splits = small ? std::min<int64_t>({cus / (per_tile * tail_tiles), nk / 8, 8}) : 1;
    if (splits >= 2 && p.ldo == p.N) {
      const uintptr_t base = reinterpret_cast<uintptr_t>(p.out);
      const uintptr_t scratch = (base + 255) & ~uintptr_t(255);
      const uintptr_t head_end = base + uintptr_t(head.row_end) * uintptr_t(p.N) * (p.out_bf16 ? 2u : 4u);
      const uintptr_t need = uintptr_t(splits) * uintptr_t(p.M - tail.row_begin) * uintptr_t(p.N) * 4u;
      if (scratch + need <= head_end) {
        const hipError_t e = launch_tail_splitk(tail, int(splits), reinterpret_cast<float*>(scratch), st, !p.b_kn);
        if (e != hipSuccess) return e;
        return launch_gemm_streaming(head, st);
      }
    }
    const hipError_t e = launch_gemm_streaming(head, st);
    if (e != hipSuccess) return e;
    return launch_gemm_tail(tail, small, st);
  }
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
    case Epi::MX: return p.b_kn ? hipErrorInvalidValue : launch_out<Epi::MX, false, false>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fp8mm
