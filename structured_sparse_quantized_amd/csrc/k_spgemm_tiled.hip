// 2:4 sparse x dense product on a pre-tiled sparse operand (gfx950 v_smfmac),
// with the per-token x per-channel rescale epilogue, and the pack kernel that
// writes the tiled operand.
// Deep reading of arXiv 2610.28947 (introduction: one operand keeps two of
// every four along the accumulate axis; section 3.1: sparse W or sparse X);
// SlideSparse blog section 2.2 step 3; LLM Compressor W8A8 scales.
//
// C[r][c] = sum_k A[r][k] B[c][k]; A = compressed operand (rows r), B = dense
// operand (rows c). side W: r = output channel n, c = token m; side X: r =
// token m, c = output channel n.
//
// Tiled sparse operand (8-bit values). A step is 128 K positions: 64
// compressed bytes and one 32-bit index word per 32 positions of each row.
//   values: rows in blocks of 16; per block and step one 1 KB block in
//     instruction lane order -- bytes 16l .. 16l+15 are compressed bytes
//     16(l/16) .. 16(l/16)+15 of row 16b + l%16 in that step. A row block's
//     steps are consecutive; the step count is padded to a multiple of 4 with
//     zero values (rows past the end are zero too).
//   metadata: per row block and group of 4 steps one 1 KB block; 32-bit word
//     4l + q is lane l's index word for step 4g + q, i.e. bytes
//     16(4g+q) + 4(l/16) .. +3 of that row's row-major metadata. Padding words
//     are 0x44444444 (positions 0 and 1 of each group, with zero values).
// A lane's instruction operands are therefore one contiguous 16-byte slice of
// a block, and a whole wave's fragment is one contiguous 1 KB read.
// bf16 values: the same bytes per step (a step is then 64 K positions, 32
// compressed values per row) and 16-bit index words: a metadata block holds 4
// steps in 512 bytes, lane l's 2-byte word for step 4g + q at byte 8l + 2q
// (bytes 8(4g+q) + 2(l/16) of the row-major metadata); padding 0x4444. The
// bf16 instruction (16x16x64) takes the word through its half-select.
//
// Product kernel: 256 (A rows) x 128 (B rows) per workgroup of 8 waves (4 x 2),
// each wave 64 x 64 = 4 x 4 instructions per step. A ring of four 1-step LDS
// stages (16 KB of A values + 16 KB of B) is filled by LDS DMA
// (global_load_lds, 1 KB per wave instruction); the index words go straight to
// registers one 4-step group ahead. Each step waits for the next step's stage,
// then reads that stage's fragments while the current step's smfmacs run.
//
// Block-scaled FP8 (LLM Compressor guide, W8A8-FP8_BLOCK: one weight scale per
// 128 x 128 block, one activation scale per token and group of 128 positions;
// side W): a step is exactly one scale group, so the same kernel runs each
// step's smfmacs from zero and adds the partial tile times s_x[m][step] *
// s_w[n / 128][step] into float32 accumulators. The token scales of each
// 4-step group reach LDS by DMA with the index words (one 256-byte load per
// wave); the weight scale is one scalar load per wave and step.
//
// Decode kernel (side W, at most 64 tokens, when the tiled grid would leave
// the chip idle): one 16-row block per workgroup of 8 waves; the waves split
// the K steps in whole 4-step index groups, stream the sparse values straight
// to registers (a 4-step ring) with the few token rows of the dense operand,
// and sum their partial tiles through LDS before the same epilogue. The
// weight stream is the HBM-bound part.
#include <algorithm>
#include <type_traits>

#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_mma.h"
#include "ss_store.h"

namespace ss {
namespace tiled {

#define SS_LDS __attribute__((address_space(3)))

constexpr int BM = 256, BN = 128, WGM = 4, WGN = 2, NW = WGM * WGN, S = 4;
constexpr int TI = BM / WGM / 16, TJ = BN / WGN / 16;          // 4 x 4 instructions per wave per step
constexpr int PA = BM / 16 / NW, PB = BN / 8 / NW, LPW = PA + PB;  // LDS DMA loads per wave per step
constexpr int A_BYTES = BM * 64, STAGE = A_BYTES + BN * 128;   // 32 KB
constexpr int LDS = S * STAGE;                                 // 128 KB
constexpr int SX_BYTES = 128 * 4 * 4;                          // block-scaled: token scales of one 4-step group
constexpr int LDS_BS = LDS + 2 * SX_BYTES;
constexpr int SC_BYTES = (BM + BN) * 4;                        // epilogue scales of one tile (A rows, B rows)
constexpr int LDS_SC = LDS + SC_BYTES;
static_assert(PA * NW * 16 == BM && PB * NW * 8 == BN, "load split");
static_assert(S >= 3 && S <= 5, "wait counts below assume 3..5 stages");

// One thread per (row block, 4-step group, lane); 4 row blocks per workgroup. ES = value bytes; ldv in
// bytes.
template <int ES>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ vals, int64_t ldv,
                                                   const uint8_t* __restrict__ meta, int64_t ldm, int R, int KS,
                                                   int KS4, int nrb, uint8_t* __restrict__ tv, uint8_t* __restrict__ tm) {
  const int g = blockIdx.x, rb = blockIdx.y * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (rb >= nrb) return;
  const int row = rb * 16 + (l & 15), c = l >> 4;
  const bool live = row < R;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int s = 4 * g + q;
    uint4 v = make_uint4(0, 0, 0, 0);
    w[q] = ES == 1 ? 0x44444444u : 0x4444u;
    if (live && s < KS) {
      v = *reinterpret_cast<const uint4*>(vals + row * ldv + 64 * s + 16 * c);
      if constexpr (ES == 1) w[q] = *reinterpret_cast<const uint32_t*>(meta + row * ldm + 16 * s + 4 * c);
      else w[q] = *reinterpret_cast<const uint16_t*>(meta + row * ldm + 8 * s + 2 * c);
    }
    *reinterpret_cast<uint4*>(tv + ((int64_t)rb * 4 * KS4 + s) * 1024 + 16 * l) = v;
  }
  if constexpr (ES == 1)
    *reinterpret_cast<uint4*>(tm + ((int64_t)rb * KS4 + g) * 1024 + 16 * l) = make_uint4(w[0], w[1], w[2], w[3]);
  else
    *reinterpret_cast<uint2*>(tm + ((int64_t)rb * KS4 + g) * 512 + 8 * l) =
        make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
}

// BS: block-scaled FP8 (AB == 1, side W); sx is [C][KS] and sw [ceil(R / 128)][KS].
// The body of the product kernel (one tile per workgroup: blockIdx.x of gridDim.x).
template <int AB, int YT, bool SIDE_X, bool BS>
__device__ __forceinline__ void spgemm_body(int R, int C, int KS, const uint8_t* __restrict__ tv,
                                            const uint8_t* __restrict__ tm, const uint8_t* __restrict__ bd, int ldb,
                                            const float* __restrict__ sx, const float* __restrict__ sw,
                                            void* __restrict__ Y, int ldy, int tiles_r, int tiles_c) {
  using Acc = typename Mma<AB>::Acc;
  using MT = Meta<AB>;
  using MV = typename MT::V;
  extern __shared__ __align__(16) uint8_t smem[];
  // the wave index is uniform: keep it (and the addresses built from it) in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  // Tile order: workgroups are dealt to the 8 XCDs round-robin; give each XCD a
  // contiguous run of tiles, walked in groups of 4 A-row tiles, so the tiles
  // that share operands also share an L2.
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  constexpr int GR = 4;
  const int group = bid / (GR * tiles_c), first_r = group * GR, gsize = min(tiles_r - first_r, GR);
  const int tr = first_r + (bid % (GR * tiles_c)) % gsize, tc = (bid % (GR * tiles_c)) / gsize;
  const int r0 = tr * BM, c0 = tc * BN;
  const int nrb = (R + 15) / 16, KS4 = (KS + 3) / 4, KSP = 4 * KS4;

  // Per-lane sources. Rows past the end are clamped to the last row; their
  // results are never stored.
  const uint8_t* pa[PA];
  uint32_t offb[PB];
  const uint8_t* pmt[TI];
#pragma unroll
  for (int q = 0; q < PA; ++q) pa[q] = tv + (int64_t)min(r0 / 16 + wave + q * NW, nrb - 1) * KSP * 1024 + lane * 16;
#pragma unroll
  for (int q = 0; q < PB; ++q) {
    const int b = (wave + q * NW) * 8 + (lane >> 3);
    offb[q] = (uint32_t)min(c0 + b, C - 1) * (uint32_t)ldb + swz(lane & 7, b & 15) * 16;
  }
#pragma unroll
  for (int t = 0; t < TI; ++t)
    pmt[t] = tm + (int64_t)min(r0 / 16 + wm * TI + t, nrb - 1) * KS4 * MT::BLOCK + lane * (4 * MT::WB);

  // Step k goes to slot k % S. Padding steps of the dense operand (KS <= k < KSP)
  // re-read its last step (in bounds; the sparse operand's padding steps are zero).
  auto issue = [&](int k) {
    SS_LDS uint8_t* base = (SS_LDS uint8_t*)smem + (k % S) * STAGE;
    const int ka = min(k, KSP - 1), kb = min(k, KS - 1);
#pragma unroll
    for (int q = 0; q < PA; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(pa[q] + (int64_t)ka * 1024),
                                       (SS_LDS void*)(base + (wave + q * NW) * 1024), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < PB; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(bd + offb[q] + (uint32_t)kb * 128),
                                       (SS_LDS void*)(base + A_BYTES + (wave + q * NW) * 1024), 16, 0, 0);
  };
  MV mcur[TI], mnxt[TI];
  auto load_meta = [&](MV* m, int g) {
#pragma unroll
    for (int t = 0; t < TI; ++t) m[t] = *reinterpret_cast<const MV*>(pmt[t] + (int64_t)g * MT::BLOCK);
  };
  // Block-scaled: token scales of 4-step group g into LDS buffer g % 2 -- wave w brings tokens 16w ..
  // 16w + 15, lane l token 16w + l / 4 and step 4g + l % 4 (clamped in bounds; never used past the end),
  // so the buffer holds 16 bytes per token.
  const float* sxrow = nullptr;
  if constexpr (BS) sxrow = sx + (int64_t)min(c0 + wave * 16 + (lane >> 2), C - 1) * KS;
  auto load_sx = [&](int g) {
    if constexpr (BS)
      __builtin_amdgcn_global_load_lds((const void*)(sxrow + min(4 * g + (lane & 3), KS - 1)),
                                       (SS_LDS void*)((SS_LDS uint8_t*)smem + LDS + (g & 1) * SX_BYTES + wave * 256),
                                       4, 0, 0);
  };
  // Block-scaled: this wave's weight-scale row (its 64 A rows lie in one 128-row block).
  const float* swrow = nullptr;
  if constexpr (BS) swrow = sw + (int64_t)min((r0 + wm * TI * 16) / 128, (R - 1) / 128) * KS;

  Acc acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int u = 0; u < TJ; ++u) acc[i][u] = Acc{0, 0, 0, 0};
  const int r16 = lane & 15, jj = lane >> 4;
  struct Frag {
    v4i a[TI];
    v4i b[TJ][2];
  };
  auto read = [&](Frag& f, int k) {
    const uint8_t* st = smem + (k % S) * STAGE;
#pragma unroll
    for (int t = 0; t < TI; ++t) f.a[t] = *reinterpret_cast<const v4i*>(st + (wm * TI + t) * 1024 + lane * 16);
#pragma unroll
    for (int u = 0; u < TJ; ++u) {
      const uint8_t* bb = st + A_BYTES + ((wn * TJ + u) * 2 + (r16 >> 3)) * 1024 + (r16 & 7) * 128;
      f.b[u][0] = *reinterpret_cast<const v4i*>(bb + swz(jj, r16) * 16);
      f.b[u][1] = *reinterpret_cast<const v4i*>(bb + swz(4 + jj, r16) * 16);
    }
  };
  auto mma = [&](const Frag& f, auto qc) {
    constexpr int Q = decltype(qc)::value;
#pragma unroll
    for (int u = 0; u < TJ; ++u)
#pragma unroll
      for (int t = 0; t < TI; ++t) acc[t][u] = mma_step<AB, Q>(f.a[t], f.b[u][0], f.b[u][1], acc[t][u], mcur[t]);
  };
  // Block-scaled step, one column u of B at a time: its TI partial tiles from zero, then (READ) its B
  // fragments and A fragment u are refilled from step knext's stage -- B in place, it is single-buffered
  // to leave registers for the partials -- and the previous column's partials, finished by now, are scaled
  // into the accumulators (one FMA per value; with the zeroing of the partials about six vector
  // instructions per smfmac, which bounds this kernel).
  static_assert(TI == TJ, "one A fragment refilled per B column");
  v4i bq[TJ][2];
  auto read_b = [&](int u, int k) {
    const uint8_t* bb = smem + (k % S) * STAGE + A_BYTES + ((wn * TJ + u) * 2 + (r16 >> 3)) * 1024 + (r16 & 7) * 128;
    bq[u][0] = *reinterpret_cast<const v4i*>(bb + swz(jj, r16) * 16);
    bq[u][1] = *reinterpret_cast<const v4i*>(bb + swz(4 + jj, r16) * 16);
  };
  auto step_bs = [&](const v4i* acur, v4i* anxt, auto qc, auto readc, const float* sc, int knext) {
    constexpr int Q = decltype(qc)::value;
    constexpr bool READ = decltype(readc)::value;
    Acc pp[TI];  // the previous column's partial tiles, scaled while this column's smfmacs run
#pragma unroll
    for (int u = 0; u < TJ; ++u) {
      Acc p[TI];
#pragma unroll
      for (int t = 0; t < TI; ++t) p[t] = mma_step<AB, Q>(acur[t], bq[u][0], bq[u][1], Acc{0, 0, 0, 0}, mcur[t]);
      // fenced: left free, the scheduler put each FMA right behind the smfmac it reads, and the wave waited
      // on the matrix core (fenced, 1.04-1.08x as fast, bit-exact)
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (READ) {
        read_b(u, knext);
        anxt[u] = *reinterpret_cast<const v4i*>(smem + (knext % S) * STAGE + (wm * TI + u) * 1024 + lane * 16);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (u > 0) {
#pragma unroll
        for (int t = 0; t < TI; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[t][u - 1][q] = __builtin_fmaf(pp[t][q], sc[u - 1], acc[t][u - 1][q]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < TI; ++t) pp[t] = p[t];
    }
#pragma unroll
    for (int t = 0; t < TI; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[t][TJ - 1][q] = __builtin_fmaf(pp[t][q], sc[TJ - 1], acc[t][TJ - 1][q]);
  };
  // Block-scaled: the scales of step k for this lane's TJ B rows: s_x[token][k] * s_w[block][k].
  auto read_scales = [&](float* sc, int k) {
    if constexpr (BS) {
      const float swk = swrow[min(k, KS - 1)];
      const float* buf = reinterpret_cast<const float*>(smem + LDS + ((k >> 2) & 1) * SX_BYTES) + (k & 3);
#pragma unroll
      for (int u = 0; u < TJ; ++u) sc[u] = __fmul_rn(buf[((wn * TJ + u) * 16 + r16) * 4], swk);
    }
  };

  // Loads complete in issue order, so "stage k+1 has landed" is a wait until at
  // most N of this wave's loads are outstanding, N = the loads issued after
  // stage k+1: the S-3 later stages (LPW each) plus the index groups issued
  // since (TI each; one is issued at every step with q == 0 except in the last
  // group, where none is). The last group issues no stage past the end, so its
  // step q counts only the real stages after k+1: min(S-3, 2-q).
  auto wait_next = [&](auto qc, auto lastc) {
    constexpr int Q = decltype(qc)::value;
    constexpr bool LAST = decltype(lastc)::value;
    constexpr int lo = Q + 6 - S, hi = Q + 3;
    // block-scaled steps issue their index loads after the stage (counted from steps j+2-S .. j-1); the
    // others before it (counted from steps j+3-S .. j-1), which leaves the stage loads free to interleave
    // with the smfmacs
    constexpr int nm = LAST ? 0
                       : BS ? (hi >= 4 && lo <= 4 ? 1 : 0) + (hi >= 8 && lo <= 8 ? 1 : 0)
                            : (hi >= 4 && lo + 1 <= 4 ? 1 : 0) + (hi >= 8 && lo + 1 <= 8 ? 1 : 0);
    constexpr int later = LAST ? (S - 3 < 2 - Q ? S - 3 : 2 - Q) : S - 3;
    constexpr int N = later * LPW + nm * (TI + (BS ? 1 : 0));
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  };
  constexpr int RD = TI + 2 * TJ, NM = TI * TJ;
  // Step j (j + 1 < KSP): make stage j+1 resident, read its fragments while
  // multiplying step j.
  float sc0[TJ], sc1[TJ];  // block-scaled: scales of the current and the next step
  auto step = [&](int j, auto qc, auto lastc, Frag& cur, Frag& nxt, float* scur, float* snxt) {
    constexpr int Q = decltype(qc)::value;
    constexpr bool LAST = decltype(lastc)::value;
    // the fences keep the scheduler from moving loads across the wait and the barrier
    __builtin_amdgcn_sched_barrier(0);
    wait_next(qc, lastc);
    __builtin_amdgcn_s_barrier();  // every wave's loads of stage j+1 landed; slot (j-1) % S is free
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!BS) {
      // index words of the next group, then (below) the stage loads spread among the smfmacs
      if (Q == 0 && !LAST) load_meta(mnxt, j / 4 + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (BS) {
      read_scales(snxt, j + 1);
      step_bs(cur.a, nxt.a, qc, std::true_type{}, scur, j + 1);
      // the step's loads after its smfmacs and fragment reads (4-7% faster than before them); same
      // order (stage, then index words and token scales), so the waits count them as before
      __builtin_amdgcn_sched_barrier(0);
      issue(j + S - 1);
      if (Q == 0) {
        // block-scaled runs the last group in the loop too: its "next" group is a re-read, never used
        const int gn = min(j / 4 + 1, KS4 - 1);
        load_meta(mnxt, gn);
        load_sx(gn);
      }
    } else {
      // the last group (j = KSP-4+q) issues only stages before the end
      constexpr bool ISSUE = !LAST || Q + S - 1 <= 3;
      // Written out in issue order (fenced, so the scheduler keeps it): smfmac p, then fragment read p of
      // stage j+1 (p < RD), and after every odd p one load of stage j+S-1 (A row blocks, then B rows, the
      // order issue() uses). Left to the scheduler, the loads bunched up at the end of the step; spread
      // this way the step was 1.00-1.09x as fast (bit-exact).
      const uint8_t* stn = smem + ((j + 1) % S) * STAGE;
      SS_LDS uint8_t* sbase = (SS_LDS uint8_t*)smem + ((j + S - 1) % S) * STAGE;
      const int ka = min(j + S - 1, KSP - 1), kb = min(j + S - 1, KS - 1);
#pragma unroll
      for (int p = 0; p < NM; ++p) {
        const int u = p / TI, t = p % TI;
        acc[t][u] = mma_step<AB, Q>(cur.a[t], cur.b[u][0], cur.b[u][1], acc[t][u], mcur[t]);
        __builtin_amdgcn_sched_barrier(0);
        if (p < RD) {
          if (p < TI) {
            nxt.a[p] = *reinterpret_cast<const v4i*>(stn + (wm * TI + p) * 1024 + lane * 16);
          } else {
            const int uu = (p - TI) / 2, h = (p - TI) % 2;
            const uint8_t* bb = stn + A_BYTES + ((wn * TJ + uu) * 2 + (r16 >> 3)) * 1024 + (r16 & 7) * 128;
            nxt.b[uu][h] = *reinterpret_cast<const v4i*>(bb + swz(h * 4 + jj, r16) * 16);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (ISSUE && (p & 1) == 1 && p / 2 < LPW) {
          const int q = p / 2;
          if (q < PA)
            __builtin_amdgcn_global_load_lds((const void*)(pa[q] + (int64_t)ka * 1024),
                                             (SS_LDS void*)(sbase + (wave + q * NW) * 1024), 16, 0, 0);
          else
            __builtin_amdgcn_global_load_lds((const void*)(bd + offb[q - PA] + (uint32_t)kb * 128),
                                             (SS_LDS void*)(sbase + A_BYTES + (wave + (q - PA) * NW) * 1024), 16, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      static_assert(2 * LPW <= NM && RD <= NM, "one load per two smfmacs, one read per smfmac");
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
  using NotLast = std::false_type;
  using Last = std::true_type;

  load_meta(mcur, 0);
  load_sx(0);
  // Epilogue scales of the tile (A rows, then B rows; indices clamped) go to LDS by DMA before the first
  // stage, so the first wait covers them and the epilogue reads them without a global round trip.
  const float* sa = SIDE_X ? sx : sw;  // scale indexed by A row
  const float* sb = SIDE_X ? sw : sx;  // scale indexed by B row
  static_assert(BM % 64 == 0 && (BM + BN) / 64 <= NW, "one 64-scale load per wave, A and B scales apart");
  if (!BS && wave < (BM + BN) / 64) {
    const int i = wave * 64 + lane;  // this lane's slot of the tile's BM + BN scales
    const float* src = i < BM ? (sa ? sa + min(r0 + i, R - 1) : nullptr) : (sb ? sb + min(c0 + i - BM, C - 1) : nullptr);
    if (src)
      __builtin_amdgcn_global_load_lds((const void*)src, (SS_LDS void*)((SS_LDS uint8_t*)smem + LDS + wave * 256), 4,
                                       0, 0);
  }
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);
  Frag f0, f1;
  {
    constexpr int N = (S - 2) * LPW;  // stage 0 landed
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (BS) {
#pragma unroll
    for (int u = 0; u < TJ; ++u) {
      read_b(u, 0);
      f0.a[u] = *reinterpret_cast<const v4i*>(smem + (wm * TI + u) * 1024 + lane * 16);
    }
  } else {
    read(f0, 0);
  }
  read_scales(sc0, 0);
  // Block-scaled: every group, the last included, runs this loop (its loads past the end re-read the last
  // step in bounds and are never used), which keeps the register allocation of the loop for the whole K.
  for (int g = 0; g + (BS ? 0 : 1) < KS4; ++g) {
    const int j = 4 * g;
    step(j, Q0{}, NotLast{}, f0, f1, sc0, sc1);
    step(j + 1, Q1{}, NotLast{}, f1, f0, sc1, sc0);
    step(j + 2, Q2{}, NotLast{}, f0, f1, sc0, sc1);
    step(j + 3, Q3{}, NotLast{}, f1, f0, sc1, sc0);
#pragma unroll
    for (int t = 0; t < TI; ++t) mcur[t] = mnxt[t];
  }
  if constexpr (!BS) {
    const int j = KSP - 4;
    step(j, Q0{}, Last{}, f0, f1, sc0, sc1);
    step(j + 1, Q1{}, Last{}, f1, f0, sc1, sc0);
    step(j + 2, Q2{}, Last{}, f0, f1, sc0, sc1);
    mma(f1, std::integral_constant<int, 3>{});
  }
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // no load may outlive the workgroup

  // Epilogue: y = fl32(fl32(float(acc) * sx[m]) * sw[n]), the scales from LDS (staged in the prologue;
  // out-of-range results are never stored). An absent scale vector reads as 1, and a multiply by 1 is exact,
  // so every result takes the same two multiplies with no branch per value.
  float s_a[TI][4], s_b[TJ];
  const float* scl = reinterpret_cast<const float*>(smem + LDS);
  const bool has_a = sa != nullptr && !BS, has_b = sb != nullptr && !BS;
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    const float4 v = *reinterpret_cast<const float4*>(scl + (wm * TI + t) * 16 + 4 * jj);
    s_a[t][0] = has_a ? v.x : 1.0f;
    s_a[t][1] = has_a ? v.y : 1.0f;
    s_a[t][2] = has_a ? v.z : 1.0f;
    s_a[t][3] = has_a ? v.w : 1.0f;
  }
#pragma unroll
  for (int u = 0; u < TJ; ++u) s_b[u] = has_b ? scl[BM + (wn * TJ + u) * 16 + r16] : 1.0f;
#pragma unroll
  for (int t = 0; t < TI; ++t) {
#pragma unroll
    for (int u = 0; u < TJ; ++u) {
      const int ar = r0 + (wm * TI + t) * 16 + 4 * jj;  // 4 consecutive A rows
      const int bc = c0 + (wn * TJ + u) * 16 + r16;     // one B row
      if (bc >= C) continue;
      float y[4];
      int32_t yi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (BS) {
          y[q] = acc[t][u][q];  // scaled step by step
        } else if constexpr (YT == 2) {
          yi[q] = (int32_t)acc[t][u][q];
        } else {
          // the token scale first, then the channel scale
          const float s1 = SIDE_X ? s_a[t][q] : s_b[u], s2 = SIDE_X ? s_b[u] : s_a[t][q];
          y[q] = __fmul_rn(__fmul_rn((float)acc[t][u][q], s1), s2);
        }
      }
      store_out<YT, SIDE_X>(Y, ldy, ar, bc, R, y, yi);
    }
  }
}

template <int AB, int YT, bool SIDE_X, bool BS = false>
__global__ __launch_bounds__(64 * NW, 1) void spgemm_kernel(int R, int C, int KS, const uint8_t* __restrict__ tv,
                                                            const uint8_t* __restrict__ tm, const uint8_t* __restrict__ bd,
                                                            int ldb, const float* __restrict__ sx,
                                                            const float* __restrict__ sw, void* __restrict__ Y, int ldy,
                                                            int tiles_r, int tiles_c) {
  spgemm_body<AB, YT, SIDE_X, BS>(R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, tiles_r, tiles_c);
}

// A batch of independent products of one shape (e.g. one per attention head): blockIdx.y selects the
// problem and every operand advances by its own stride (bytes for the tiled operand and the dense rows,
// elements for the scales and Y).
template <int AB, int YT, bool SIDE_X>
__global__ __launch_bounds__(64 * NW, 1) void spgemm_batched_kernel(
    int R, int C, int KS, const uint8_t* __restrict__ tv, int64_t s_tv, const uint8_t* __restrict__ tm, int64_t s_tm,
    const uint8_t* __restrict__ bd, int64_t s_bd, int ldb, const float* __restrict__ sx, int64_t s_sx,
    const float* __restrict__ sw, int64_t s_sw, void* __restrict__ Y, int64_t s_y, int ldy, int tiles_r, int tiles_c) {
  const int64_t b = blockIdx.y;
  constexpr int64_t YB = YT == 0 ? 2 : 4;  // output element bytes
  spgemm_body<AB, YT, SIDE_X, false>(R, C, KS, tv + b * s_tv, tm + b * s_tm, bd + b * s_bd, ldb,
                                     sx ? sx + b * s_sx : nullptr, sw ? sw + b * s_sw : nullptr,
                                     static_cast<uint8_t*>(Y) + b * s_y * YB, ldy, tiles_r, tiles_c);
}

template <int AB, int YT, bool SIDE_X>
hipError_t launch_batched(int batch, int R, int C, int KS, const uint8_t* tv, int64_t s_tv, const uint8_t* tm,
                          int64_t s_tm, const uint8_t* bd, int64_t s_bd, int ldb, const float* sx, int64_t s_sx,
                          const float* sw, int64_t s_sw, void* Y, int64_t s_y, int ldy, hipStream_t st) {
  auto kern = spgemm_batched_kernel<AB, YT, SIDE_X>;
  const hipError_t e = lds_limit((const void*)kern, LDS_SC);
  if (e != hipSuccess) return e;
  const int tr = (R + BM - 1) / BM, tc = (C + BN - 1) / BN;
  hipLaunchKernelGGL(kern, dim3(tr * tc, batch), dim3(64 * NW), LDS_SC, st, R, C, KS, tv, s_tv, tm, s_tm, bd, s_bd, ldb, sx,
                     s_sx, sw, s_sw, Y, s_y, ldy, tr, tc);
  return hipGetLastError();
}

template <int AB, int YT, bool SIDE_X, bool BS = false>
hipError_t launch(int R, int C, int KS, const uint8_t* tv, const uint8_t* tm, const uint8_t* bd, int ldb,
                  const float* sx, const float* sw, void* Y, int ldy, hipStream_t st) {
  auto kern = spgemm_kernel<AB, YT, SIDE_X, BS>;
  constexpr int lds = BS ? LDS_BS : LDS_SC;
  const hipError_t e = lds_limit((const void*)kern, lds);
  if (e != hipSuccess) return e;
  const int tr = (R + BM - 1) / BM, tc = (C + BN - 1) / BN;
  hipLaunchKernelGGL(kern, dim3(tr * tc), dim3(64 * NW), lds, st, R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, tr, tc);
  return hipGetLastError();
}

}  // namespace tiled


namespace decode {

constexpr int NW = 8;

// One workgroup per 16-row block of the sparse operand; NCT = 16-token column tiles (C <= 16 * NCT).
template <int AB, int YT, int NCT>
__global__ __launch_bounds__(64 * NW, 1) void decode_kernel(int R, int C, int KS, const uint8_t* __restrict__ tv,
                                                            const uint8_t* __restrict__ tm,
                                                            const uint8_t* __restrict__ bd, int ldb,
                                                            const float* __restrict__ sx,
                                                            const float* __restrict__ sw, void* __restrict__ Y,
                                                            int ldy) {
  using Acc = typename tiled::Mma<AB>::Acc;
  using MT = tiled::Meta<AB>;
  using MV = typename MT::V;
  __shared__ Acc red[NW][NCT][64];
  const int rb = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, jj = lane >> 4;
  const int KS4 = (KS + 3) / 4, KSP = 4 * KS4;
  const int g0 = KS4 * wave / NW, g1 = KS4 * (wave + 1) / NW;  // this wave's 4-step groups
  Acc acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = Acc{0, 0, 0, 0};
  if (g0 < g1) {
    const uint8_t* pa = tv + (int64_t)rb * KSP * 1024 + lane * 16;
    const uint8_t* pm = tm + (int64_t)rb * KS4 * MT::BLOCK + lane * (4 * MT::WB);
    const uint8_t* pb[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) pb[c] = bd + (int64_t)min(c * 16 + r16, C - 1) * ldb + 16 * jj;
    tiled::v4i A[4], B[4][NCT][2];
    MV mcur, mnxt;
    // padded steps (>= KS) hold zero values; their dense slices re-read step KS-1
    auto load_step = [&](int slot, int k) {
      const int kb = min(k, KS - 1);
      // the weights stream through once per call: non-temporal loads (1.04-1.10x at 1-16 tokens on
      // Qwen2.5-7B-shaped layers; the token rows, read by every workgroup, stay cached)
      A[slot] = __builtin_nontemporal_load(reinterpret_cast<const tiled::v4i*>(pa + (int64_t)k * 1024));
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        B[slot][c][0] = *reinterpret_cast<const tiled::v4i*>(pb[c] + (int64_t)kb * 128);
        B[slot][c][1] = *reinterpret_cast<const tiled::v4i*>(pb[c] + (int64_t)kb * 128 + 64);
      }
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) load_step(q, 4 * g0 + q);
    mcur = *reinterpret_cast<const MV*>(pm + (int64_t)g0 * MT::BLOCK);
    mnxt = *reinterpret_cast<const MV*>(pm + (int64_t)min(g0 + 1, KS4 - 1) * MT::BLOCK);
    for (int g = g0; g < g1; ++g) {
      const int kn = min(4 * (g + 1), KSP - 4);  // next group (re-read past the end, never used)
      auto one = [&](auto qc) {
        constexpr int Q = decltype(qc)::value;
#pragma unroll
        for (int c = 0; c < NCT; ++c) acc[c] = tiled::mma_step<AB, Q>(A[Q], B[Q][c][0], B[Q][c][1], acc[c], mcur);
        load_step(Q, kn + Q);
      };
      one(std::integral_constant<int, 0>{});
      one(std::integral_constant<int, 1>{});
      one(std::integral_constant<int, 2>{});
      one(std::integral_constant<int, 3>{});
      mcur = mnxt;
      mnxt = *reinterpret_cast<const MV*>(pm + (int64_t)min(g + 2, KS4 - 1) * MT::BLOCK);
    }
  }
#pragma unroll
  for (int c = 0; c < NCT; ++c) red[wave][c][lane] = acc[c];
  __syncthreads();
  if (wave < NCT) {
    const int c = wave;
    Acc s = red[0][c][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) s += red[w][c][lane];
    const int ar = rb * 16 + 4 * jj, bc = c * 16 + r16;
    if (bc < C) {
      float y[4];
      int32_t yi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (YT == 2) {
          yi[q] = (int32_t)s[q];
        } else {
          float f = (float)s[q];
          if (sx) f = __fmul_rn(f, sx[bc]);
          if (sw) f = __fmul_rn(f, sw[min(ar + q, R - 1)]);
          y[q] = f;
        }
      }
      store_out<YT, false>(Y, ldy, ar, bc, R, y, yi);
    }
  }
}

template <int AB, int YT>
hipError_t launch(int R, int C, int KS, const uint8_t* tv, const uint8_t* tm, const uint8_t* bd, int ldb,
                  const float* sx, const float* sw, void* Y, int ldy, hipStream_t st) {
  const int nrb = (R + 15) / 16;
  if (C <= 16)
    hipLaunchKernelGGL((decode_kernel<AB, YT, 1>), dim3(nrb), dim3(64 * NW), 0, st, R, C, KS, tv, tm, bd, ldb, sx, sw, Y,
                       ldy);
  else if (C <= 32)
    hipLaunchKernelGGL((decode_kernel<AB, YT, 2>), dim3(nrb), dim3(64 * NW), 0, st, R, C, KS, tv, tm, bd, ldb, sx, sw, Y,
                       ldy);
  else
    hipLaunchKernelGGL((decode_kernel<AB, YT, 4>), dim3(nrb), dim3(64 * NW), 0, st, R, C, KS, tv, tm, bd, ldb, sx, sw, Y,
                       ldy);
  return hipGetLastError();
}

// Few tokens, quant+lift fused in (SlideSparse blog section 3.2 fuses the lift into the quantisation; here
// both move into the product's prologue, which removes a launch and the X' round trip when the launches,
// not the bytes, dominate): every workgroup reads the M <= 4 bf16/f32 token rows itself, reduces their
// absmax, and writes their codes at the lifted positions X'[4(n-1)g + 4w + j] = q(X[2n g + 2w + j]) into
// LDS; then, persistent, it runs the row-block product for row blocks blockIdx.x, + gridDim.x, ...,
// reading the dense operand from LDS. Same arithmetic as quant_lift_kernel and decode_kernel<AB, YT, 1>
// (same per-wave K split and partial-sum order), so the results equal the two calls bit for bit.
constexpr int FMAXM = 4;  // tokens
// LDS bytes of the staging row of the lifts that gather from plain codes: K padded to whole 2n-groups,
// plus the word the last window's read reaches into, rounded to 16
__host__ __device__ inline int fused_stage_bytes(int64_t K, int n) {
  const int64_t kpad = (K + 2 * n - 1) / (2 * n) * (2 * n);
  if (n < 3) return (int)((kpad + 15) / 16 * 16);
  // the lift reads whole periods of its pattern: zeros past K through the last period's source bytes
  const int64_t nchunk = (kpad / (2 * n) * (n - 1) + 3) / 4, pc = lift_period_chunks(n);
  const int64_t need = (nchunk + pc - 1) / pc * lift_period_bytes(n);
  return (int)(((need > kpad ? need : kpad) + 15) / 16 * 16);
}
// The lifted row from a staged row of plain codes (zero past K through the last period's source bytes):
// nwin 4-byte windows, written as whole periods of 16-byte chunks.
template <int N>
__device__ __forceinline__ void lift_row(const uint8_t* st, uint8_t* row, int nwin, int tid) {
  using LP = LiftPeriod<N>;
  const int nchunk = (nwin + 3) / 4, nper = (nchunk + LP::PC - 1) / LP::PC;
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(st);
  for (int p = tid; p < nper; p += 64 * NW) {
    uint32_t s[LP::SW], o[4 * LP::PC];
#pragma unroll
    for (int i = 0; i < LP::SW; ++i) s[i] = s32[p * LP::SW + i];
    LP::emit(s, o);
#pragma unroll
    for (int h = 0; h < LP::PC; ++h) {
      const int c = p * LP::PC + h;
      if (c < nchunk)
        *reinterpret_cast<uint4*>(row + 16 * c) = make_uint4(o[4 * h], o[4 * h + 1], o[4 * h + 2], o[4 * h + 3]);
    }
  }
}
// 16-byte vectors of a token row held per thread: K <= 20480 (bf16) / 16384 (f32)
template <typename TIn> constexpr int fmaxv() { return sizeof(TIn) == 2 ? 5 : 8; }

template <int AB, int YT, typename TIn>
__global__ __launch_bounds__(64 * NW, 1) void fused_decode_kernel(int R, int M, int K, int n, int KS,
                                                                  const TIn* __restrict__ X, int64_t ldx,
                                                                  const uint8_t* __restrict__ tv,
                                                                  const uint8_t* __restrict__ tm,
                                                                  const float* __restrict__ sw, void* __restrict__ Y,
                                                                  int ldy, float* __restrict__ sx_out) {
  using Acc = typename tiled::Mma<AB>::Acc;
  using MT = tiled::Meta<AB>;
  using MV = typename MT::V;
  using Qz = Quant<AB == 1>;
  constexpr int E = 16 / (int)sizeof(TIn);  // elements per 16-byte vector
  constexpr int FMAXV = fmaxv<TIn>();
  extern __shared__ __align__(16) uint8_t xl[];  // [M][Kc] lifted codes, then (other lifts) a staging row
  __shared__ Acc red[NW][64];
  __shared__ float wmax[FMAXM][NW];
  __shared__ float s_x[FMAXM];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, jj = lane >> 4;
  const int Kc = KS * 128, nvec = K / E, tail0 = nvec * E;
  // n = 2 (no lift) and 6:8 from bf16 write the lifted codes straight from registers; other lifts stage
  // a token's plain codes in LDS and gather the windows from there (zero past K)
  const bool gather = !(n == 2 || (E == 8 && n == 4));
  const int Kpad = (K + 2 * n - 1) / (2 * n) * (2 * n);
  const int nwin = Kpad / (2 * n) * (n - 1);  // 4-byte windows of a lifted row
  uint8_t* st = xl + M * Kc;
  const int lds_bytes = M * Kc + (gather ? fused_stage_bytes(K, n) : 0);

  for (int o = tid * 16; o < lds_bytes; o += 64 * NW * 16) *reinterpret_cast<uint4*>(xl + o) = make_uint4(0, 0, 0, 0);
  auto elem = [&](const uint4& q, int e) -> float {
    if constexpr (E == 8) {
      const uint32_t w = (&q.x)[e >> 1];
      return bf16_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFF)));
    } else {
      return __uint_as_float((&q.x)[e]);
    }
  };
  // one token at a time, its row read twice (the absmax pass, then the codes; the second read hits the
  // cache), so few registers are live and four workgroups fit a CU, as for the row-block kernel
  for (int m = 0; m < M; ++m) {
    const TIn* xr = X + (int64_t)m * ldx;
    float tl = 0.0f;
    if (tail0 + tid < K) {
      if constexpr (E == 8) tl = bf16_to_f32(xr[tail0 + tid]);
      else tl = xr[tail0 + tid];
    }
    float a = fabsf(tl);
#pragma unroll
    for (int i = 0; i < FMAXV; ++i) {
      const int vi = tid + i * 64 * NW;
      if (vi < nvec) {
        const uint4 q = reinterpret_cast<const uint4*>(xr)[vi];
#pragma unroll
        for (int e = 0; e < E; ++e) a = fmaxf(a, fabsf(elem(q, e)));
      }
    }
    a = wave_max(a);
    if (lane == 0) wmax[m][wave] = a;
    __syncthreads();  // (the first one also orders the clearing of xl before the scatter below)
    a = wmax[m][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) a = fmaxf(a, wmax[m][w]);
    const bool zero = a == 0.0f;
    const float inv = zero ? 0.0f : Qz::Q / a;
    if (tid == 0) {
      const float sxm = zero ? 0.0f : a / Qz::Q;
      s_x[m] = sxm;
      if (sx_out && blockIdx.x == 0) sx_out[m] = sxm;
    }
    uint8_t* row = xl + m * Kc;
#pragma unroll 1
    for (int i = 0; i < FMAXV; ++i) {
      const int vi = tid + i * 64 * NW;
      if (vi >= nvec) continue;
      const uint4 q = reinterpret_cast<const uint4*>(xr)[vi];
      uint32_t c[E / 4];
#pragma unroll
      for (int h = 0; h < E / 4; ++h)
        c[h] = zero ? 0u : Qz::pack4(elem(q, 4 * h), elem(q, 4 * h + 1), elem(q, 4 * h + 2), elem(q, 4 * h + 3), inv);
      if (E == 8 && n == 4) {  // one 8-group: windows are bytes 0-3, 2-5, 4-7 of its codes
        uint32_t* o = reinterpret_cast<uint32_t*>(row + vi * 12);
        o[0] = c[0];
        o[1] = (c[0] >> 16) | (c[E / 4 - 1] << 16);
        o[2] = c[E / 4 - 1];
      } else {  // plain codes: the row itself (n = 2) or the staging row
        uint8_t* dst = gather ? st : row;
#pragma unroll
        for (int h = 0; h < E / 4; ++h) *reinterpret_cast<uint32_t*>(dst + vi * E + 4 * h) = c[h];
      }
    }
    if (tail0 + tid < K) {  // at most E - 1 elements past the last whole vector
      const uint8_t code = zero ? 0 : Qz::code(tl, inv);
      if (gather) {
        st[tail0 + tid] = code;
      } else if (n == 2) {
        row[tail0 + tid] = code;
      } else {  // 6:8: element k = 8g + r lies in the windows w = (r-2)/2 .. r/2 of 0..2, at 12g + r + 2w
        const int k = tail0 + tid, g = k >> 3, r = k & 7;
        for (int w = r >= 3 ? (r - 2) >> 1 : 0; w <= min(r >> 1, 2); ++w) row[12 * g + r + 2 * w] = code;
      }
    }
    if (gather) {
      __syncthreads();  // the staged codes are complete (the next token's first barrier guards their reuse)
      // whole periods of the lift pattern per thread (LiftPeriod), written into the token's LDS row
      switch (n) {
        case 3: lift_row<3>(st, row, nwin, tid); break;
        case 5: lift_row<5>(st, row, nwin, tid); break;
        case 4: lift_row<4>(st, row, nwin, tid); break;
        case 6: lift_row<6>(st, row, nwin, tid); break;
        case 7: lift_row<7>(st, row, nwin, tid); break;
        default: lift_row<8>(st, row, nwin, tid); break;
      }
    }
  }
  __syncthreads();

  // the row-block product (decode_kernel with one 16-token column tile), dense operand from LDS
  const int KS4 = (KS + 3) / 4, KSP = 4 * KS4, nrb = (R + 15) / 16;
  const int g0 = KS4 * wave / NW, g1 = KS4 * (wave + 1) / NW;
  for (int rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
  Acc acc = Acc{0, 0, 0, 0};
  // the epilogue's channel scales (wave 0 writes the block), loaded before the product
  float esw[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  if (YT != 2 && wave == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) esw[q] = sw[min(rb * 16 + 4 * jj + q, R - 1)];
  }
  if (g0 < g1) {
    const uint8_t* pa = tv + (int64_t)rb * KSP * 1024 + lane * 16;
    const uint8_t* pm = tm + (int64_t)rb * KS4 * MT::BLOCK + lane * (4 * MT::WB);
    const SS_LDS uint8_t* pb = (const SS_LDS uint8_t*)xl + min(r16, M - 1) * Kc + 16 * jj;
    tiled::v4i A[4], B[4][2];
    MV mcur, mnxt;
    auto load_step = [&](int slot, int k) {
      const int kb = min(k, KS - 1);
      A[slot] = __builtin_nontemporal_load(reinterpret_cast<const tiled::v4i*>(pa + (int64_t)k * 1024));
      B[slot][0] = *reinterpret_cast<const SS_LDS tiled::v4i*>(pb + kb * 128);
      B[slot][1] = *reinterpret_cast<const SS_LDS tiled::v4i*>(pb + kb * 128 + 64);
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) load_step(q, 4 * g0 + q);
    mcur = *reinterpret_cast<const MV*>(pm + (int64_t)g0 * MT::BLOCK);
    mnxt = *reinterpret_cast<const MV*>(pm + (int64_t)min(g0 + 1, KS4 - 1) * MT::BLOCK);
    for (int g = g0; g < g1; ++g) {
      const int kn = min(4 * (g + 1), KSP - 4);
      auto one = [&](auto qc) {
        constexpr int Q = decltype(qc)::value;
        acc = tiled::mma_step<AB, Q>(A[Q], B[Q][0], B[Q][1], acc, mcur);
        load_step(Q, kn + Q);
      };
      one(std::integral_constant<int, 0>{});
      one(std::integral_constant<int, 1>{});
      one(std::integral_constant<int, 2>{});
      one(std::integral_constant<int, 3>{});
      mcur = mnxt;
      mnxt = *reinterpret_cast<const MV*>(pm + (int64_t)min(g + 2, KS4 - 1) * MT::BLOCK);
    }
  }
  // Wait states between the last smfmac and the LDS store that reads its result: inside this row-block
  // loop the compiler emitted the store right after the loop's exit branch with none (the smfmac result
  // is not readable by a DS instruction for several cycles), so they are written out here.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    Acc sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += red[w][lane];
    const int ar = rb * 16 + 4 * jj, bc = r16;
    if (bc < M) {
      float y[4];
      int32_t yi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (YT == 2) {
          yi[q] = (int32_t)sum[q];
        } else {
          float f = (float)sum[q];
          f = __fmul_rn(f, s_x[bc]);
          f = __fmul_rn(f, esw[q]);
          y[q] = f;
        }
      }
      store_out<YT, false>(Y, ldy, ar, bc, R, y, yi);
    }
  }
  __syncthreads();  // red is rewritten by the next row block
  }
}

}  // namespace decode

// Split-K product for a few tokens (side W, C <= 64). A workgroup of 8 waves
// takes 8 row blocks (128 rows) and one range of K: every step, each wave
// brings its own row block's 1 KB of values and one 8-row x 128-byte block of
// the dense operand (whole lines, XOR-swizzled as in the tiled kernel) into a
// ring of LDS stages, so the 64 token rows of a step come from L2 once per
// workgroup instead of once per wave, and the kernel streams the sparse values
// at HBM rate. Each workgroup writes its partial tile (int32 for INT8, float
// otherwise) to a workspace [split][C][RP]; a second kernel sums the splits in
// order and applies the epilogue (INT8 stays exact).
namespace splitk {

constexpr int NW = 8, S = 4, BROWS = 64;
constexpr int A_BYTES = NW * 1024, STAGE = A_BYTES + BROWS * 128, LDS = S * STAGE;  // 16 KB stages, 64 KB
constexpr int LPW = 2;  // LDS DMA loads per wave per step: own value block + one dense block

template <int AB, int NCT>
__global__ __launch_bounds__(64 * NW, 4) void splitk_kernel(int R, int C, int KS, int GPS, const uint8_t* __restrict__ tv,
                                                            const uint8_t* __restrict__ tm,
                                                            const uint8_t* __restrict__ bd, int ldb,
                                                            void* __restrict__ ws, int RP) {
  using Acc = typename tiled::Mma<AB>::Acc;
  using MT = tiled::Meta<AB>;
  using MV = typename MT::V;
  using tiled::v4i;
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, jj = lane >> 4;
  const int nrb = (R + 15) / 16, KS4 = (KS + 3) / 4, KSP = 4 * KS4;
  const int sp = blockIdx.y;
  const int g0 = sp * GPS, ng = min(KS4, g0 + GPS) - g0;  // this split's 4-step groups (ng >= 1)
  const int k0 = 4 * g0, nst = 4 * ng;
  const int rbw = blockIdx.x * NW + wave;  // this wave's row block
  const int rb = min(rbw, nrb - 1);        // clamped: in bounds, results not stored
  const uint8_t* pa = tv + (int64_t)rb * KSP * 1024 + lane * 16;
  const uint8_t* pm = tm + (int64_t)rb * KS4 * MT::BLOCK + lane * (4 * MT::WB);
  const int brow = 8 * wave + (lane >> 3);  // dense rows past C re-read row C-1 (never stored)
  const uint32_t offb = (uint32_t)min(brow, C - 1) * (uint32_t)ldb + tiled::swz(lane & 7, brow & 15) * 16;

  // local step i -> slot i % S; past the range the last step is re-read (in bounds, never consumed)
  auto issue = [&](int i) {
    SS_LDS uint8_t* base = (SS_LDS uint8_t*)smem + (i % S) * STAGE;
    const int k = k0 + min(i, nst - 1), kb = min(k, KS - 1);
    // the weights stream through once per call: non-temporal (cache-policy bit 2, `nt` in the assembly;
    // 1.01-1.04x at 32-64 tokens), the token rows stay cached
    __builtin_amdgcn_global_load_lds((const void*)(pa + (int64_t)k * 1024), (SS_LDS void*)(base + wave * 1024), 16, 0, 2);
    __builtin_amdgcn_global_load_lds((const void*)(bd + offb + (uint32_t)kb * 128),
                                     (SS_LDS void*)(base + A_BYTES + wave * 1024), 16, 0, 0);
  };
  MV mcur, mnxt;
  auto load_meta = [&](MV& m, int g) { m = *reinterpret_cast<const MV*>(pm + (int64_t)g * MT::BLOCK); };
  struct Frag {
    v4i a;
    v4i b[NCT][2];
  };
  auto read = [&](Frag& f, int i) {
    const uint8_t* st = smem + (i % S) * STAGE;
    f.a = *reinterpret_cast<const v4i*>(st + wave * 1024 + lane * 16);
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const uint8_t* bb = st + A_BYTES + (2 * c + (r16 >> 3)) * 1024 + (r16 & 7) * 128;
      f.b[c][0] = *reinterpret_cast<const v4i*>(bb + tiled::swz(jj, r16) * 16);
      f.b[c][1] = *reinterpret_cast<const v4i*>(bb + tiled::swz(4 + jj, r16) * 16);
    }
  };
  Acc acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = Acc{0, 0, 0, 0};
  auto mma = [&](const Frag& f, auto qc) {
    constexpr int Q = decltype(qc)::value;
#pragma unroll
    for (int c = 0; c < NCT; ++c) acc[c] = tiled::mma_step<AB, Q>(f.a, f.b[c][0], f.b[c][1], acc[c], mcur);
  };
  // stage i+1 landed: outstanding loads = the S-3 later stages plus an index group issued since (one per
  // group, at its first step, except in the last group)
  auto wait_next = [&](auto qc, auto lastc) {
    constexpr int Q = decltype(qc)::value;
    constexpr bool LAST = decltype(lastc)::value;
    constexpr int lo = Q + 6 - S, hi = Q + 3;
    constexpr int nm = LAST ? 0 : (hi >= 4 && lo <= 4 ? 1 : 0) + (hi >= 8 && lo <= 8 ? 1 : 0);
    constexpr int N = (S - 3) * LPW + nm;
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  };
  auto step = [&](int j, auto qc, auto lastc, Frag& cur, Frag& nxt) {
    constexpr int Q = decltype(qc)::value;
    constexpr bool LAST = decltype(lastc)::value;
    __builtin_amdgcn_sched_barrier(0);
    wait_next(qc, lastc);
    __builtin_amdgcn_s_barrier();  // stage j+1 landed for every wave; slot (j-1) % S is free
    __builtin_amdgcn_sched_barrier(0);
    issue(j + S - 1);
    if (Q == 0 && !LAST) load_meta(mnxt, g0 + j / 4 + 1);
    __builtin_amdgcn_sched_barrier(0);
    read(nxt, j + 1);
    mma(cur, qc);
    __builtin_amdgcn_sched_barrier(0);
  };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
  load_meta(mcur, g0);
#pragma unroll
  for (int i = 0; i < S - 1; ++i) issue(i);
  Frag f0, f1;
  {
    constexpr int N = (S - 2) * LPW;  // stage 0 landed
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read(f0, 0);
  for (int g = 0; g + 1 < ng; ++g) {
    const int j = 4 * g;
    step(j, Q0{}, std::false_type{}, f0, f1);
    step(j + 1, Q1{}, std::false_type{}, f1, f0);
    step(j + 2, Q2{}, std::false_type{}, f0, f1);
    step(j + 3, Q3{}, std::false_type{}, f1, f0);
    mcur = mnxt;
  }
  {
    const int j = nst - 4;
    step(j, Q0{}, std::true_type{}, f0, f1);
    step(j + 1, Q1{}, std::true_type{}, f1, f0);
    step(j + 2, Q2{}, std::true_type{}, f0, f1);
    mma(f1, Q3{});
  }
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // no load may outlive the workgroup
  if (rbw < nrb) {
    const int ar = rb * 16 + 4 * jj;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int bc = c * 16 + r16;
      if (bc < C) {
        int32_t* o = static_cast<int32_t*>(ws) + ((int64_t)sp * C + bc) * RP + ar;
        if constexpr (AB == 0)
          *reinterpret_cast<int4*>(o) = make_int4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
        else
          *reinterpret_cast<float4*>(o) = make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
      }
    }
  }
}

// Sum the splits in order (exact for int32) and apply the epilogue: one thread per 4 rows of one token.
template <int AB, int YT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(int R, int C, int RP, int splits,
                                                            const void* __restrict__ ws, const float* __restrict__ sx,
                                                            const float* __restrict__ sw, void* __restrict__ Y,
                                                            int ldy) {
  const int quads = RP / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int bc = (int)(idx / quads), ar = (int)(idx % quads) * 4;
  if (bc >= C || ar >= R) return;
  float y[4];
  int32_t yi[4];
  if constexpr (AB == 0) {
    int4 s = make_int4(0, 0, 0, 0);
    for (int p = 0; p < splits; ++p) {
      const int4 v = *reinterpret_cast<const int4*>(static_cast<const int32_t*>(ws) + ((int64_t)p * C + bc) * RP + ar);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    yi[0] = s.x; yi[1] = s.y; yi[2] = s.z; yi[3] = s.w;
  } else {
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int p = 0; p < splits; ++p) {
      const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(ws) + ((int64_t)p * C + bc) * RP + ar);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    y[0] = s.x; y[1] = s.y; y[2] = s.z; y[3] = s.w;
  }
  if constexpr (YT != 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float f = AB == 0 ? (float)yi[q] : y[q];
      if (sx) f = __fmul_rn(f, sx[bc]);
      if (sw) f = __fmul_rn(f, sw[min(ar + q, R - 1)]);
      y[q] = f;
    }
  }
  store_out<YT, false>(Y, ldy, ar, bc, R, y, yi);
}

struct Plan {
  int splits = 0, gps = 0, rp = 0;
  int64_t bytes = 0;
};

// Split count: at most one workgroup per CU over (row groups x splits) -- a CU holding two would
// finish last at half speed -- with whole 4-step groups per split.
inline Plan plan(int64_t R, int64_t C, int64_t KS) {
  Plan p;
  const int64_t nrb = (R + 15) / 16, nrg = (nrb + NW - 1) / NW, ks4 = (KS + 3) / 4;
  int64_t sk = (int64_t)num_cus_p() / nrg;
  sk = std::max<int64_t>(1, std::min<int64_t>(sk, ks4));
  p.gps = (int)((ks4 + sk - 1) / sk);
  p.splits = (int)((ks4 + p.gps - 1) / p.gps);
  p.rp = (int)(nrb * 16);
  p.bytes = (int64_t)p.splits * C * p.rp * 4;
  return p;
}

template <int AB, int YT>
hipError_t launch(int R, int C, int KS, const uint8_t* tv, const uint8_t* tm, const uint8_t* bd, int ldb,
                  const float* sx, const float* sw, void* Y, int ldy, void* ws, hipStream_t st) {
  const Plan p = plan(R, C, KS);
  const int nrg = ((R + 15) / 16 + NW - 1) / NW;
  const dim3 grid((unsigned)nrg, (unsigned)p.splits);
  auto go = [&](auto kern) -> hipError_t {
    const hipError_t a = lds_limit((const void*)kern, LDS);
    if (a != hipSuccess) return a;
    hipLaunchKernelGGL(kern, grid, dim3(64 * NW), LDS, st, R, C, KS, p.gps, tv, tm, bd, ldb, ws, p.rp);
    return hipGetLastError();
  };
  hipError_t e = C <= 16 ? go(splitk_kernel<AB, 1>) : C <= 32 ? go(splitk_kernel<AB, 2>) : go(splitk_kernel<AB, 4>);
  if (e != hipSuccess) return e;
  const int64_t threads = (int64_t)C * (p.rp / 4);
  hipLaunchKernelGGL((splitk_reduce_kernel<AB, YT>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, R, C, p.rp,
                     p.splits, (const void*)ws, sx, sw, Y, ldy);
  return hipGetLastError();
}

}  // namespace splitk

int64_t tiled_vals_bytes(int64_t rows, int64_t Kc, int es) {
  const int64_t ks4 = (Kc * es / 128 + 3) / 4;
  return (rows + 15) / 16 * ks4 * 4 * 1024;
}

int64_t tiled_meta_bytes(int64_t rows, int64_t Kc, int es) {
  const int64_t ks4 = (Kc * es / 128 + 3) / 4;
  return (rows + 15) / 16 * ks4 * 256 * (4 / es);
}

hipError_t launch_pack_tiled(int es, const uint8_t* vals, int64_t ldv_bytes, const uint8_t* meta, int64_t ldm,
                             int64_t rows, int64_t Kc, uint8_t* tv, uint8_t* tm, hipStream_t st) {
  const int KS = (int)(Kc * es / 128), KS4 = (KS + 3) / 4, nrb = (int)((rows + 15) / 16);
  if (es == 1)
    hipLaunchKernelGGL(tiled::pack_kernel<1>, dim3(KS4, (nrb + 3) / 4), dim3(256), 0, st, vals, ldv_bytes, meta, ldm,
                       (int)rows, KS, KS4, nrb, tv, tm);
  else
    hipLaunchKernelGGL(tiled::pack_kernel<2>, dim3(KS4, (nrb + 3) / 4), dim3(256), 0, st, vals, ldv_bytes, meta, ldm,
                       (int)rows, KS, KS4, nrb, tv, tm);
  return hipGetLastError();
}

// Few tokens on the weight-sparse side and too few 256-row tiles to fill the chip.
static bool few_tokens(bool side_x, int64_t R, int64_t C) {
  const int64_t tiles = ((R + tiled::BM - 1) / tiled::BM) * ((C + tiled::BN - 1) / tiled::BN);
  return !side_x && C <= 64 && (C <= 8 || tiles < 128);
}
// The wide-wave prefill kernel (k_spgemm_wide.hip) on the weight-sparse side: 256 x 256 tiles wherever they
// still give every CU four or more (measured 1.07-1.3x this file's 256 x 128 kernel on the Llama-shaped layers
// at 16384 tokens and on gate_up at 4096), for reductions longer than 64 steps from 0.6 of one per CU, and
// from two per CU when they fill whole rounds of CUs (below), else its 256 x 128 form with two workgroups per
// CU wherever that gives a CU more than one tile (1.06-1.34x this file's kernel from 384 to 900 tiles on those layers at 512-8192
// tokens; with one tile per CU or fewer, this file's eight waves per tile win). Its buffer loads take 32-bit
// offsets, so each operand stays below 2 GB. The sparse-activation side takes the 256 x 128 form under the
// same rule (1.2x this file's kernel on an 8192 x 4096 x 4096 product). Returns the tile width, or 0 for this
// file's kernel.
static int wide_bn(bool side_x, int64_t R, int64_t C, int64_t KS, int64_t ldb_bytes) {
  const int64_t sparse_bytes = (R + 15) / 16 * ((KS + 3) / 4 * 4) * 1024, dense_bytes = C * ldb_bytes;
  if (sparse_bytes >= (INT64_C(1) << 31) || dense_bytes >= (INT64_C(1) << 31)) return 0;
  const int64_t cus = num_cus_p(), t256 = ((R + 255) / 256) * ((C + 255) / 256);
  if (!side_x && t256 >= 4 * cus) return 256;
  // Reductions longer than 64 steps amortise a tile's prologue and epilogue, so 256 x 256 tiles pay from
  // 0.6 of a tile per CU on: against the 256 x 128 form, Llama-shaped down (K = 14336, 2:4 and 6:8) measured
  // 1.07-1.09x at 2560-3072 tokens, 1.07-1.27x at 4096, 1.19-1.26x at 6144-12288, the Qwen-shaped 4:6 and
  // 8:10 down at 4096 tokens 1.10-1.12x; at half a tile per CU (2048 tokens) 0.88x.
  if (!side_x && KS > 64 && 5 * t256 >= 3 * cus) return 256;
  // Shorter reductions: from two tiles per CU when the last round of tiles fills 90% of the CUs or more
  // (o and qkv at 8192 and 12288 tokens, 512-768 tiles: 1.017-1.037x the 256 x 128 form, the 6:8 o at 8192
  // tokens 1.03x; gate_up at 2048 tokens, 896 tiles, 0.98x).
  if (!side_x && t256 >= 2 * cus && 10 * t256 >= 9 * ((t256 + cus - 1) / cus) * cus) return 256;
  if (((R + 255) / 256) * ((C + 127) / 128) > cus) return 128;
  return 0;
}
// The split-K path (with a workspace) serves the few-token products with more than 16 tokens.
static bool use_splitk(bool side_x, int64_t R, int64_t C) { return few_tokens(side_x, R, C) && C > 16; }

hipError_t launch_spgemm_tiled_batched(bool side_x, int ab, int yt, int64_t batch, int64_t R, int64_t C, int64_t Kc,
                                       const uint8_t* tv, int64_t s_tv, const uint8_t* tm, int64_t s_tm, const void* bd,
                                       int64_t ldb_bytes, int64_t s_bd, const float* sx, int64_t s_sx, const float* sw,
                                       int64_t s_sw, void* Y, int64_t ldy, int64_t s_y, hipStream_t st) {
  const uint8_t* b = static_cast<const uint8_t*>(bd);
  const int bt = (int)batch, r = (int)R, c = (int)C, ks = (int)(Kc * (ab == 2 ? 2 : 1) / 128), lb = (int)ldb_bytes,
            ly = (int)ldy;
#define SS_TB(AB_, YT_)                                                                                                 \
  return side_x ? tiled::launch_batched<AB_, YT_, true>(bt, r, c, ks, tv, s_tv, tm, s_tm, b, s_bd, lb, sx, s_sx, sw,     \
                                                        s_sw, Y, s_y, ly, st)                                           \
                : tiled::launch_batched<AB_, YT_, false>(bt, r, c, ks, tv, s_tv, tm, s_tm, b, s_bd, lb, sx, s_sx, sw,    \
                                                         s_sw, Y, s_y, ly, st)
  if (ab == 0) {
    if (yt == 0) SS_TB(0, 0);
    if (yt == 1) SS_TB(0, 1);
    SS_TB(0, 2);
  }
  if (ab == 1) {
    if (yt == 0) SS_TB(1, 0);
    SS_TB(1, 1);
  }
  if (yt == 0) SS_TB(2, 0);
  SS_TB(2, 1);
#undef SS_TB
}

hipError_t launch_spgemm_tiled_block(int yt, int64_t R, int64_t C, int64_t Kc, const uint8_t* tv, const uint8_t* tm,
                                     const void* bd, int64_t ldb_bytes, const float* sx, const float* sw, void* Y,
                                     int64_t ldy, hipStream_t st) {
  const uint8_t* b = static_cast<const uint8_t*>(bd);
  const int r = (int)R, c = (int)C, ks = (int)(Kc / 128), lb = (int)ldb_bytes, ly = (int)ldy;
  if (yt == 0) return tiled::launch<1, 0, false, true>(r, c, ks, tv, tm, b, lb, sx, sw, Y, ly, st);
  return tiled::launch<1, 1, false, true>(r, c, ks, tv, tm, b, lb, sx, sw, Y, ly, st);
}

bool quant_lift_spgemm_fits(bool x_bf16, int64_t M, int64_t K, int64_t Kc) {
  const int64_t max_k = x_bf16 ? 8 * decode::fmaxv<uint16_t>() * 64 * decode::NW : 4 * decode::fmaxv<float>() * 64 * decode::NW;
  return M >= 1 && M <= decode::FMAXM && M * Kc <= 131072 && K <= max_k;
}

hipError_t launch_quant_lift_spgemm(bool x_bf16, int ab, int yt, const void* X, int64_t ldx, int64_t M, int64_t K, int n,
                                    int64_t N, int64_t Kc, const uint8_t* tv, const uint8_t* tm, const float* sw,
                                    void* Y, int64_t ldy, float* sx_out, hipStream_t st) {
  const int R = (int)N, m = (int)M, k = (int)K, ks = (int)(Kc / 128), ly = (int)ldy;
  const bool gather = !(n == 2 || (x_bf16 && n == 4));  // as in the kernel
  const size_t lds = (size_t)(M * Kc) + (gather ? (size_t)decode::fused_stage_bytes(K, n) : 0);
  // persistent, two workgroups a CU where the LDS holds two (each quantises the tokens once; measured
  // against one row block per workgroup and against up to four a CU, equal or faster on every shape)
  const int64_t per_cu = 2 * (int64_t)(lds + 9 * 1024) <= 160 * 1024 ? 2 : 1;
  const int64_t nrb = (N + 15) / 16;
  const unsigned grid = (unsigned)std::min<int64_t>(nrb, per_cu * num_cus_p());
  auto go = [&](auto kern, const auto* x) -> hipError_t {
    const hipError_t e = lds_limit((const void*)kern, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * decode::NW), lds, st, R, m, k, n, ks, x, ldx, tv, tm, sw, Y, ly,
                       sx_out);
    return hipGetLastError();
  };
  const uint16_t* xb = static_cast<const uint16_t*>(X);
  const float* xf = static_cast<const float*>(X);
#define SS_FD(AB_, YT_) \
  return x_bf16 ? go(decode::fused_decode_kernel<AB_, YT_, uint16_t>, xb) : go(decode::fused_decode_kernel<AB_, YT_, float>, xf)
  if (ab == 0) {
    if (yt == 0) SS_FD(0, 0);
    if (yt == 1) SS_FD(0, 1);
    SS_FD(0, 2);
  }
  if (yt == 0) SS_FD(1, 0);
  SS_FD(1, 1);
#undef SS_FD
}

int64_t spgemm_tiled_workspace_bytes(bool side_x, int ab, int64_t R, int64_t C, int64_t Kc) {
  if (!use_splitk(side_x, R, C)) return 0;
  return splitk::plan(R, C, Kc * (ab == 2 ? 2 : 1) / 128).bytes;
}

hipError_t launch_spgemm_tiled(bool side_x, int ab, int yt, int64_t R, int64_t C, int64_t Kc, const uint8_t* tv,
                               const uint8_t* tm, const void* bd, int64_t ldb_bytes, const float* sx, const float* sw,
                               void* Y, int64_t ldy, void* ws, hipStream_t st) {
  const uint8_t* b = static_cast<const uint8_t*>(bd);
  const int r = (int)R, c = (int)C, ks = (int)(Kc * (ab == 2 ? 2 : 1) / 128), lb = (int)ldb_bytes, ly = (int)ldy;
  // few tokens: split-K when a workspace is given and the problem uses one, else the row-block decode kernel
  const bool dec = few_tokens(side_x, R, C);
  const bool spk = ws != nullptr && use_splitk(side_x, R, C);
  const int bn = spk || dec ? 0 : wide_bn(side_x, R, C, ks, ldb_bytes);
  if (bn) return launch_spgemm_wide(bn, side_x, ab, yt, r, c, ks, tv, tm, b, lb, sx, sw, Y, ly, st);
#define SS_TL(AB_, YT_)                                                                                   \
  return spk      ? splitk::launch<AB_, YT_>(r, c, ks, tv, tm, b, lb, sx, sw, Y, ly, ws, st)               \
         : dec    ? decode::launch<AB_, YT_>(r, c, ks, tv, tm, b, lb, sx, sw, Y, ly, st)                   \
         : side_x ? tiled::launch<AB_, YT_, true>(r, c, ks, tv, tm, b, lb, sx, sw, Y, ly, st)               \
                  : tiled::launch<AB_, YT_, false>(r, c, ks, tv, tm, b, lb, sx, sw, Y, ly, st)
  if (ab == 0) {
    if (yt == 0) SS_TL(0, 0);
    if (yt == 1) SS_TL(0, 1);
    SS_TL(0, 2);
  }
  if (ab == 1) {
    if (yt == 0) SS_TL(1, 0);
    SS_TL(1, 1);
  }
  if (yt == 0) SS_TL(2, 0);
  SS_TL(2, 1);
#undef SS_TL
}

}  // namespace ss
