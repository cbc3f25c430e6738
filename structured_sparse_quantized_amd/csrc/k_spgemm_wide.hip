// Wide-tile prefill product on the tiled sparse operand (gfx950 v_smfmac), with the per-token x
// per-channel rescale epilogue. Deep reading of arXiv 2610.28947 (introduction: one operand keeps two of
// every four along the accumulate axis; section 3.1: sparse W or sparse X); LLM Compressor W8A8 scales.
//
// C[r][c] = sum_k A[r][k] B[c][k]; A = the tiled compressed operand (rows r), B = the dense operand (rows c),
// as in the 256 x 128 product of k_spgemm_tiled.hip, whose tiled layout this kernel reads unchanged.
//
// Why wide waves: a 16x16x128 sparse instruction does the work of a dense 16x16x128 one in half the
// matrix-core cycles, so per cycle it needs twice the operand bytes; waves of 128 A rows read fewer LDS bytes
// per operation than waves of 64. Waves are 128 A rows tall, two along A and W / 2 along B; three forms:
//  * BN = 256 (256 x 256 tiles): a 256 x 256 tile moves 48 KB of operands (16 KB of compressed A values,
//    32 KB of dense B rows) into LDS per 128-position step for 16.8 M dense-equivalent operations, 25% fewer
//    L2 -> LDS bytes per operation than 256 x 128. LDS: a ring of three 48 KB stages and the 16 KB
//    index-word slot (160 KB), so one workgroup per CU. Two wave layouts:
//    - W = 4 (one wave per SIMD): waves of 128 x 128 = 8 x 8 instructions per step, the 256 accumulators
//      per lane in the accumulation registers, A fragments double-buffered in registers. The fewest LDS
//      bytes read per operation; taken for long reductions.
//    - W = 8 (two waves per SIMD): waves of 128 x 64 = 8 x 4 instructions per step (243 registers). A third
//      more LDS bytes read per step, but one wave's waits in the prologue and epilogue overlap the other's
//      work, which pays where those are a large share of a tile (short reductions).
//  * BN = 128, W = 4: 256 x 128 tiles, waves of 128 x 64 (128 accumulators per lane, 245 registers in all); a
//    ring of two 32 KB stages and the index-word slot (80 KB), so two workgroups share a CU and the prologue
//    and epilogue of one overlap the other's instructions. For problems with more than one such tile per CU
//    but too few 256 x 256 tiles to keep every CU busy.
// Waves of 128 x 64 refill their A fragments right after their last use (the step's last column).
// LDS stages are filled by LDS DMA (buffer loads into LDS, 1 KB per wave instruction; B rows swizzled so
// fragment reads are conflict-free); the index-word slot holds the current 4-step group's index words (the
// tiled layout's metadata block of each of the 16 row blocks, brought in by DMA one group ahead and read into
// registers after the last instruction of the group before) and takes the tile's epilogue scales during the
// last group. B fragments are refilled column by column of B.
// Synchronisation: one barrier per step. At the top of step j every wave waits until its own loads of
// stage j+1 have landed (loads complete in issue order, so this is a wait for a fixed count of later
// loads) and its own LDS reads are done, then the barrier makes stage j+1 visible and frees the slot of
// stage j (read during step j-1), into which stage j+S (S stages in the ring) is loaded during step j, spread
// over the step's columns (with one wave per SIMD, a run of loads would leave the matrix core idle while it
// issues: spreading them was 6-13% faster than issuing the stage at the top of the step).
#include <algorithm>

#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_mma.h"
#include "ss_store.h"

namespace ss {
namespace wide {

using tiled::Meta;
using tiled::Mma;
using tiled::swz;
using tiled::v4i;
#define SS_LDS __attribute__((address_space(3)))

constexpr int BM = 256, TI = 8;  // A rows per tile, A blocks per wave (waves are 128 A rows tall, two along A)
constexpr int RBT = BM / 16;     // row blocks of the sparse operand per tile
constexpr int A_BYTES = BM * 64; // 16 KB of compressed A values per step
constexpr int NSC = 2;           // scale loads per wave (A rows, B rows)
constexpr int TJMAX = 8, PAMAX = 4;

// BN: tile width along B; W: waves per workgroup (2 along A, W / 2 along B)
template <int BN, int W> struct Shape {
  static constexpr int NW = W, WGN = W / 2;
  static constexpr int TJ = BN / 16 / WGN;        // B blocks per wave: 8 x TJ instructions per step
  static constexpr int PA = RBT / NW;             // A loads per wave per step (1 KB each)
  static constexpr int PB = BN / 8 / NW;          // B loads per wave per step (8 rows x 128 bytes each)
  static constexpr int LPW = PA + PB;
  static constexpr int STAGE = A_BYTES + BN * 128;
  static constexpr int S = BN == 256 ? 3 : 2;     // stages in the ring
  static constexpr int META = S * STAGE;          // index-word slot (then the epilogue scales)
  static constexpr bool ADB = TJ == 8;            // A fragments double-buffered
  static constexpr int SLOTS = ADB ? 2 : 3;       // loads per column
  static_assert(PA * NW * 16 == BM && PB * NW * 8 == BN && TJ <= TJMAX && PA <= PAMAX, "load split");
  static_assert((BM + BN) * 4 <= 8 * 1024, "the epilogue scales fit the index-word slot");
};
template <int BN> constexpr int occupancy() { return BN == 256 ? 1 : 2; }  // workgroups per CU
template <int AB> constexpr int meta_slot() { return RBT * Meta<AB>::BLOCK; }    // 16 KB / 8 KB
template <int AB, int NW> constexpr int mpw() { return meta_slot<AB>() / 1024 / NW; }   // meta loads per wave
template <int BN, int W, int AB> constexpr int lds_bytes() { return Shape<BN, W>::META + meta_slot<AB>(); }
constexpr int up_rows(int tj, int cap) { return tj > cap && tj > 1 ? up_rows(tj / 2, cap) : tj; }

constexpr int vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }  // s_waitcnt vmcnt(n)

// raw buffer resource over [p, p + bytes): base and size in scalar registers, 32-bit untyped data
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// (arrays that the loads index have fixed lengths: a length that depends on a template parameter in these
// calls drops the kernel's host launch stub without a diagnostic)
template <int BN, int W, int AB, int YT, bool SX, int GR>
__global__ __launch_bounds__(64 * W, occupancy<BN>()) void wide_kernel(
    int R, int C, int KS, const uint8_t* __restrict__ tv, const uint8_t* __restrict__ tm, const uint8_t* __restrict__ bd,
    int ldb, const float* __restrict__ sx, const float* __restrict__ sw, void* __restrict__ Y, int ldy, int tiles_r,
    int tiles_c) {
  using SH = Shape<BN, W>;
  constexpr int TJ = SH::TJ, PA = SH::PA, PB = SH::PB, LPW = SH::LPW, STAGE = SH::STAGE, S = SH::S, META = SH::META;
  constexpr int NW = SH::NW, WGN = SH::WGN;
  using Acc = typename Mma<AB>::Acc;
  using MT = Meta<AB>;
  using MV = typename MT::V;
  constexpr int MPW = mpw<AB, NW>();
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int r16 = lane & 15, jj = lane >> 4;

  // Tile order: workgroups are dealt to the 8 XCDs round-robin; each XCD takes a contiguous run of tiles,
  // walked in groups of GR A-row tiles, so the tiles that share operands also share an L2.
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int group = bid / (GR * tiles_c), first_r = group * GR, gsize = min(tiles_r - first_r, GR);
  const int tr = first_r + (bid % (GR * tiles_c)) % gsize, tc = (bid % (GR * tiles_c)) / gsize;
  const int r0 = tr * BM, c0 = tc * BN;
  const int nrb = (R + 15) / 16, KS4 = (KS + 3) / 4, KSP = 4 * KS4, G = KS4;

  // Per-lane DMA sources. Rows past the end are clamped to the last row (block); their results are never
  // stored. Sparse rows past R inside the last row block are zero in the tiled layout.
  // The loads are buffer loads: a resource (base and size) in scalar registers, a 32-bit lane offset that stays
  // constant through the loop and a uniform offset that carries the step, so no vector instruction computes
  // an address (the 64-bit address arithmetic of global loads cost 2-6%). The launcher keeps every operand
  // below 2 GB.
  const uint32_t l16 = lane * 16;
  const uint32_t nA = (uint32_t)nrb * (uint32_t)KSP * 1024u, nB = (uint32_t)C * (uint32_t)ldb,
                 nM = (uint32_t)nrb * (uint32_t)KS4 * (uint32_t)MT::BLOCK;
  uint32_t sA[PAMAX];  // PA of them, uniform: byte offset of A row block q of this wave
#pragma unroll
  for (int q = 0; q < PA; ++q)
    sA[q] = __builtin_amdgcn_readfirstlane((uint32_t)min(r0 / 16 + wave + q * NW, nrb - 1) * (uint32_t)KSP * 1024u);
  uint32_t offb[TJMAX];  // PB of them
#pragma unroll
  for (int q = 0; q < PB; ++q) {
    const int b = (wave + q * NW) * 8 + (lane >> 3);
    offb[q] = (uint32_t)min(c0 + b, C - 1) * (uint32_t)ldb + swz(lane & 7, b & 15) * 16;
  }
  // index-word DMA: instruction i of this wave brings bytes 1024 (wave + NW i) + 16 lane of the slot, i.e.
  // row block rb of the tile at offset off of its group block
  // (8-bit: one row block per instruction; bf16: two 512-byte blocks, the upper half of the wave the second)
  constexpr uint32_t MBLK = MT::BLOCK;
  uint32_t om[4];  // MPW of them
  static_assert(MPW <= 4, "index-word loads per wave");
  const uint32_t moff = MT::BLOCK == 1024 ? l16 : (lane & 31) * 16;
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
    const int rb = (wave + NW * i) * (1024 / MT::BLOCK) + (MT::BLOCK == 1024 ? 0 : (lane >> 5));
    om[i] = (uint32_t)min(r0 / 16 + rb, nrb - 1) * (uint32_t)KS4 * (uint32_t)MT::BLOCK + moff;
  }
  const float* sa = SX ? sx : sw;  // scale indexed by A row
  const float* sb = SX ? sw : sx;  // scale indexed by B row

  // Sources are a uniform base (scalar registers) plus a 32-bit lane offset; the stage's LDS offset is
  // uniform too.
  auto issue = [&](int k, uint32_t so) {  // stage k into the slot at LDS offset so
    SS_LDS uint8_t* base = (SS_LDS uint8_t*)smem + so;
    const uint32_t kb = (uint32_t)min(k, KS - 1) * 128u;  // padding steps re-read the dense operand's last step
#pragma unroll
    for (int q = 0; q < PA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(tv, nA), (SS_LDS void*)(base + (wave + q * NW) * 1024), 16, l16,
                                               sA[q] + (uint32_t)k * 1024u, 0, 0);
#pragma unroll
    for (int q = 0; q < PB; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(bd, nB), (SS_LDS void*)(base + A_BYTES + (wave + q * NW) * 1024), 16,
                                               offb[q], kb, 0, 0);
  };
  auto issue_meta = [&](int g) {  // the index words of 4-step group g into the slot
#pragma unroll
    for (int i = 0; i < MPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(tm, nM), (SS_LDS void*)((SS_LDS uint8_t*)smem + META + (wave + NW * i) * 1024),
                                               16, om[i], g * MBLK, 0, 0);
  };

  // single loads, so a step can spread them among its instructions: load i of stage k (i < PA: an A row
  // block, else 8 B rows), index-word load i of group g, scale load i (A rows, then B rows)
  auto issue_one = [&](int i, int k, uint32_t so) {
    SS_LDS uint8_t* base = (SS_LDS uint8_t*)smem + so;
    if (i < PA) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(tv, nA), (SS_LDS void*)(base + (wave + i * NW) * 1024), 16, l16,
                                               sA[i] + (uint32_t)k * 1024u, 0, 0);
    } else {
      const int q = i - PA;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(bd, nB), (SS_LDS void*)(base + A_BYTES + (wave + q * NW) * 1024), 16,
                                               offb[q], (uint32_t)min(k, KS - 1) * 128u, 0, 0);
    }
  };
  auto meta_one = [&](int i, int g) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(tm, nM), (SS_LDS void*)((SS_LDS uint8_t*)smem + META + (wave + NW * i) * 1024),
                                             16, om[i], g * MBLK, 0, 0);
  };
  // A rows r0 + 64 (wave % 4) + lane; B rows c0 + 64 (wave % (BN / 64)) + lane (waves past the rows' count
  // bring the same bytes as the first ones)
  auto scale_one = [&](int i) {
    // a missing scale vector loads junk from a valid address (never used), so the count stays fixed
    const int wb = i == 0 ? wave % (BM / 64) : wave % (BN / 64);
    const int e = wb * 64 + lane;
    const float* s = i == 0 ? (sa ? sa + min(r0 + e, R - 1) : reinterpret_cast<const float*>(tm) + lane)
                            : (sb ? sb + min(c0 + e, C - 1) : reinterpret_cast<const float*>(tm) + lane);
    __builtin_amdgcn_global_load_lds((const void*)s, (SS_LDS void*)((SS_LDS uint8_t*)smem + META + i * 1024 + wb * 256), 4,
                                     0, 0);
  };

  Acc acc[TI][TJMAX];
#pragma unroll
  for (int t = 0; t < TI; ++t)
#pragma unroll
    for (int u = 0; u < TJ; ++u) acc[t][u] = Acc{0, 0, 0, 0};

  // fragments: A double-buffered (a0 / a1) or refilled after its last use (a0 only), B single-buffered (each
  // column refilled right after its use)
  v4i a0[TI], a1[TI], b[TJMAX][2];
  MV mcur[TI];
  // LDS addresses: one per-lane base per operand (constant across steps) plus the stage's offset, so every
  // fragment read is that sum plus an immediate (all fragment offsets of a stage are below 48 KB).
  const uint32_t la = (wm * TI) * 1024 + lane * 16;
  const uint32_t lb0 = A_BYTES + (wn * TJ * 2 + (r16 >> 3)) * 1024 + (r16 & 7) * 128 + swz(jj, r16) * 16;
  const uint32_t lb1 = A_BYTES + (wn * TJ * 2 + (r16 >> 3)) * 1024 + (r16 & 7) * 128 + swz(4 + jj, r16) * 16;
  const uint32_t lm = META + (wm * TI) * MT::BLOCK + lane * (4 * MT::WB);
  auto lds = [&](uint32_t off) -> const SS_LDS uint8_t* { return (const SS_LDS uint8_t*)smem + off; };
  // va/vb0/vb1: the three per-lane bases plus a stage offset, computed once per step (kept opaque so the
  // compiler does not keep one address register per fragment)
  struct Addr {
    uint32_t a, b0, b1;
  };
  auto addr = [&](uint32_t so) {
    Addr r{so + la, so + lb0, so + lb1};
    asm volatile("" : "+v"(r.a), "+v"(r.b0), "+v"(r.b1));
    return r;
  };
  auto read_a = [&](v4i* a, int t, const Addr& ad) { a[t] = *reinterpret_cast<const SS_LDS v4i*>(lds(ad.a) + t * 1024); };
  auto read_b = [&](int u, const Addr& ad) {
    b[u][0] = *reinterpret_cast<const SS_LDS v4i*>(lds(ad.b0) + u * 2048);
    b[u][1] = *reinterpret_cast<const SS_LDS v4i*>(lds(ad.b1) + u * 2048);
  };
  auto read_meta = [&](MV* m, int t) { m[t] = *reinterpret_cast<const SS_LDS MV*>(lds(lm) + t * MT::BLOCK); };

  // Step j = 4g + Q: wait for stage j+1, barrier, issue stage j+S (and the next group's index words, or at
  // the last group the epilogue scales), then the 8 x TJ instructions of step j on (acur, b, mcur) column by
  // column, each column followed by the reads of stage j+1's B column; stage j+1's A fragments go to anxt
  // (one per column, BN = 256) or back into acur right after their last use (BN = 128); at Q = 3 the next
  // group's index words replace mcur after the last column.
  // sl = slot of stage j (= slot of stage j + S), sl1 = slot of stage j + 1 (LDS offsets)
  auto step = [&](int j, auto qc, auto lastc, v4i* acur, v4i* anxt, uint32_t sl, uint32_t sl1) {
    constexpr int Q = decltype(qc)::value;
    constexpr bool LAST = decltype(lastc)::value;
    constexpr bool NEXT = !(LAST && Q == 3);  // stage j+1 exists
    constexpr bool SJ = !LAST || Q + S <= 3;   // stage j+S exists
    // loads issued after this wave's stage j+1 (issued at step j+1-S): with three stages, stage j+2 (if it
    // exists); the index words or scales issued right after a group's first stage load (at steps j-2 / j-1
    // with three stages, at step j-1 with two)
    constexpr int N = (S == 3 && (!LAST || Q < 2) ? LPW : 0) +
                      ((Q == 1 || (S == 3 && Q == 2)) ? (LAST ? NSC : MPW) : 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) {
      __builtin_amdgcn_s_waitcnt(vm(N));
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads of stage j (and the slot) are done
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_sched_barrier(0);
    // The step's loads (stage j+S, then the next group's index words or the epilogue scales) are spread over
    // its instructions, SLOTS per column: one wave per SIMD has no other wave to issue instructions while it
    // sends a run of loads, so the matrix core would idle behind it. BN = 256: load slot s goes after
    // instruction t = 0 (s even) or t = 4 (s odd) of column s / 2, the A fragment of stage j+1 after t = 1;
    // BN = 128: slots after t = 0, 3, 6 (on random codes 0-6% faster per product than after 1, 4, 7, on the
    // Llama-shaped layer at 4096 tokens no different; 2, 5, 7 no better). The two B
    // fragment halves follow the column's last instruction (their
    // registers are free from then on).
    constexpr int NL = (SJ ? LPW : 0) + (Q == 0 ? (LAST ? NSC : MPW) : 0);
    auto load_slot = [&](int s) {
      if (s >= NL) return;
      if (SJ && s < LPW) issue_one(s, j + S, sl);
      else if (!LAST) meta_one(s - (SJ ? LPW : 0), j / 4 + 1);
      else scale_one(s - (SJ ? LPW : 0));
    };
    static_assert(LPW + MPW <= SH::SLOTS * TJ && LPW + NSC <= SH::SLOTS * TJ, "load slots per column");
    const Addr st = addr(sl1);
#pragma unroll
    for (int u = 0; u < TJ; ++u) {
#pragma unroll
      for (int t = 0; t < TI; ++t) {
        acc[t][u] = tiled::mma_step<AB, Q>(acur[t], b[u][0], b[u][1], acc[t][u], mcur[t]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SH::ADB) {
          if (t == 0) {
            load_slot(2 * u);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (t == 1 && NEXT) {
            read_a(anxt, u, st);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (t == 4) {
            load_slot(2 * u + 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          if (u == TJ - 1 && NEXT) {
            read_a(anxt, t, st);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (t == 0 || t == 3 || t == 6) {
            load_slot(3 * u + t / 3);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      if constexpr (NEXT) {
        read_b(u, st);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (Q == 3 && !LAST) {  // after the step's last use of this group's words
#pragma unroll
      for (int t = 0; t < TI; ++t) read_meta(mcur, t);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
  using NotLast = std::false_type;
  using Last = std::true_type;

  // prologue: group 0's index words, stages 0 .. S-1; wait for stage 0
  issue_meta(0);
#pragma unroll
  for (int k = 0; k < S; ++k) issue(k, k * STAGE);
  __builtin_amdgcn_s_waitcnt(vm((S - 1) * LPW));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  {
    const Addr st = addr(0);
#pragma unroll
    for (int t = 0; t < TI; ++t) read_a(a0, t, st);
#pragma unroll
    for (int u = 0; u < TJ; ++u) read_b(u, st);
#pragma unroll
    for (int t = 0; t < TI; ++t) read_meta(mcur, t);
  }
  // slot offsets of stages j, j+1 (and j+2) (uniform), rotated every step
  uint32_t s0 = 0, s1 = STAGE, s2 = 2 * STAGE;
  auto rot = [&]() {
    const uint32_t t = s0;
    s0 = __builtin_amdgcn_readfirstlane(s1);
    if constexpr (S == 3) {
      s1 = __builtin_amdgcn_readfirstlane(s2);
      s2 = __builtin_amdgcn_readfirstlane(t);
    } else {
      s1 = __builtin_amdgcn_readfirstlane(t);
    }
  };
  v4i* const ax = SH::ADB ? a1 : a0;  // the second A buffer (the first again when single-buffered)
  for (int g = 0; g + 1 < G; ++g) {
    const int j = 4 * g;
    step(j, Q0{}, NotLast{}, a0, ax, s0, s1);
    rot();
    step(j + 1, Q1{}, NotLast{}, ax, a0, s0, s1);
    rot();
    step(j + 2, Q2{}, NotLast{}, a0, ax, s0, s1);
    rot();
    step(j + 3, Q3{}, NotLast{}, ax, a0, s0, s1);
    rot();
  }
  {
    const int j = KSP - 4;
    step(j, Q0{}, Last{}, a0, ax, s0, s1);
    rot();
    step(j + 1, Q1{}, Last{}, ax, a0, s0, s1);
    rot();
    step(j + 2, Q2{}, Last{}, a0, ax, s0, s1);
    rot();
    step(j + 3, Q3{}, Last{}, ax, a0, s0, s1);
  }
  __builtin_amdgcn_s_waitcnt(vm(0));  // the scales (and no load may outlive the workgroup)
  __builtin_amdgcn_s_barrier();

  // Epilogue: y = fl32(fl32(float(acc) * sx[m]) * sw[n]); out-of-range results are never stored. The lane
  // and wave coordinates are derived again here from a value the compiler cannot see through, so it does not
  // keep the epilogue's address terms alive through the main loop.
  {
    int etid = threadIdx.x;
    asm volatile("" : "+v"(etid));
    const int lane = etid & 63, wave = __builtin_amdgcn_readfirstlane(etid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int r16 = lane & 15, jj = lane >> 4;
    // This lane's scales, read once: A rows (wm TI + t) 16 + 4 jj + q and B row (wn TJ + u) 16 + r16. An absent
    // scale vector reads as 1 (its slot holds junk, never used), and a multiply by 1 is exact, so every result
    // takes the same two multiplies with no branch per value.
    const float* scl = reinterpret_cast<const float*>(smem + META);
    const bool has_a = sa != nullptr, has_b = sb != nullptr;
    float s_a[TI][4], s_b[TJMAX];
  #pragma unroll
    for (int t = 0; t < TI; ++t) {
      const float4 v = *reinterpret_cast<const float4*>(scl + (wm * TI + t) * 16 + 4 * jj);
      s_a[t][0] = has_a ? v.x : 1.0f;
      s_a[t][1] = has_a ? v.y : 1.0f;
      s_a[t][2] = has_a ? v.z : 1.0f;
      s_a[t][3] = has_a ? v.w : 1.0f;
    }
  #pragma unroll
    for (int u = 0; u < TJ; ++u) s_b[u] = has_b ? scl[256 + (wn * TJ + u) * 16 + r16] : 1.0f;
    // lane's 4 results of instruction tile (t, u): A rows 16 t + 4 jj + q, B row 16 u + r16 (wave-local);
    // the token scale first, then the channel scale
    auto result = [&](int t, int u, float* y, int32_t* yi) {
  #pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (YT == 2) {
          yi[q] = (int32_t)acc[t][u][q];
        } else {
          const float s1 = SX ? s_a[t][q] : s_b[u], s2 = SX ? s_b[u] : s_a[t][q];
          y[q] = __fmul_rn(__fmul_rn((float)acc[t][u][q], s1), s2);
        }
      }
    };
    constexpr int EB = YT == 0 ? 2 : 4;  // output element bytes
    const bool vec = ((int64_t)ldy * EB) % 16 == 0;
    uint8_t* Yb = static_cast<uint8_t*>(Y);
    // one 16-byte piece of staged results: whole when it lies inside Y and rows are 16-byte aligned, else
    // element by element (row: the output row; col: its first column; n: columns in Y)
    auto put = [&](const v4i& v, int row, int col, int ncol) {
      uint8_t* dst = Yb + ((int64_t)row * ldy + col) * EB;
      if (vec && col + 16 / EB <= ncol) {
        __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst));  // whole rows: no line left to merge in L2
      } else {
        const uint32_t w[4] = {(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
  #pragma unroll
        for (int e = 0; e < 16 / EB; ++e) {
          if (col + e >= ncol) break;
          if constexpr (EB == 2) reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          else reinterpret_cast<uint32_t*>(dst)[e] = w[e];
        }
      }
    };
    if constexpr (SX) {
      // Y[A row][B row]: a lane's 4 results of a tile lie in 4 output rows. The wave's 128 x 16 TJ results go
      // through its part of the idle ring as [A row][B row] (16 RX A rows per pass, rows padded by 16 bytes: the
      // 2- or 4-byte writes of a tile and the 16-byte reads are free of bank conflicts) and leave as 16-byte
      // pieces of output rows.
      constexpr int STRIDE = 16 * TJ * EB + 16, CPR = TJ * EB;                  // row bytes, 16-byte chunks
      constexpr int RX = up_rows(TI, META / NW / (16 * STRIDE)), NP = TI / RX;  // A blocks per pass; passes
      static_assert(NW * 16 * RX * STRIDE <= META, "staging fits the stage ring");
      SS_LDS uint8_t* stg = (SS_LDS uint8_t*)smem + wave * 16 * RX * STRIDE;
  #pragma unroll
      for (int p = 0; p < NP; ++p) {
  #pragma unroll
        for (int tt = 0; tt < RX; ++tt) {
  #pragma unroll
          for (int u = 0; u < TJ; ++u) {
            float y[4];
            int32_t yi[4];
            result(p * RX + tt, u, y, yi);
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              SS_LDS uint8_t* d = stg + (tt * 16 + 4 * jj + q) * STRIDE + (u * 16 + r16) * EB;
              if constexpr (YT == 0) *reinterpret_cast<SS_LDS uint16_t*>(d) = (uint16_t)pack_bf16x2(y[q], 0.0f);
              else if constexpr (YT == 1) *reinterpret_cast<SS_LDS float*>(d) = y[q];
              else *reinterpret_cast<SS_LDS int32_t*>(d) = yi[q];
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
        const int ar0 = r0 + (wm * TI + p * RX) * 16, bc0 = c0 + wn * TJ * 16;
        if (vec && ar0 + 16 * RX <= R && bc0 + 16 * TJ <= C) {
          // the pass's rows lie inside Y: every LDS read first, then every store
          constexpr int IT = 16 * RX * CPR / 64;
          v4i v[IT];
  #pragma unroll
          for (int k = 0; k < IT; ++k) {
            const int i = lane + 64 * k;
            v[k] = *reinterpret_cast<const SS_LDS v4i*>(stg + (i / CPR) * STRIDE + (i % CPR) * 16);
          }
  #pragma unroll
          for (int k = 0; k < IT; ++k) {
            const int i = lane + 64 * k;
            __builtin_nontemporal_store(
                v[k], reinterpret_cast<v4i*>(Yb + ((int64_t)(ar0 + i / CPR) * ldy + bc0 + (i % CPR) * (16 / EB)) * EB));
          }
        } else {
  #pragma unroll 4
          for (int i = lane; i < 16 * RX * CPR; i += 64) {
            const int row = i / CPR, ch = i % CPR;
            const v4i v = *reinterpret_cast<const SS_LDS v4i*>(stg + row * STRIDE + ch * 16);
            const int ar = ar0 + row;
            if (ar >= R) continue;
            put(v, ar, bc0 + ch * (16 / EB), C);
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
      return;
    }
    // Y[B row][A row]: each lane holds 4 consecutive A rows of one B row (8 or 16 bytes). The wave's 128 x 16 TJ
    // results go through its own part of the (now idle) stage ring, 16 UP B rows per pass, rows padded by 16
    // bytes so both the writes and the reads are free of bank conflicts, and leave as 16-byte pieces that
    // cover whole output rows.
    constexpr int STRIDE = 128 * EB + 16, CPR = 128 * EB / 16;                 // row bytes, 16-byte chunks
    constexpr int UP = up_rows(TJ, META / NW / (16 * STRIDE)), NP = TJ / UP;  // B fragments per pass; passes
    constexpr int RP = 16 * UP;                                                // rows per pass
    static_assert(NW * RP * STRIDE <= META, "staging fits the stage ring");
    SS_LDS uint8_t* stg = (SS_LDS uint8_t*)smem + wave * RP * STRIDE;
  #pragma unroll
    for (int p = 0; p < NP; ++p) {
  #pragma unroll
      for (int uu = 0; uu < UP; ++uu) {
  #pragma unroll
        for (int t = 0; t < TI; ++t) {
          float y[4];
          int32_t yi[4];
          result(t, p * UP + uu, y, yi);
          SS_LDS uint8_t* d = stg + (uu * 16 + r16) * STRIDE + (t * 16 + 4 * jj) * EB;
          if constexpr (YT == 0) {
            *reinterpret_cast<SS_LDS tiled::v2i*>(d) = tiled::v2i{(int)pack_bf16x2(y[0], y[1]), (int)pack_bf16x2(y[2], y[3])};
          } else if constexpr (YT == 1) {
            *reinterpret_cast<SS_LDS v4i*>(d) = v4i{__float_as_int(y[0]), __float_as_int(y[1]), __float_as_int(y[2]),
                                                    __float_as_int(y[3])};
          } else {
            *reinterpret_cast<SS_LDS v4i*>(d) = v4i{yi[0], yi[1], yi[2], yi[3]};
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      const int bc0 = c0 + (wn * TJ + p * UP) * 16, ar0 = r0 + wm * TI * 16;
      if (vec && bc0 + RP <= C && ar0 + 128 <= R) {
        // the pass's rows lie inside Y: every LDS read first, then every store (one read in flight at a time
        // would leave each wave waiting out the LDS latency once per 16-byte piece)
        constexpr int IT = RP * CPR / 64;
        v4i v[IT];
  #pragma unroll
        for (int k = 0; k < IT; ++k) {
          const int i = lane + 64 * k;
          v[k] = *reinterpret_cast<const SS_LDS v4i*>(stg + (i / CPR) * STRIDE + (i % CPR) * 16);
        }
  #pragma unroll
        for (int k = 0; k < IT; ++k) {
          const int i = lane + 64 * k;
          __builtin_nontemporal_store(
              v[k], reinterpret_cast<v4i*>(Yb + ((int64_t)(bc0 + i / CPR) * ldy + ar0 + (i % CPR) * (16 / EB)) * EB));
        }
      } else {
  #pragma unroll 4
        for (int i = lane; i < RP * CPR; i += 64) {
          const int row = i / CPR, ch = i % CPR;
          const v4i v = *reinterpret_cast<const SS_LDS v4i*>(stg + row * STRIDE + ch * 16);
          const int bc = bc0 + row;
          if (bc >= C) continue;
          put(v, bc, ar0 + ch * (16 / EB), R);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

template <int BN, int W, int AB, int YT, bool SX, int GR = 8>
hipError_t launch(int R, int C, int KS, const uint8_t* tv, const uint8_t* tm, const uint8_t* bd, int ldb, const float* sx,
                  const float* sw, void* Y, int ldy, hipStream_t st) {
  auto kern = wide_kernel<BN, W, AB, YT, SX, GR>;
  constexpr int lds = lds_bytes<BN, W, AB>();
  const hipError_t e = lds_limit((const void*)kern, lds);
  if (e != hipSuccess) return e;
  const int tr = (R + BM - 1) / BM, tc = (C + BN - 1) / BN;
  hipLaunchKernelGGL(kern, dim3(tr * tc), dim3(64 * W), lds, st, R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, tr, tc);
  return hipGetLastError();
}

template <int BN, int W, bool SX>
hipError_t launch_bn(int ab, int yt, int R, int C, int KS, const uint8_t* tv, const uint8_t* tm, const uint8_t* bd, int ldb,
                     const float* sx, const float* sw, void* Y, int ldy, hipStream_t st) {
  if (ab == 0) {
    if (yt == 0) return launch<BN, W, 0, 0, SX>(R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, st);
    if (yt == 1) return launch<BN, W, 0, 1, SX>(R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, st);
    return launch<BN, W, 0, 2, SX>(R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, st);
  }
  if (ab == 1) {
    if (yt == 0) return launch<BN, W, 1, 0, SX>(R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, st);
    return launch<BN, W, 1, 1, SX>(R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, st);
  }
  if (yt == 0) return launch<BN, W, 2, 0, SX>(R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, st);
  return launch<BN, W, 2, 1, SX>(R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, st);
}

}  // namespace wide

// 256 x 256 tiles take eight waves up to this many steps of the reduction, four beyond: on Llama-shaped FP8
// layers at 16384 tokens eight waves were 1.02x on qkv and o and 1.005-1.02x on gate_up (32 steps), 0.97x on
// down (112 steps).
constexpr int kWide8MaxSteps = 64;

hipError_t launch_spgemm_wide(int bn, bool side_x, int ab, int yt, int R, int C, int KS, const uint8_t* tv,
                              const uint8_t* tm, const uint8_t* bd, int ldb, const float* sx, const float* sw, void* Y,
                              int ldy, hipStream_t st) {
  if (side_x) return wide::launch_bn<128, 4, true>(ab, yt, R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, st);
  if (bn != 256) return wide::launch_bn<128, 4, false>(ab, yt, R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, st);
  return KS <= kWide8MaxSteps ? wide::launch_bn<256, 8, false>(ab, yt, R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, st)
                              : wide::launch_bn<256, 4, false>(ab, yt, R, C, KS, tv, tm, bd, ldb, sx, sw, Y, ldy, st);
}

}  // namespace ss
