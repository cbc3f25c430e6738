// Prefill layer with the per-token quantisation moved into the sparse product's prologue: the product
// reads the bf16 activations themselves and codes them into its LDS stages, so the quantised activation
// X' never makes a round trip through HBM (SlideSparse blog, section 3.2, fuses the lift into the
// quantisation kernel; this moves both into the product). 2:4 weights (no lift: K' = K), INT8 or FP8
// codes, per-token x per-channel scales (LLM Compressor W8A8 rows).
//
// Three launches: (1) per-token absmax of X into sx; (2) the product: a 256 x 128 tile per workgroup of 8
// waves on the tiled sparse weights, as the 256 x 128 kernel of k_spgemm_tiled.hip -- sparse values by LDS
// DMA into a ring of four stages, index words into registers one 4-step group ahead -- except that each
// wave loads 16 token rows x 128 positions of bf16 straight into registers one step ahead, codes them with
// the token's fl32(Q / a) exactly as ss_quant_lift_act does, and writes the codes into the stage's swizzled
// rows; (3) sx[m] = a / Q. The codes, the products and the sums are those of ss_quant_lift_act followed
// by ss_spgemm_tiled, bit for bit.
#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_mma.h"
#include "ss_store.h"

namespace ss {
namespace fq {

using tiled::Meta;
using tiled::Mma;
using tiled::swz;
using tiled::v4i;
#define SS_LDS __attribute__((address_space(3)))

constexpr int BM = 256, BN = 128, WGN = 2, NW = 8, S = 4, TI = 4, TJ = 4;
constexpr int PA = BM / 16 / NW;  // sparse-value DMA loads per wave per step (1 KB each)
constexpr int XL = 4;             // bf16 loads per wave per step: 16 token rows x 256 bytes
constexpr int A_BYTES = BM * 64, STAGE = A_BYTES + BN * 128, LDS = S * STAGE;
constexpr int SCL = LDS, LDS_TOTAL = LDS + (BM + BN) * 4;  // epilogue: channel scales, then token absmax

constexpr int vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Per-token absmax of bf16 rows (exact: max of magnitudes), one workgroup per row.
__global__ __launch_bounds__(kBlock) void absmax_kernel(const uint16_t* __restrict__ X, int64_t ldx, int K,
                                                        float* __restrict__ amax) {
  __shared__ float red[kBlock / 64];
  const uint16_t* xr = X + (int64_t)blockIdx.x * ldx;
  float a = 0.0f;
  for (int v = threadIdx.x; v < K / 8; v += kBlock) {
    const uint4 q = reinterpret_cast<const uint4*>(xr)[v];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a = fmaxf(a, fmaxf(fabsf(bf16_to_f32((uint16_t)(w[i] & 0xFFFF))), fabsf(bf16_to_f32((uint16_t)(w[i] >> 16)))));
  }
  a = block_max(a, red);
  if (threadIdx.x == 0) amax[blockIdx.x] = a;
}

// sx[m] = a / Q (0 for an all-zero token), as ss_quant_lift_act writes it.
template <bool FP8>
__global__ __launch_bounds__(kBlock) void scale_kernel(float* __restrict__ sx, int M) {
  const int m = blockIdx.x * kBlock + threadIdx.x;
  if (m >= M) return;
  const float a = sx[m];
  sx[m] = a == 0.0f ? 0.0f : a / Quant<FP8>::Q;
}

// R = output channels (sparse rows), C = tokens, KS = 128-position steps of Kc, KX = steps that hold
// tokens' positions (K / 128; later steps are zero codes).
template <int AB, int YT>
__global__ __launch_bounds__(64 * NW, 1) void fq_kernel(int R, int C, int KS, int KX, const uint8_t* __restrict__ tv,
                                                        const uint8_t* __restrict__ tm, const uint16_t* __restrict__ X,
                                                        int ldx, const float* __restrict__ amax,
                                                        const float* __restrict__ sw, void* __restrict__ Y, int ldy,
                                                        int tiles_r, int tiles_c) {
  using Acc = typename Mma<AB>::Acc;
  using MT = Meta<AB>;
  using MV = typename MT::V;
  using Qz = Quant<AB == 1>;
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int r16 = lane & 15, jj = lane >> 4;

  // tile order as in the 256 x 128 kernel: each XCD a contiguous run, groups of 4 A-row tiles
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  constexpr int GR = 4;
  const int group = bid / (GR * tiles_c), first_r = group * GR, gsize = min(tiles_r - first_r, GR);
  const int tr = first_r + (bid % (GR * tiles_c)) % gsize, tc = (bid % (GR * tiles_c)) / gsize;
  const int r0 = tr * BM, c0 = tc * BN;
  const int nrb = (R + 15) / 16, KS4 = (KS + 3) / 4, KSP = 4 * KS4;

  // sparse values (DMA) and index words (registers), rows past the end clamped (never stored)
  const uint8_t* pa[PA];
#pragma unroll
  for (int q = 0; q < PA; ++q) pa[q] = tv + (int64_t)min(r0 / 16 + wave + q * NW, nrb - 1) * KSP * 1024 + lane * 16;
  const uint8_t* pmt[TI];
#pragma unroll
  for (int t = 0; t < TI; ++t)
    pmt[t] = tm + (int64_t)min(r0 / 16 + wm * TI + t, nrb - 1) * KS4 * MT::BLOCK + lane * (4 * MT::WB);
  // token rows: load i of this wave is stage row b = 16 wave + 4 i + lane / 16, eight positions 8 (lane % 16)
  const uint16_t* px[XL];
  float inv[XL];
  bool zero[XL];
  uint32_t lw[XL];  // LDS byte offset of the lane's 8 codes in a stage (row b, swizzled 16-byte chunk, half)
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int b = wave * 16 + 4 * i + jj, tok = min(c0 + b, C - 1);
    px[i] = X + (int64_t)tok * ldx + 8 * r16;
    const float a = amax[tok];
    zero[i] = a == 0.0f;
    inv[i] = zero[i] ? 0.0f : Qz::Q / a;
    lw[i] = A_BYTES + (b >> 3) * 1024 + (b & 7) * 128 + swz(r16 >> 1, b) * 16 + (r16 & 1) * 8;
  }

  auto issue_a = [&](int k) {  // stage k's sparse values into slot k % S (k clamped in bounds; extras unused)
    SS_LDS uint8_t* base = (SS_LDS uint8_t*)smem + (k % S) * STAGE;
    const int ka = min(k, KSP - 1);
#pragma unroll
    for (int q = 0; q < PA; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(pa[q] + (int64_t)ka * 1024),
                                       (SS_LDS void*)(base + (wave + q * NW) * 1024), 16, 0, 0);
  };
  v4i xb[XL];
  auto load_x = [&](int k) {  // stage k's bf16 (a step past the tokens' positions re-reads the last one)
    const int kx = min(k, KX - 1);
#pragma unroll
    for (int i = 0; i < XL; ++i) xb[i] = *reinterpret_cast<const v4i*>(px[i] + 128 * kx);
  };
  auto code_x = [&](int k) {  // codes of stage k from xb into slot k % S (zero past the tokens' positions)
    SS_LDS uint8_t* base = (SS_LDS uint8_t*)smem + (k % S) * STAGE;
    const bool live = k < KX;
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const uint32_t w[4] = {(uint32_t)xb[i][0], (uint32_t)xb[i][1], (uint32_t)xb[i][2], (uint32_t)xb[i][3]};
      auto e = [&](int h) { return bf16_to_f32((uint16_t)((h & 1) ? (w[h >> 1] >> 16) : (w[h >> 1] & 0xFFFF))); };
      const bool z = zero[i] || !live;
      const uint32_t lo = z ? 0u : Qz::pack4(e(0), e(1), e(2), e(3), inv[i]);
      const uint32_t hi = z ? 0u : Qz::pack4(e(4), e(5), e(6), e(7), inv[i]);
      *reinterpret_cast<SS_LDS tiled::v2i*>(base + lw[i]) = tiled::v2i{(int)lo, (int)hi};
    }
  };
  MV mcur[TI], mnxt[TI];
  auto load_meta = [&](MV* m, int g) {
    const int gg = min(g, KS4 - 1);
#pragma unroll
    for (int t = 0; t < TI; ++t) m[t] = *reinterpret_cast<const MV*>(pmt[t] + (int64_t)gg * MT::BLOCK);
  };

  Acc acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int u = 0; u < TJ; ++u) acc[i][u] = Acc{0, 0, 0, 0};
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
      for (int t = 0; t < TI; ++t) acc[t][u] = tiled::mma_step<AB, Q>(f.a[t], f.b[u][0], f.b[u][1], acc[t][u], mcur[t]);
  };

  // Every step issues the same loads (past the end they re-read in bounds into free slots, never used), in
  // this order: token rows of stage j+2, sparse values of stage j+3, and at the first step of a group the
  // next group's index words. At the top of step j the loads issued after this wave's token rows of stage
  // j+1 are the sparse values of stage j+2 and, if step j-1 began a group, its index words.
  auto step = [&](int j, auto qc, Frag& cur, Frag& nxt) {
    constexpr int Q = decltype(qc)::value;
    constexpr int N = PA + (Q == 1 ? TI : 0);
    const bool next = j + 1 < KSP;
    __builtin_amdgcn_sched_barrier(0);
    if (next) {
      __builtin_amdgcn_s_waitcnt(vm(N));
      code_x(j + 1);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the codes are in LDS (and this wave's reads of stage j)
    }
    __builtin_amdgcn_s_barrier();  // stage j+1 complete for every wave; slot (j+3) % S (stage j-1) is free
    __builtin_amdgcn_sched_barrier(0);
    load_x(j + 2);
    issue_a(j + 3);
    if (Q == 0) load_meta(mnxt, j / 4 + 1);
    __builtin_amdgcn_sched_barrier(0);
    if (next) read(nxt, j + 1);
    mma(cur, qc);
    __builtin_amdgcn_sched_barrier(0);
    if (Q == 3) {
#pragma unroll
      for (int t = 0; t < TI; ++t) mcur[t] = mnxt[t];
    }
  };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;

  // prologue: epilogue scales (channel scales, token absmax) into LDS, group 0's index words, sparse values
  // of stages 0 and 1, token rows of stage 0 -> codes; then token rows of stage 1 and sparse values of stage 2
  if (wave < (BM + BN) / 64) {
    const int i = wave * 64 + lane;
    const float* src = i < BM ? sw + min(r0 + i, R - 1) : amax + min(c0 + i - BM, C - 1);
    __builtin_amdgcn_global_load_lds((const void*)src, (SS_LDS void*)((SS_LDS uint8_t*)smem + SCL + wave * 256), 4, 0, 0);
  }
  load_meta(mcur, 0);
  issue_a(0);
  issue_a(1);
  load_x(0);
  __builtin_amdgcn_s_waitcnt(vm(0));
  code_x(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  load_x(1);
  issue_a(2);
  __builtin_amdgcn_sched_barrier(0);
  Frag f0, f1;
  read(f0, 0);
  for (int g = 0; g < KS4; ++g) {
    const int j = 4 * g;
    step(j, Q0{}, f0, f1);
    step(j + 1, Q1{}, f1, f0);
    step(j + 2, Q2{}, f0, f1);
    step(j + 3, Q3{}, f1, f0);
  }
  __builtin_amdgcn_s_waitcnt(vm(0));  // no load may outlive the workgroup

  // Epilogue: y = fl32(fl32(float(acc) * s_x[m]) * s_w[n]), s_x = a / Q from the token's absmax
  const float* scl = reinterpret_cast<const float*>(smem + SCL);
  float s_b[TJ];
#pragma unroll
  for (int u = 0; u < TJ; ++u) {
    const float a = scl[BM + (wn * TJ + u) * 16 + r16];
    s_b[u] = a == 0.0f ? 0.0f : a / Qz::Q;
  }
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    float s_a[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) s_a[q] = scl[(wm * TI + t) * 16 + 4 * jj + q];
    const int ar = r0 + (wm * TI + t) * 16 + 4 * jj;
#pragma unroll
    for (int u = 0; u < TJ; ++u) {
      const int bc = c0 + (wn * TJ + u) * 16 + r16;
      if (bc >= C) continue;
      float y[4];
      int32_t yi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = __fmul_rn(__fmul_rn((float)acc[t][u][q], s_b[u]), s_a[q]);
      store_out<YT, false>(Y, ldy, ar, bc, R, y, yi);
    }
  }
}

}  // namespace fq

hipError_t launch_quant_spgemm_prefill(int ab, int yt, const uint16_t* X, int64_t ldx, int64_t M, int64_t K,
                                       const uint8_t* tv, const uint8_t* tm, const float* sw, int64_t N, void* Y,
                                       int64_t ldy, float* sx, hipStream_t st) {
  hipLaunchKernelGGL(fq::absmax_kernel, dim3((unsigned)M), dim3(kBlock), 0, st, X, ldx, (int)K, sx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t Kc = (K + 255) / 256 * 256;
  const int R = (int)N, C = (int)M, KS = (int)(Kc / 128), KX = (int)(K / 128);
  const int tr = (R + fq::BM - 1) / fq::BM, tc = (C + fq::BN - 1) / fq::BN;
  auto go = [&](auto kern) -> hipError_t {
    const hipError_t a = lds_limit((const void*)kern, fq::LDS_TOTAL);
    if (a != hipSuccess) return a;
    hipLaunchKernelGGL(kern, dim3(tr * tc), dim3(64 * fq::NW), fq::LDS_TOTAL, st, R, C, KS, KX, tv, tm, X, (int)ldx,
                       (const float*)sx, sw, Y, (int)ldy, tr, tc);
    return hipGetLastError();
  };
  e = ab == 0 ? (yt == 0 ? go(fq::fq_kernel<0, 0>) : go(fq::fq_kernel<0, 1>))
              : (yt == 0 ? go(fq::fq_kernel<1, 0>) : go(fq::fq_kernel<1, 1>));
  if (e != hipSuccess) return e;
  const unsigned g = (unsigned)((M + kBlock - 1) / kBlock);
  if (ab == 0) hipLaunchKernelGGL(fq::scale_kernel<false>, dim3(g), dim3(kBlock), 0, st, sx, (int)M);
  else hipLaunchKernelGGL(fq::scale_kernel<true>, dim3(g), dim3(kBlock), 0, st, sx, (int)M);
  return hipGetLastError();
}

}  // namespace ss
