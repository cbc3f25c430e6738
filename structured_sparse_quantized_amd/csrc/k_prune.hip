// 2:4 magnitude prune + compress along K, for weights (offline; per-channel
// scales) and activations (online; per-token scales). Deep reading of arXiv
// 2610.28947, introduction and sections 1 and 2.3; LLM Compressor guide for
// the scale granularity.
//
// A "unit" is 4 consecutive 4-groups (16 input elements) and produces 8 kept
// values and 2 metadata bytes. When quantised output is requested the row
// absmax is reduced first.
#include "ss_device.h"
#include "ss_kernels.h"

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

namespace ss {

template <typename TIn> struct Unit;
template <> struct Unit<uint16_t> {  // 16 bf16 = 2 x 16 bytes
  uint4 a, b;
  __device__ void load(const uint16_t* p) {
    a = reinterpret_cast<const uint4*>(p)[0];
    b = reinterpret_cast<const uint4*>(p)[1];
  }
  __device__ uint32_t bits(int i) const {
    const uint4& v = (i < 8) ? a : b;
    const uint32_t w = (&v.x)[(i & 7) >> 1];
    return (i & 1) ? (w >> 16) : (w & 0xFFFF);
  }
  __device__ float val(int i) const { return bf16_to_f32((uint16_t)bits(i)); }
  __device__ uint32_t key(int i) const { return mag_key_bf16((uint16_t)bits(i)); }
};
template <> struct Unit<float> {  // 16 float = 4 x 16 bytes
  uint4 q[4];
  __device__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = reinterpret_cast<const uint4*>(p)[i];
  }
  __device__ float val(int i) const { return __uint_as_float((&q[i >> 2].x)[i & 3]); }
  __device__ uint32_t key(int i) const { return mag_key_f32(val(i)); }
};

// Prune one unit: 16-bit metadata (4 nibbles) and the kept values packed as 8 codes (w[0..1]) or
// 8 bf16 (w[0..3]). OUT: 0 = int8, 1 = fp8, 2 = bf16
template <typename TIn, int OUT>
__device__ __forceinline__ uint32_t prune_unit(const Unit<TIn>& u, bool zero_row, float inv, uint32_t* w) {
  uint32_t meta = 0;
  float kv[8];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t nib = top2_nibble(u.key(4 * g), u.key(4 * g + 1), u.key(4 * g + 2), u.key(4 * g + 3));
    meta |= nib << (4 * g);
    const float c0 = u.val(4 * g), c1 = u.val(4 * g + 1), c2 = u.val(4 * g + 2), c3 = u.val(4 * g + 3);
    const uint32_t i0 = nib & 3, i1 = nib >> 2;  // i0 < i1
    // select among compile-time indices (a runtime index would put the unit in scratch memory)
    const float v0 = i0 == 0 ? c0 : i0 == 1 ? c1 : c2;
    const float v1 = i1 == 1 ? c1 : i1 == 2 ? c2 : c3;
    kv[2 * g] = (v0 == 0.0f) ? 0.0f : v0;  // zeros are stored as +0
    kv[2 * g + 1] = (v1 == 0.0f) ? 0.0f : v1;
  }
  if constexpr (OUT == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(kv[2 * i]) | ((uint32_t)f32_to_bf16(kv[2 * i + 1]) << 16);
  } else {
    w[0] = zero_row ? 0u : Quant<OUT == 1>::pack4(kv[0], kv[1], kv[2], kv[3], inv);
    w[1] = zero_row ? 0u : Quant<OUT == 1>::pack4(kv[4], kv[5], kv[6], kv[7], inv);
  }
  return meta;
}

// Prune one unit and store it in the row-major compressed layout.
template <typename TIn, int OUT>
__device__ __forceinline__ void emit_unit(const Unit<TIn>& u, bool zero_row, float inv, uint8_t* vrow,
                                          uint8_t* mrow, int64_t unit) {
  uint32_t w[4];
  const uint32_t meta = prune_unit<TIn, OUT>(u, zero_row, inv, w);
  *reinterpret_cast<uint16_t*>(mrow + unit * 2) = (uint16_t)meta;
  if constexpr (OUT == 2) *reinterpret_cast<uint4*>(vrow + unit * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  else *reinterpret_cast<uint2*>(vrow + unit * 8) = make_uint2(w[0], w[1]);
}

// Prune one unit of row `row` and store it in the tiled layout of the product (k_spgemm_tiled.hip):
// a step is 64 value bytes per row (8 units of 8-bit codes, 4 units of bf16); lane row%16 + 16*chunk.
template <typename TIn, int OUT>
__device__ __forceinline__ void emit_unit_tiled(const Unit<TIn>& u, bool zero_row, float inv, uint8_t* tv, uint8_t* tm,
                                                int row, int unit, int KSP) {
  uint32_t w[4];
  const uint32_t meta = prune_unit<TIn, OUT>(u, zero_row, inv, w);
  const int rb = row >> 4, r = row & 15, KS4 = KSP >> 2;
  if constexpr (OUT == 2) {
    const int s = unit >> 2, lane = r + 16 * (unit & 3);
    *reinterpret_cast<uint4*>(tv + ((int64_t)rb * KSP + s) * 1024 + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint16_t*>(tm + ((int64_t)rb * KS4 + (s >> 2)) * 512 + 8 * lane + 2 * (s & 3)) = (uint16_t)meta;
  } else {
    const int s = unit >> 3, lane = r + 16 * ((unit >> 1) & 3), half = unit & 1;
    *reinterpret_cast<uint2*>(tv + ((int64_t)rb * KSP + s) * 1024 + 16 * lane + 8 * half) = make_uint2(w[0], w[1]);
    *reinterpret_cast<uint16_t*>(tm + ((int64_t)rb * KS4 + (s >> 2)) * 1024 + 16 * lane + 4 * (s & 3) + 2 * half) =
        (uint16_t)meta;
  }
}

// Load unit `unit` (elements 16*unit .. 16*unit + 15) of a row, zeros past K. The row's end is read with
// the same 16-byte loads: a 16-byte chunk (16-byte aligned, as rows are) that starts before K is loaded
// whole and its elements at K and beyond are zeroed in registers; chunks that start at or past K are not
// read. No element-wise loads (their staging array costs registers). WHOLE: whole units take one
// unmasked load first (fewer instructions per unit; the row kernels), else every chunk goes through the
// mask (fewer registers; the lane kernel).
template <typename TIn, bool WHOLE = true>
__device__ __forceinline__ void load_unit_vec(Unit<TIn>& u, const TIn* xr, int64_t unit, int64_t K) {
  constexpr int CE = 16 / (int)sizeof(TIn), NC = 16 / CE;  // elements per chunk, chunks per unit
  const int64_t e0 = unit * 16;
  if (WHOLE && e0 + 16 <= K) {
    u.load(xr + e0);
    return;
  }
  uint4 ch[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t st = e0 + CE * j;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (st < K) v = *reinterpret_cast<const uint4*>(xr + st);
    if (st + CE > K) {  // the chunk holding the row's last element
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t keep;
        if constexpr (sizeof(TIn) == 2)
          keep = (st + 2 * w < K ? 0x0000FFFFu : 0u) | (st + 2 * w + 1 < K ? 0xFFFF0000u : 0u);
        else
          keep = st + w < K ? 0xFFFFFFFFu : 0u;
        (&v.x)[w] &= keep;
      }
    }
    ch[j] = v;
  }
  u.load(reinterpret_cast<const TIn*>(ch));
}

template <typename TIn> __device__ __forceinline__ float unit_absmax(const Unit<TIn>& u) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(u.val(i)));
  return m;
}

// Persistent workgroups walk rows r, r + grid, ...; UPT units per thread are
// held in registers and the next row is loaded before the current one is
// reduced and written, so HBM reads and writes overlap.
// TILED: vals/meta are the tiled operand (ldv_bytes = padded step count KSP, ldm unused); rows up to the
// next multiple of 16 are written (zero past M) and units up to the padded step count; iteration i takes
// row xcd_row(i, rows) so a 16-row block is written through one L2.
template <typename TIn, int OUT, int UPT, bool PIPE, bool TILED = false>
__global__ __launch_bounds__(kBlock, (PIPE || UPT > 2) ? 2 : ((UPT > 1 || TILED) ? 4 : 8)) void prune24_kernel(const TIn* __restrict__ X, int64_t ldx, int M, int K,
                                                         uint8_t* __restrict__ vals, int64_t ldv_bytes,
                                                         uint8_t* __restrict__ meta, int64_t ldm, int Kc,
                                                         float* __restrict__ scale) {
  __shared__ float red[kBlock / 64];
  const int tid = threadIdx.x;
  const int KSP = (int)ldv_bytes;
  // includes padding units (all zero)
  const int units = TILED ? KSP * (OUT == 2 ? 4 : 8) : Kc / 16;
  const int rows = TILED ? (M + 15) / 16 * 16 : M;
  const int data_units = (K + 15) / 16;
  Unit<TIn> cur[UPT], nxt[PIPE ? UPT : 1];
  auto load = [&](Unit<TIn>* u, int r) {
    const TIn* xr = X + (int64_t)(r < M ? r : 0) * ldx;
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int un = tid + i * kBlock;
      if (un < data_units && r < M) load_unit_vec(u[i], xr, un, K);
      else u[i] = Unit<TIn>{};
    }
  };
  auto rowof = [&](int it) { return TILED ? xcd_row(it, rows) : it; };
  int it = blockIdx.x;
  if (it < rows) load(cur, rowof(it));
  for (; it < rows; it += gridDim.x) {
    const int r = rowof(it);
    const int itn = it + gridDim.x;
    if (PIPE && itn < rows) load(nxt, rowof(itn));
    bool zero_row = false;
    float inv = 0.0f;
    if constexpr (OUT != 2) {
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < UPT; ++i) amax = fmaxf(amax, unit_absmax(cur[i]));
      amax = block_max(amax, red);
      constexpr float Q = (OUT == 1) ? 448.0f : 127.0f;
      zero_row = (amax == 0.0f);
      inv = zero_row ? 0.0f : Q / amax;
      if (tid == 0 && r < M) scale[r] = zero_row ? 0.0f : amax / Q;
    }
    if constexpr (TILED) {
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        const int un = tid + i * kBlock;
        if (un < units) emit_unit_tiled<TIn, OUT>(cur[i], zero_row, inv, vals, meta, r, un, KSP);
      }
    } else {
      uint8_t* vr = vals + (int64_t)r * ldv_bytes;
      uint8_t* mr = meta + (int64_t)r * ldm;
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        const int un = tid + i * kBlock;
        if (un < units) emit_unit<TIn, OUT>(cur[i], zero_row, inv, vr, mr, un);
      }
    }
    if constexpr (PIPE) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) cur[u] = nxt[u];
    } else if (itn < rows) {
      load(cur, rowof(itn));
    }
  }
}

// Rows longer than kBlock * 4 units: absmax pass, then a second read. TILED as in prune24_kernel (grid
// covers the rows up to the next multiple of 16; M = the real row count).
template <typename TIn, int OUT, bool TILED = false>
__global__ __launch_bounds__(kBlock) void prune24_long_kernel(const TIn* __restrict__ X, int64_t ldx, int64_t K,
                                                              uint8_t* __restrict__ vals, int64_t ldv_bytes,
                                                              uint8_t* __restrict__ meta, int64_t ldm, int64_t Kc,
                                                              float* __restrict__ scale, int64_t M = 0) {
  __shared__ float red[kBlock / 64];
  const int64_t row = TILED ? xcd_row(blockIdx.x, gridDim.x) : blockIdx.x;
  const bool live = !TILED || row < M;
  const TIn* xr = X + (live ? row : 0) * ldx;
  const int KSP = (int)ldv_bytes;
  const int64_t units = TILED ? (int64_t)KSP * (OUT == 2 ? 4 : 8) : Kc / 16;
  const int64_t data_units = live ? (K + 15) / 16 : 0;
  bool zero_row = false;
  float inv = 0.0f;
  if constexpr (OUT != 2) {
    float amax = 0.0f;
    for (int64_t un = threadIdx.x; un < data_units; un += kBlock) {
      Unit<TIn> t;
      load_unit_vec(t, xr, un, K);
      amax = fmaxf(amax, unit_absmax(t));
    }
    amax = block_max(amax, red);
    constexpr float Q = (OUT == 1) ? 448.0f : 127.0f;
    zero_row = (amax == 0.0f);
    inv = zero_row ? 0.0f : Q / amax;
    if (threadIdx.x == 0 && live) scale[row] = zero_row ? 0.0f : amax / Q;
  }
  for (int64_t un = threadIdx.x; un < units; un += kBlock) {
    Unit<TIn> t{};
    if (un < data_units) load_unit_vec(t, xr, un, K);
    if constexpr (TILED) emit_unit_tiled<TIn, OUT>(t, zero_row, inv, vals, meta, (int)row, (int)un, KSP);
    else emit_unit<TIn, OUT>(t, zero_row, inv, vals + row * ldv_bytes, meta + row * ldm, un);
  }
}

// bf16 output in the tiled layout (no scale, one read pass): one workgroup per 16-row block, 8 waves;
// lane l of a wave owns row l%16 and the 16-byte lane chunk l/16 of each step of its 4-step groups, so
// every step's values leave as one 1 KB block and every group's index words as one 512-byte block. The
// wave's next group is loaded while this one is pruned and stored (5% on a 1 GB batch).
__global__ __launch_bounds__(512) void prune24_act_tiled_bf16_kernel(const uint16_t* __restrict__ X, int64_t ldx, int M,
                                                                     int K, int KS, uint8_t* __restrict__ tv,
                                                                     uint8_t* __restrict__ tm) {
  constexpr int NWV = 8;
  const int rb = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, c = lane >> 4, row = rb * 16 + r;
  const bool live = row < M;
  const uint16_t* xr = X + (int64_t)(live ? row : 0) * ldx;
  const int KS4 = KS / 4;  // KS is a multiple of 4 for bf16 (Kc % 256 == 0)
  auto load = [&](Unit<uint16_t>* x, int g) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // a step is 64 K positions: 4 units, one per lane chunk
      const int unit = (4 * g + q) * 4 + c;
      if (live && unit * 16 < K) load_unit_vec<uint16_t, false>(x[q], xr, unit, K);
      else x[q] = Unit<uint16_t>{};
    }
  };
  Unit<uint16_t> x[4], nx[4];
  if (wave < KS4) load(x, wave);
  for (int g = wave; g < KS4; g += NWV) {
    if (g + NWV < KS4) load(nx, g + NWV);
    uint32_t mw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t w[4];
      mw[q] = prune_unit<uint16_t, 2>(x[q], false, 0.0f, w);
      *reinterpret_cast<uint4*>(tv + ((int64_t)rb * KS + 4 * g + q) * 1024 + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    *reinterpret_cast<uint2*>(tm + ((int64_t)rb * KS4 + g) * 512 + 8 * lane) =
        make_uint2(mw[0] | (mw[1] << 16), mw[2] | (mw[3] << 16));
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = nx[q];
  }
}


// Persistent grids hold as many workgroups per CU as fit at once (registers; at most 8), so every workgroup
// is resident from the start: a fixed 8 per CU ran the last ones as a partly filled extra round (the FP8
// activation prune of 8192 x 4096 fits 7: 1.05x).
template <typename TIn, int OUT>
static hipError_t launch_p24_tiled(const TIn* X, int64_t ldx, int64_t M, int64_t K, int64_t Kc, uint8_t* tv,
                                   uint8_t* tm, float* sx, hipStream_t st) {
  const int es = OUT == 2 ? 2 : 1;
  const int KS = (int)(Kc * es / 128), KSP = (KS + 3) / 4 * 4;
  const int units = KSP * (OUT == 2 ? 4 : 8);
  const int64_t upt = (units + kBlock - 1) / kBlock;
  const int64_t rows = (M + 15) / 16 * 16;
  const bool pipe = rows > 16 * (int64_t)num_cus_p();
  const unsigned grid = (unsigned)rows;
  const int m = (int)M, k = (int)K, kc = (int)Kc;
#define SS_PT(U_)                                                                                                      \
  do {                                                                                                                 \
    if (pipe)                                                                                                          \
      hipLaunchKernelGGL((prune24_kernel<TIn, OUT, U_, true, true>),                                                   \
                         dim3((unsigned)(std::min(occupancy_p((const void*)prune24_kernel<TIn, OUT, U_, true, true>,    \
                                                              kBlock, 0), 8) * num_cus_p())),                         \
                         dim3(kBlock), 0, st, X, ldx, m, k, tv, (int64_t)KSP, tm, (int64_t)0, kc, sx);                \
    else                                                                                                               \
      hipLaunchKernelGGL((prune24_kernel<TIn, OUT, U_, false, true>), dim3(grid), dim3(kBlock), 0, st, X, ldx, m, k, \
                         tv, (int64_t)KSP, tm, (int64_t)0, kc, sx);                                                    \
  } while (0)
  if (upt > 4) {  // long rows: absmax pass, then a second read
    hipLaunchKernelGGL((prune24_long_kernel<TIn, OUT, true>), dim3((unsigned)rows), dim3(kBlock), 0, st, X, ldx, K, tv,
                       (int64_t)KSP, tm, (int64_t)0, Kc, sx, M);
    return hipGetLastError();
  }
  if (upt <= 1) SS_PT(1);
  else if (upt <= 2) SS_PT(2);
  else SS_PT(4);
#undef SS_PT
  return hipGetLastError();
}

hipError_t launch_prune24_act_tiled(int out, const void* X, int64_t ldx, int64_t M, int64_t K, int64_t Kc, void* tv,
                                    uint8_t* tm, float* sx, hipStream_t st) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  uint8_t* v = static_cast<uint8_t*>(tv);
  switch (out) {
    case 0: return launch_p24_tiled<uint16_t, 0>(x, ldx, M, K, Kc, v, tm, sx, st);
    case 1: return launch_p24_tiled<uint16_t, 1>(x, ldx, M, K, Kc, v, tm, sx, st);
    default: {
      const int KS = (int)(Kc * 2 / 128);
      hipLaunchKernelGGL(prune24_act_tiled_bf16_kernel, dim3((unsigned)((M + 15) / 16)), dim3(512), 0, st, x, ldx, (int)M,
                         (int)K, KS, v, tm);
      return hipGetLastError();
    }
  }
}

hipError_t launch_prune24_tiled(bool in_bf16, int out, const void* W, int64_t ldw, int64_t rows, int64_t K, int64_t Kc,
                                void* tv, uint8_t* tm, float* scale, hipStream_t st) {
  uint8_t* v = static_cast<uint8_t*>(tv);
  if (in_bf16) {
    const uint16_t* w = static_cast<const uint16_t*>(W);
    if (out == 2) return launch_prune24_act_tiled(2, W, ldw, rows, K, Kc, tv, tm, scale, st);
    return out == 0 ? launch_p24_tiled<uint16_t, 0>(w, ldw, rows, K, Kc, v, tm, scale, st)
                    : launch_p24_tiled<uint16_t, 1>(w, ldw, rows, K, Kc, v, tm, scale, st);
  }
  const float* w = static_cast<const float*>(W);
  switch (out) {
    case 0: return launch_p24_tiled<float, 0>(w, ldw, rows, K, Kc, v, tm, scale, st);
    case 1: return launch_p24_tiled<float, 1>(w, ldw, rows, K, Kc, v, tm, scale, st);
    default: return launch_p24_tiled<float, 2>(w, ldw, rows, K, Kc, v, tm, scale, st);
  }
}

// Block-scaled FP8 weights (LLM Compressor guide, W8A8-FP8_BLOCK): 2:4 prune along K, then FP8 codes with
// one scale per block of 128 rows x 128 positions, written to the tiled operand. One workgroup per block:
// its 1024 units (128 rows x 8) are held in registers, 4 per thread, while the block absmax is reduced
// (a magnitude prune keeps every group maximum, so the absmax of the raw block is the block's). Blocks
// past the last scale group are the tiled layout's step padding and rows past the end up to the next
// 16 are zero: both are written as zero units (index words of positions 0 and 1).
template <typename TIn>
__global__ __launch_bounds__(kBlock) void prune24_block_kernel(const TIn* __restrict__ W, int64_t ldw, int rows,
                                                               int K, int KS, int KSP, uint8_t* __restrict__ tv,
                                                               uint8_t* __restrict__ tm, float* __restrict__ sw) {
  __shared__ float red[kBlock / 64];
  const int g = blockIdx.x, b = blockIdx.y;  // scale group (= step of the tiled operand), 128-row block
  const int rows16 = (rows + 15) & ~15;
  Unit<TIn> u[4];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int lu = threadIdx.x + kBlock * j, row = b * 128 + (lu >> 3), unit = g * 8 + (lu & 7);
    u[j] = Unit<TIn>{};
    if (row < rows && g < KS) load_unit_vec(u[j], W + (int64_t)row * ldw, unit, K);
    amax = fmaxf(amax, unit_absmax(u[j]));
  }
  amax = block_max(amax, red);
  const bool zero = amax == 0.0f;
  const float inv = zero ? 0.0f : Quant<true>::Q / amax;
  if (threadIdx.x == 0 && g < KS) sw[(int64_t)b * KS + g] = zero ? 0.0f : amax / Quant<true>::Q;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int lu = threadIdx.x + kBlock * j, row = b * 128 + (lu >> 3), unit = g * 8 + (lu & 7);
    if (row < rows16) emit_unit_tiled<TIn, 1>(u[j], zero, inv, tv, tm, row, unit, KSP);
  }
}

hipError_t launch_prune24_block(bool in_bf16, const void* W, int64_t ldw, int64_t rows, int64_t K, int64_t Kc,
                                void* tv, uint8_t* tm, float* sw, hipStream_t st) {
  const int KS = (int)(Kc / 128), KSP = (KS + 3) / 4 * 4;
  const dim3 grid((unsigned)KSP, (unsigned)((rows + 127) / 128));
  uint8_t* v = static_cast<uint8_t*>(tv);
  if (in_bf16)
    hipLaunchKernelGGL(prune24_block_kernel<uint16_t>, grid, dim3(kBlock), 0, st, static_cast<const uint16_t*>(W), ldw,
                       (int)rows, (int)K, KS, KSP, v, tm, sw);
  else
    hipLaunchKernelGGL(prune24_block_kernel<float>, grid, dim3(kBlock), 0, st, static_cast<const float*>(W), ldw,
                       (int)rows, (int)K, KS, KSP, v, tm, sw);
  return hipGetLastError();
}

// Dynamic-LDS limit of a kernel, raised once per device and kernel: the attribute persists, so later launches
// that need no more bytes skip the runtime call.
hipError_t lds_limit(const void* kern, int bytes) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> have;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> g(mu);
  int& cur = have[{kern, dev}];
  if (cur >= bytes) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) cur = bytes;
  return e;
}

// Resident workgroups per CU of a kernel at a block size and dynamic LDS size, cached per device.
int occupancy_p(const void* kern, int block, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, int, size_t>, int> have;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> g(mu);
  const auto key = std::make_tuple(kern, dev, block, lds);
  const auto it = have.find(key);
  if (it != have.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, block, lds) != hipSuccess || n < 1) n = 1;
  have[key] = n;
  return n;
}

int num_cus_p() {
  // cached per device (the library may be used on several GPUs from several threads)
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::atomic<int>* slot = dev < kMaxDev ? &cache[dev] : nullptr;
  int n = slot ? slot->load(std::memory_order_relaxed) : 0;
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (slot) slot->store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename TIn, int OUT>
static hipError_t launch_out(const TIn* X, int64_t ldx, int64_t M, int64_t K, uint8_t* v, int64_t ldv_bytes,
                             uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  const int64_t upt = (Kc / 16 + kBlock - 1) / kBlock;
  if (upt > 4 || K >= (1 << 30) || Kc >= (1 << 30) || M >= (1 << 30)) {
    hipLaunchKernelGGL((prune24_long_kernel<TIn, OUT>), dim3((unsigned)M), dim3(kBlock), 0, st, X, ldx, K, v, ldv_bytes,
                       meta, ldm, Kc, scale);
    return hipGetLastError();
  }
  const bool pipe = M > 16 * (int64_t)num_cus_p();
  const int m = (int)M, k = (int)K, kc = (int)Kc;
#define SS_P(U_) \
  do { if (pipe) hipLaunchKernelGGL((prune24_kernel<TIn, OUT, U_, true>), dim3((unsigned)(std::min(occupancy_p((const void*)prune24_kernel<TIn, OUT, U_, true>, kBlock, 0), 8) * num_cus_p())), dim3(kBlock), 0, st, X, ldx, m, k, v, ldv_bytes, meta, ldm, kc, scale); else hipLaunchKernelGGL((prune24_kernel<TIn, OUT, U_, false>), dim3((unsigned)M), dim3(kBlock), 0, st, X, ldx, m, k, v, ldv_bytes, meta, ldm, kc, scale); } while (0)
  if (upt <= 1) SS_P(1);
  else if (upt <= 2) SS_P(2);
  else SS_P(4);
#undef SS_P
  return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_p24(int out, const TIn* X, int64_t ldx, int64_t M, int64_t K, void* vals, int64_t ldv_bytes,
                             uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  uint8_t* v = static_cast<uint8_t*>(vals);
  switch (out) {
    case 0: return launch_out<TIn, 0>(X, ldx, M, K, v, ldv_bytes, meta, ldm, Kc, scale, st);
    case 1: return launch_out<TIn, 1>(X, ldx, M, K, v, ldv_bytes, meta, ldm, Kc, scale, st);
    default: return launch_out<TIn, 2>(X, ldx, M, K, v, ldv_bytes, meta, ldm, Kc, scale, st);
  }
}

hipError_t launch_prune24(bool in_bf16, int out, const void* X, int64_t ldx, int64_t M, int64_t K, void* vals,
                          int64_t ldv_bytes, uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  if (in_bf16)
    return launch_p24<uint16_t>(out, static_cast<const uint16_t*>(X), ldx, M, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
  return launch_p24<float>(out, static_cast<const float*>(X), ldx, M, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
}

}  // namespace ss
