// Offline SlideSparse weight preparation (SlideSparse article, sliding-window
// decomposition section and figure 2; SlideSparse blog sections 2.2-2.3):
// (2n-2):2n magnitude prune of each 2n-group, greedy assignment of the kept
// nonzeros to the n-1 stride-2 width-4 windows, per-channel quantisation and
// 2:4 compression of W' directly in K' order.
//
// One workgroup per weight row; thread i owns groups i, i + 256, ... A group is
// loaded once (8-byte vectors for float32, 4-byte for bf16), pruned, split into
// its n-1 windows, quantised and written into an LDS image of the output row,
// which is then stored with 16-byte writes. Rows whose groups fit in the
// register budget (G <= 256 * kGPT) are read from HBM once; longer rows are
// read twice (the second pass mostly from cache).
#include "ss_device.h"
#include "ss_kernels.h"

namespace ss {
namespace {

constexpr int kGPT = 8;  // groups per thread held in registers

template <typename TIn> struct GroupIO;
template <> struct GroupIO<float> {
  // 2n floats at element offset 2n*g: 8-byte aligned for every n
  __device__ static void load(const float* row, int64_t g, int n, int64_t K, float* e) {
    const int64_t e0 = (int64_t)g * 2 * n;
    if (e0 + 2 * n <= K) {
      const float2* p = reinterpret_cast<const float2*>(row + e0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n) { const float2 v = p[i]; e[2 * i] = v.x; e[2 * i + 1] = v.y; }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < 2 * n) e[i] = (e0 + i < K) ? row[e0 + i] : 0.0f;
    }
  }
};
template <> struct GroupIO<uint16_t> {
  __device__ static void load(const uint16_t* row, int64_t g, int n, int64_t K, float* e) {
    const int64_t e0 = (int64_t)g * 2 * n;
    if (e0 + 2 * n <= K) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(row + e0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n) { const uint32_t v = p[i]; e[2 * i] = bf16_to_f32((uint16_t)(v & 0xFFFF)); e[2 * i + 1] = bf16_to_f32((uint16_t)(v >> 16)); }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < 2 * n) e[i] = (e0 + i < K) ? bf16_to_f32(row[e0 + i]) : 0.0f;
    }
  }
};

// Keep the 2n-2 largest magnitudes of the group (equal magnitudes keep the
// lower index); returns the bit mask of kept nonzero positions.
template <int N>
__device__ __forceinline__ uint32_t keep_nonzero(const float* e) {
  constexpr int W = 2 * N;
  uint32_t key[W];
#pragma unroll
  for (int i = 0; i < W; ++i) key[i] = mag_key_f32(e[i]);
  uint32_t nz = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    int rank = 0;
#pragma unroll
    for (int j = 0; j < W; ++j) rank += (j < i) ? (key[j] >= key[i]) : (j > i ? (key[j] > key[i]) : 0);
    if (rank < W - 2 && key[i] != 0) nz |= 1u << i;
  }
  return nz;
}

// Emit the n-1 windows of one group into the LDS row image: values (ES bytes
// each) at window slot 2t, 2t+1 and the nibble of window t into metadata word t/8.
template <int N, int OUT>
__device__ __forceinline__ void emit_group(const float* e, int64_t g, bool zero_row, float inv, uint8_t* lv, uint32_t* lm) {
  const uint32_t nz = keep_nonzero<N>(e);
  uint32_t claimed = 0;
#pragma unroll
  for (int w = 0; w < N - 1; ++w) {
    // window w takes the unassigned nonzeros of positions 2w..2w+3, lowest first, up to two
    uint32_t cand = nz & ~claimed & (0xFu << (2 * w));
    const uint32_t m1 = cand & (0u - cand);
    cand &= ~m1;
    const uint32_t m2 = cand & (0u - cand);
    const uint32_t mine = m1 | m2;
    claimed |= mine;
    const uint32_t own = mine >> (2 * w);
    uint32_t fill = own;  // slots: owned positions, then the lowest free ones
    while (__builtin_popcount(fill) < 2) fill |= (~fill) & (fill + 1);
    const uint32_t i0 = __builtin_ctz(fill), i1 = __builtin_ctz(fill & (fill - 1));
    // select with compile-time indices (a runtime index would put e[] in scratch memory)
    const float c0 = e[2 * w], c1 = e[2 * w + 1], c2 = e[2 * w + 2], c3 = e[2 * w + 3];
    const float x0 = i0 == 0 ? c0 : i0 == 1 ? c1 : i0 == 2 ? c2 : c3;
    const float x1 = i1 == 1 ? c1 : i1 == 2 ? c2 : c3;  // i1 > i0 >= 0
    const float v0 = (own >> i0 & 1) ? x0 : 0.0f;
    const float v1 = (own >> i1 & 1) ? x1 : 0.0f;
    const int64_t t = g * (N - 1) + w;
    if constexpr (OUT == 2) {
      reinterpret_cast<uint32_t*>(lv)[t] = (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
    } else {
      const uint32_t c0 = zero_row ? 0u : (uint32_t)Quant<OUT == 1>::code(v0, inv);
      const uint32_t c1 = zero_row ? 0u : (uint32_t)Quant<OUT == 1>::code(v1, inv);
      reinterpret_cast<uint16_t*>(lv)[t] = (uint16_t)(c0 | (c1 << 8));
    }
    atomicOr(&lm[t >> 3], (i0 | (i1 << 2)) << (4 * (t & 7)));
  }
}

template <typename TIn, int N, int OUT>
__global__ __launch_bounds__(kBlock) void slide_kernel(const TIn* __restrict__ W, int64_t ldw, int64_t K,
                                                       uint8_t* __restrict__ vals, int64_t ldv_bytes,
                                                       uint8_t* __restrict__ meta, int64_t ldm, int64_t Kc,
                                                       float* __restrict__ scale) {
  constexpr int ES = (OUT == 2) ? 2 : 1;
  extern __shared__ __align__(16) uint8_t lds[];  // [Kc/2 * ES] values, then [Kc/8] metadata
  __shared__ float red[kBlock / 64];
  uint8_t* lv = lds;
  uint32_t* lm = reinterpret_cast<uint32_t*>(lds + Kc / 2 * ES);
  const int64_t row = blockIdx.x;
  const TIn* wr = W + row * ldw;
  const int tid = threadIdx.x;
  const int64_t G = (K + 2 * N - 1) / (2 * N);
  const bool in_regs = G <= (int64_t)kBlock * kGPT;

  for (int64_t i = tid; i < Kc / 32; i += kBlock) lm[i] = 0;

  float e[kGPT][16];
  float amax = 0.0f;
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < kGPT; ++q) {
      const int64_t g = tid + (int64_t)q * kBlock;
      if (g < G) {
        GroupIO<TIn>::load(wr, g, N, K, e[q]);
#pragma unroll
        for (int i = 0; i < 2 * N; ++i) amax = fmaxf(amax, fabsf(e[q][i]));
      }
    }
  } else {
    for (int64_t g = tid; g < G; g += kBlock) {
      float t[16];
      GroupIO<TIn>::load(wr, g, N, K, t);
#pragma unroll
      for (int i = 0; i < 2 * N; ++i) amax = fmaxf(amax, fabsf(t[i]));
    }
  }
  bool zero_row = false;
  float inv = 0.0f;
  if constexpr (OUT != 2) {
    amax = block_max(amax, red);  // also orders the metadata clear before the ORs below
    constexpr float Q = (OUT == 1) ? 448.0f : 127.0f;
    zero_row = (amax == 0.0f);
    inv = zero_row ? 0.0f : Q / amax;
    if (tid == 0) scale[row] = zero_row ? 0.0f : amax / Q;
  } else {
    __syncthreads();
  }
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < kGPT; ++q) {
      const int64_t g = tid + (int64_t)q * kBlock;
      if (g < G) emit_group<N, OUT>(e[q], g, zero_row, inv, lv, lm);
    }
  } else {
    for (int64_t g = tid; g < G; g += kBlock) {
      float t[16];
      GroupIO<TIn>::load(wr, g, N, K, t);
      emit_group<N, OUT>(t, g, zero_row, inv, lv, lm);
    }
  }
  // padding windows (K' rounded up to Kc): zero values, positions (0, 1)
  for (int64_t t = G * (N - 1) + tid; t < Kc / 4; t += kBlock) {
    if constexpr (OUT == 2) reinterpret_cast<uint32_t*>(lv)[t] = 0;
    else reinterpret_cast<uint16_t*>(lv)[t] = 0;
    atomicOr(&lm[t >> 3], 0x4u << (4 * (t & 7)));
  }
  __syncthreads();
  uint8_t* vr = vals + row * ldv_bytes;
  uint8_t* mr = meta + row * ldm;
  for (int64_t c = tid; c < Kc / 2 * ES / 16; c += kBlock)
    reinterpret_cast<uint4*>(vr)[c] = reinterpret_cast<const uint4*>(lv)[c];
  for (int64_t c = tid; c < Kc / 8 / 16; c += kBlock)
    reinterpret_cast<uint4*>(mr)[c] = reinterpret_cast<const uint4*>(lm)[c];
}

template <typename TIn, int N>
hipError_t launch_n(int out, const TIn* W, int64_t ldw, int64_t rows, int64_t K, void* vals, int64_t ldv_bytes,
                    uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  dim3 grid((unsigned)rows), block(kBlock);
  uint8_t* v = static_cast<uint8_t*>(vals);
  const size_t lds = (size_t)Kc / 2 * (out == 2 ? 2 : 1) + (size_t)Kc / 8;
  const void* fn = out == 0 ? (const void*)slide_kernel<TIn, N, 0> : out == 1 ? (const void*)slide_kernel<TIn, N, 1>
                                                                              : (const void*)slide_kernel<TIn, N, 2>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  switch (out) {
    case 0: hipLaunchKernelGGL((slide_kernel<TIn, N, 0>), grid, block, lds, st, W, ldw, K, v, ldv_bytes, meta, ldm, Kc, scale); break;
    case 1: hipLaunchKernelGGL((slide_kernel<TIn, N, 1>), grid, block, lds, st, W, ldw, K, v, ldv_bytes, meta, ldm, Kc, scale); break;
    default: hipLaunchKernelGGL((slide_kernel<TIn, N, 2>), grid, block, lds, st, W, ldw, K, v, ldv_bytes, meta, ldm, Kc, scale); break;
  }
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_sl(int out, const TIn* W, int64_t ldw, int64_t rows, int64_t K, int n, void* vals, int64_t ldv_bytes,
                     uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  switch (n) {
    case 2: return launch_n<TIn, 2>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    case 3: return launch_n<TIn, 3>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    case 4: return launch_n<TIn, 4>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    case 5: return launch_n<TIn, 5>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    case 6: return launch_n<TIn, 6>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    case 7: return launch_n<TIn, 7>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    default: return launch_n<TIn, 8>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
  }
}

}  // namespace

hipError_t launch_slide(bool in_bf16, int out, const void* W, int64_t ldw, int64_t rows, int64_t K, int n, void* vals,
                        int64_t ldv_bytes, uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  if (in_bf16)
    return launch_sl<uint16_t>(out, static_cast<const uint16_t*>(W), ldw, rows, K, n, vals, ldv_bytes, meta, ldm, Kc, scale, st);
  return launch_sl<float>(out, static_cast<const float*>(W), ldw, rows, K, n, vals, ldv_bytes, meta, ldm, Kc, scale, st);
}

}  // namespace ss
