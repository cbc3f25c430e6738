// Offline SlideSparse weight preparation (SlideSparse article, sliding-window
// decomposition section and figure 2; SlideSparse blog sections 2.2-2.3):
// (2n-2):2n magnitude prune of each 2n-group, greedy assignment of the kept
// nonzeros to the n-1 stride-2 width-4 windows, per-channel quantisation and
// 2:4 compression of W' directly in K' order.
//
// One workgroup per weight row. A unit is 4 consecutive windows (one 16-wide
// slice of K') -> 8 values + 2 metadata bytes. Each window recomputes its own
// group's prune and window claims (2n <= 16 elements; this is offline work).
#include "ss_device.h"
#include "ss_kernels.h"

namespace ss {

template <typename TIn> __device__ __forceinline__ float load_elem(const TIn* xr, int64_t i, int64_t K);
template <> __device__ __forceinline__ float load_elem<float>(const float* xr, int64_t i, int64_t K) {
  return i < K ? xr[i] : 0.0f;
}
template <> __device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* xr, int64_t i, int64_t K) {
  return i < K ? bf16_to_f32(xr[i]) : 0.0f;
}

// Positions (bits of a 2n-wide mask) that window w owns in group g.
template <typename TIn>
__device__ __forceinline__ uint32_t window_owned(const TIn* xr, int64_t K, int n, int64_t g, int w, float* e /*[16]*/) {
  const int width = 2 * n;
  uint32_t key[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < width) {
      e[i] = load_elem<TIn>(xr, g * width + i, K);
      key[i] = mag_key_f32(e[i]);
    } else {
      e[i] = 0.0f;
      key[i] = 0;
    }
  }
  // keep the 2n-2 largest magnitudes; equal keys keep the lower index
  uint32_t nz = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i >= width) break;
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= width) break;
      rank += (j < i) ? (key[j] >= key[i]) : (j > i ? (key[j] > key[i]) : 0);
    }
    if (rank < width - 2 && key[i] != 0) nz |= 1u << i;
  }
  // windows in order take unassigned nonzeros of their span, lowest first, up to two
  uint32_t claimed = 0, mine = 0;
  for (int ww = 0; ww <= w; ++ww) {
    uint32_t cand = nz & ~claimed & (0xFu << (2 * ww));
    const uint32_t m1 = cand & (0u - cand);
    cand &= ~m1;
    const uint32_t m2 = cand & (0u - cand);
    mine = m1 | m2;
    claimed |= mine;
  }
  return mine >> (2 * w);  // 4-bit mask relative to the window start
}

// OUT: 0 = int8, 1 = fp8, 2 = bf16
template <typename TIn, int OUT>
__global__ __launch_bounds__(kBlock) void slide_kernel(const TIn* __restrict__ W, int64_t ldw, int64_t K, int n,
                                                       uint8_t* __restrict__ vals, int64_t ldv_bytes,
                                                       uint8_t* __restrict__ meta, int64_t ldm, int64_t Kc,
                                                       float* __restrict__ scale) {
  __shared__ float red[kBlock / 64];
  const int64_t row = blockIdx.x;
  const TIn* wr = W + row * ldw;
  uint8_t* vr = vals + row * ldv_bytes;
  uint8_t* mr = meta + row * ldm;
  const int tid = threadIdx.x;

  bool zero_row = false;
  float inv = 0.0f;
  if constexpr (OUT != 2) {
    float amax = 0.0f;
    for (int64_t k = tid; k < K; k += kBlock) amax = fmaxf(amax, fabsf(load_elem<TIn>(wr, k, K)));
    amax = block_max(amax, red);
    constexpr float Q = (OUT == 1) ? 448.0f : 127.0f;
    zero_row = (amax == 0.0f);
    inv = zero_row ? 0.0f : Q / amax;
    if (tid == 0) scale[row] = zero_row ? 0.0f : amax / Q;
  }
  const int64_t groups = (K + 2 * n - 1) / (2 * n);
  const int64_t windows = groups * (n - 1);
  const int64_t units = Kc / 16;
  for (int64_t un = tid; un < units; un += kBlock) {
    uint32_t mt = 0;
    float kv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t t = un * 4 + q;
      uint32_t own = 0;
      float e[16];
      int w = 0;
      if (t < windows) {
        const int64_t g = t / (n - 1);
        w = (int)(t - g * (n - 1));
        own = window_owned<TIn>(wr, K, n, g, w, e);
      }
      // slots: owned positions, then the lowest free positions, ascending
      uint32_t fill = own;
      while (__builtin_popcount(fill) < 2) fill |= (~fill) & (fill + 1);
      const uint32_t i0 = __builtin_ctz(fill), i1 = __builtin_ctz(fill & (fill - 1));
      mt |= (i0 | (i1 << 2)) << (4 * q);
      kv[2 * q] = (own >> i0 & 1) ? e[2 * w + i0] : 0.0f;
      kv[2 * q + 1] = (own >> i1 & 1) ? e[2 * w + i1] : 0.0f;
    }
    *reinterpret_cast<uint16_t*>(mr + un * 2) = (uint16_t)mt;
    if constexpr (OUT == 2) {
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (uint32_t)f32_to_bf16(kv[2 * i]) | ((uint32_t)f32_to_bf16(kv[2 * i + 1]) << 16);
      *reinterpret_cast<uint4*>(vr + un * 16) = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      uint32_t o[2] = {0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t c = zero_row ? 0u : (uint32_t)Quant<OUT == 1>::code(kv[i], inv);
        o[i >> 2] |= c << (8 * (i & 3));
      }
      *reinterpret_cast<uint2*>(vr + un * 8) = make_uint2(o[0], o[1]);
    }
  }
}

template <typename TIn>
static hipError_t launch_sl(int out, const TIn* W, int64_t ldw, int64_t rows, int64_t K, int n, void* vals,
                            int64_t ldv_bytes, uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  dim3 grid((unsigned)rows), block(kBlock);
  uint8_t* v = static_cast<uint8_t*>(vals);
  switch (out) {
    case 0: hipLaunchKernelGGL((slide_kernel<TIn, 0>), grid, block, 0, st, W, ldw, K, n, v, ldv_bytes, meta, ldm, Kc, scale); break;
    case 1: hipLaunchKernelGGL((slide_kernel<TIn, 1>), grid, block, 0, st, W, ldw, K, n, v, ldv_bytes, meta, ldm, Kc, scale); break;
    default: hipLaunchKernelGGL((slide_kernel<TIn, 2>), grid, block, 0, st, W, ldw, K, n, v, ldv_bytes, meta, ldm, Kc, scale); break;
  }
  return hipGetLastError();
}

hipError_t launch_slide(bool in_bf16, int out, const void* W, int64_t ldw, int64_t rows, int64_t K, int n, void* vals,
                        int64_t ldv_bytes, uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  if (in_bf16)
    return launch_sl<uint16_t>(out, static_cast<const uint16_t*>(W), ldw, rows, K, n, vals, ldv_bytes, meta, ldm, Kc, scale, st);
  return launch_sl<float>(out, static_cast<const float*>(W), ldw, rows, K, n, vals, ldv_bytes, meta, ldm, Kc, scale, st);
}

}  // namespace ss
