// Fused per-token quantisation + activation lift (SlideSparse article,
// activation-lifting paragraph; SlideSparse blog section 3.2): one pass reads
// a token row, reduces its absmax, quantises, and writes the row gathered into
// window order X'[4(n-1)g + 4w + j] = q(X[2n g + 2w + j]), zero-padded to Kc.
//
// One workgroup per token row. The row is held in registers between the
// absmax reduction and the quantisation, so X is read from HBM once; for the
// lift the codes are staged in LDS and gathered into 16-byte output chunks.
#include "ss_device.h"
#include "ss_kernels.h"

namespace ss {

template <typename TIn> struct InVec;
template <> struct InVec<uint16_t> {  // 8 bf16 per 16-byte vector
  static constexpr int E = 8;
  __device__ static float get(const uint4& v, int i) {
    const uint32_t w = (&v.x)[i >> 1];
    return bf16_to_f32((uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFF)));
  }
  __device__ static float scalar(const uint16_t* p) { return bf16_to_f32(*p); }
};
template <> struct InVec<float> {  // 4 float per 16-byte vector
  static constexpr int E = 4;
  __device__ static float get(const uint4& v, int i) { return __uint_as_float((&v.x)[i]); }
  __device__ static float scalar(const float* p) { return *p; }
};

// VPT = 16-byte vectors per thread held in registers (row fits when
// K <= kBlock * VPT * E; the host picks VPT).
template <typename TIn, bool FP8, int VPT>
__global__ __launch_bounds__(kBlock) void quant_lift_kernel(const TIn* __restrict__ X, int64_t ldx, int64_t K,
                                                            int n, uint8_t* __restrict__ Xq, int64_t ldq,
                                                            int64_t Kc, float* __restrict__ sx) {
  using V = InVec<TIn>;
  constexpr int E = V::E;
  extern __shared__ __align__(16) uint8_t lds[];  // [Kpad] codes (lift only)
  __shared__ float red[kBlock / 64];

  const int64_t row = blockIdx.x;
  const TIn* xr = X + row * ldx;
  uint8_t* qr = Xq + row * ldq;
  const int tid = threadIdx.x;
  const int64_t nvec = K / E;  // full vectors; the K % E tail is read scalar

  uint4 v[VPT];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int64_t vi = tid + (int64_t)i * kBlock;
    if (vi < nvec) {
      v[i] = reinterpret_cast<const uint4*>(xr)[vi];
#pragma unroll
      for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(V::get(v[i], e)));
    } else {
      v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  const int64_t tail0 = nvec * E;
  float tailv = 0.0f;
  if (tail0 + tid < K) {
    tailv = V::scalar(xr + tail0 + tid);
    amax = fmaxf(amax, fabsf(tailv));
  }
  amax = block_max(amax, red);

  using Qz = Quant<FP8>;
  const bool zero_row = (amax == 0.0f);
  const float inv = zero_row ? 0.0f : Qz::Q / amax;
  if (tid == 0) sx[row] = zero_row ? 0.0f : amax / Qz::Q;

  auto code = [&](float f) -> uint32_t { return zero_row ? 0u : (uint32_t)Qz::code(f, inv); };

  if (n == 2) {
    // no lift: codes go straight out; then zero padding up to Kc
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t vi = tid + (int64_t)i * kBlock;
      if (vi < nvec) {
        if constexpr (E == 8) {
          uint2 o;
          o.x = code(V::get(v[i], 0)) | code(V::get(v[i], 1)) << 8 | code(V::get(v[i], 2)) << 16 |
                code(V::get(v[i], 3)) << 24;
          o.y = code(V::get(v[i], 4)) | code(V::get(v[i], 5)) << 8 | code(V::get(v[i], 6)) << 16 |
                code(V::get(v[i], 7)) << 24;
          *reinterpret_cast<uint2*>(qr + vi * 8) = o;
        } else {
          const uint32_t o = code(V::get(v[i], 0)) | code(V::get(v[i], 1)) << 8 | code(V::get(v[i], 2)) << 16 |
                             code(V::get(v[i], 3)) << 24;
          *reinterpret_cast<uint32_t*>(qr + vi * 4) = o;
        }
      }
    }
    if (tail0 + tid < K) qr[tail0 + tid] = (uint8_t)code(tailv);
    for (int64_t c = K + tid; c < Kc; c += kBlock) qr[c] = 0;
    return;
  }

  // lift: stage codes of the (zero-padded) row in LDS, then gather windows
  const int64_t Kpad = (K + 2 * n - 1) / (2 * n) * (2 * n);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int64_t vi = tid + (int64_t)i * kBlock;
    if (vi < nvec) {
#pragma unroll
      for (int e = 0; e < E; ++e) lds[vi * E + e] = (uint8_t)code(V::get(v[i], e));
    }
  }
  if (tail0 + tid < K) lds[tail0 + tid] = (uint8_t)code(tailv);
  for (int64_t c = K + tid; c < Kpad; c += kBlock) lds[c] = 0;
  __syncthreads();

  const int64_t kl = Kpad / (2 * n) * 4 * (n - 1);  // logical K'
  const int64_t nchunk = Kc / 16;
  const uint16_t* l16 = reinterpret_cast<const uint16_t*>(lds);
  for (int64_t c = tid; c < nchunk; c += kBlock) {
    uint32_t w4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t t = c * 4 + q;  // flat window index
      if (4 * t < kl) {
        const int64_t g = t / (n - 1), w = t - g * (n - 1);
        const int64_t base = 2 * n * g + 2 * w;  // even, so two aligned halves
        w4[q] = (uint32_t)l16[base >> 1] | ((uint32_t)l16[(base >> 1) + 1] << 16);
      } else {
        w4[q] = 0;
      }
    }
    *reinterpret_cast<uint4*>(qr + c * 16) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
}

// Rows too long for the register path: two passes over global memory.
template <typename TIn, bool FP8>
__global__ __launch_bounds__(kBlock) void quant_lift_long_kernel(const TIn* __restrict__ X, int64_t ldx, int64_t K,
                                                                 int n, uint8_t* __restrict__ Xq, int64_t ldq,
                                                                 int64_t Kc, float* __restrict__ sx) {
  using V = InVec<TIn>;
  __shared__ float red[kBlock / 64];
  const int64_t row = blockIdx.x;
  const TIn* xr = X + row * ldx;
  uint8_t* qr = Xq + row * ldq;
  float amax = 0.0f;
  for (int64_t k = threadIdx.x; k < K; k += kBlock) amax = fmaxf(amax, fabsf(V::scalar(xr + k)));
  amax = block_max(amax, red);
  using Qz = Quant<FP8>;
  const bool zero_row = (amax == 0.0f);
  const float inv = zero_row ? 0.0f : Qz::Q / amax;
  if (threadIdx.x == 0) sx[row] = zero_row ? 0.0f : amax / Qz::Q;
  const int64_t Kpad = (K + 2 * n - 1) / (2 * n) * (2 * n);
  const int64_t kl = Kpad / (2 * n) * 4 * (n - 1);
  for (int64_t kp = threadIdx.x; kp < Kc; kp += kBlock) {
    uint8_t q = 0;
    if (kp < kl) {
      const int64_t t = kp >> 2, j = kp & 3;
      const int64_t g = t / (n - 1), w = t - g * (n - 1);
      const int64_t src = 2 * n * g + 2 * w + j;
      if (src < K && !zero_row) q = Qz::code(V::scalar(xr + src), inv);
    }
    qr[kp] = q;
  }
}

template <typename TIn, bool FP8>
static hipError_t launch_ql(const TIn* X, int64_t ldx, int64_t M, int64_t K, int n, uint8_t* Xq, int64_t ldq,
                            int64_t Kc, float* sx, hipStream_t st) {
  constexpr int E = InVec<TIn>::E;
  const int64_t nvec = K / E;
  const int64_t vpt = (nvec + kBlock - 1) / kBlock;
  const size_t lds = (n == 2) ? 0 : (size_t)(((K + 2 * n - 1) / (2 * n) * (2 * n) + 15) / 16 * 16);
  dim3 grid((unsigned)M), block(kBlock);
  if (lds <= 64 * 1024) {
    if (vpt <= 1) { hipLaunchKernelGGL((quant_lift_kernel<TIn, FP8, 1>), grid, block, lds, st, X, ldx, K, n, Xq, ldq, Kc, sx); return hipGetLastError(); }
    if (vpt <= 2) { hipLaunchKernelGGL((quant_lift_kernel<TIn, FP8, 2>), grid, block, lds, st, X, ldx, K, n, Xq, ldq, Kc, sx); return hipGetLastError(); }
    if (vpt <= 4) { hipLaunchKernelGGL((quant_lift_kernel<TIn, FP8, 4>), grid, block, lds, st, X, ldx, K, n, Xq, ldq, Kc, sx); return hipGetLastError(); }
    if (vpt <= 8) { hipLaunchKernelGGL((quant_lift_kernel<TIn, FP8, 8>), grid, block, lds, st, X, ldx, K, n, Xq, ldq, Kc, sx); return hipGetLastError(); }
    if (vpt <= 12) { hipLaunchKernelGGL((quant_lift_kernel<TIn, FP8, 12>), grid, block, lds, st, X, ldx, K, n, Xq, ldq, Kc, sx); return hipGetLastError(); }
  }
  hipLaunchKernelGGL((quant_lift_long_kernel<TIn, FP8>), grid, block, 0, st, X, ldx, K, n, Xq, ldq, Kc, sx);
  return hipGetLastError();
}

hipError_t launch_quant_lift(bool x_bf16, bool fp8, const void* X, int64_t ldx, int64_t M, int64_t K, int n,
                             void* Xq, int64_t ldq, int64_t Kc, float* sx, hipStream_t st) {
  uint8_t* q = static_cast<uint8_t*>(Xq);
  if (x_bf16) {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    return fp8 ? launch_ql<uint16_t, true>(x, ldx, M, K, n, q, ldq, Kc, sx, st)
               : launch_ql<uint16_t, false>(x, ldx, M, K, n, q, ldq, Kc, sx, st);
  }
  const float* x = static_cast<const float*>(X);
  return fp8 ? launch_ql<float, true>(x, ldx, M, K, n, q, ldq, Kc, sx, st)
             : launch_ql<float, false>(x, ldx, M, K, n, q, ldq, Kc, sx, st);
}

}  // namespace ss
