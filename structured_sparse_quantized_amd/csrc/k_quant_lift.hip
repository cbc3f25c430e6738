// Fused per-token quantisation + activation lift (SlideSparse article,
// activation-lifting paragraph; SlideSparse blog section 3.2): one pass reads a
// token row, reduces its absmax, quantises, and writes the row gathered into
// window order X'[4(n-1)g + 4w + j] = q(X[2n g + 2w + j]), zero-padded to Kc.
//
// Persistent workgroups walk rows r, r + grid, ...; the next row is loaded
// into registers before the current one is reduced and written, so HBM reads
// and writes overlap. For n > 2 the codes of a row are staged in LDS (zero past
// K) and each thread forms whole periods of the lift's byte pattern
// (LiftPeriod): the period's source words read once, its 16-byte output chunks
// built with constant shifts.
#include "ss_device.h"
#include "ss_kernels.h"

#include <algorithm>

namespace ss {
namespace {

// The input row is read once, so its loads are non-temporal (they leave the caches to the data that is
// read again): 1.03-1.20x on 2048-16384 token batches timed alone, and within the product that follows the
// step is no slower (1.000-1.024x). The codes take ordinary stores: the product reads them next, and
// non-temporal stores cost it 1-1.4% of the step.
typedef unsigned int nt_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const nt_u4 t = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void st_stream(uint8_t* p, uint32_t a, uint32_t b) {  // 8-byte aligned
  *reinterpret_cast<uint2*>(p) = make_uint2(a, b);
}
__device__ __forceinline__ void st_stream(uint8_t* p, uint32_t a, uint32_t b, uint32_t c) {  // 4-byte aligned
  uint32_t* o = reinterpret_cast<uint32_t*>(p);
  o[0] = a;
  o[1] = b;
  o[2] = c;
}
__device__ __forceinline__ void st_stream(uint8_t* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {  // 16-byte
  *reinterpret_cast<uint4*>(p) = make_uint4(a, b, c, d);
}

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

// VPT = 16-byte vectors per thread (the row fits when K <= kBlock*VPT*E).
template <typename TIn, bool FP8, int N, int VPT, bool PIPE>
__global__ __launch_bounds__(kBlock, (PIPE || VPT > 4) ? 2 : (VPT > 2 ? 4 : 8)) void quant_lift_kernel(const TIn* __restrict__ X, int64_t ldx, int M, int K,
                                                            uint8_t* __restrict__ Xq, int64_t ldq, int Kc,
                                                            float* __restrict__ sx) {
  using V = InVec<TIn>;
  constexpr int E = V::E;
  using Qz = Quant<FP8>;
  extern __shared__ __align__(16) uint8_t lds[];  // codes of one padded row (lift only)
  __shared__ float red[kBlock / 64];
  const int tid = threadIdx.x;
  const int nvec = K / E, tail0 = nvec * E;
  const int Kpad = (K + 2 * N - 1) / (2 * N) * (2 * N);
  const int kl = Kpad / (2 * N) * 4 * (N - 1);  // logical K'

  uint4 cur[VPT], nxt[PIPE ? VPT : 1];
  float ctail = 0.0f, ntail = 0.0f;
  auto load = [&](uint4* v, float& tl, int r) {
    const TIn* xr = X + (int64_t)r * ldx;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int vi = tid + i * kBlock;
      v[i] = vi < nvec ? ld_stream(reinterpret_cast<const uint4*>(xr) + vi) : make_uint4(0, 0, 0, 0);
    }
    tl = (tail0 + tid < K) ? V::scalar(xr + tail0 + tid) : 0.0f;
  };

  int r = blockIdx.x;
  if (r < M) load(cur, ctail, r);
  for (; r < M; r += gridDim.x) {
    const int rn = r + gridDim.x;
    if (PIPE && rn < M) load(nxt, ntail, rn);

    float amax = fabsf(ctail);
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(V::get(cur[i], e)));
    amax = block_max(amax, red);
    const bool zero_row = (amax == 0.0f);
    const float inv = zero_row ? 0.0f : Qz::Q / amax;
    if (tid == 0) sx[r] = zero_row ? 0.0f : amax / Qz::Q;
    auto code = [&](float f) -> uint32_t { return zero_row ? 0u : (uint32_t)Qz::code(f, inv); };
    // four codes of vector i from element e0 (same bytes as code())
    auto code4 = [&](const uint4& v, int e0) -> uint32_t {
      return zero_row ? 0u : Qz::pack4(V::get(v, e0), V::get(v, e0 + 1), V::get(v, e0 + 2), V::get(v, e0 + 3), inv);
    };
    uint8_t* qr = Xq + (int64_t)r * ldq;

    if constexpr (N == 2) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int vi = tid + i * kBlock;
        if (vi < nvec) {
          if constexpr (E == 8) {
            uint2 o;
            o.x = code4(cur[i], 0);
            o.y = code4(cur[i], 4);
            st_stream(qr + vi * 8, o.x, o.y);
          } else {
            *reinterpret_cast<uint32_t*>(qr + vi * 4) =
                code4(cur[i], 0);
          }
        }
      }
      if (tail0 + tid < K) qr[tail0 + tid] = (uint8_t)code(ctail);
      for (int c = K + tid; c < Kc; c += kBlock) qr[c] = 0;
    } else if (N == 4 && E == 8 && (K & 7) == 0) {
      // 6:8 from bf16 with whole 8-groups: a thread's vector is one group g, and its three windows
      // (positions 2w .. 2w+3) are bytes 0-3, 2-5 and 4-7 of its eight codes -- written straight to
      // X'[12g .. 12g+11] without the LDS gather
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int vi = tid + i * kBlock;
        if (vi < nvec) {
          const uint32_t lo = code4(cur[i], 0), hi = code4(cur[i], 4);
          st_stream(qr + vi * 12, lo, (lo >> 16) | (hi << 16), hi);
        }
      }
      for (int c = kl + tid; c < Kc; c += kBlock) qr[c] = 0;
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int vi = tid + i * kBlock;
        if (vi < nvec) {
          if constexpr (E == 8) {
            uint2 o;
            o.x = code4(cur[i], 0);
            o.y = code4(cur[i], 4);
            *reinterpret_cast<uint2*>(lds + vi * 8) = o;
          } else {
            *reinterpret_cast<uint32_t*>(lds + vi * 4) =
                code4(cur[i], 0);
          }
        }
      }
      if (tail0 + tid < K) lds[tail0 + tid] = (uint8_t)code(ctail);
      // zero past K through the last period's source bytes: windows past the last group read zeros, so
      // the output from the logical K' to Kc is zero
      using LP = LiftPeriod<N>;
      const int nchunk = Kc / 16, nper = (nchunk + LP::PC - 1) / LP::PC;
      for (int c = K + tid; c < nper * LP::SB; c += kBlock) lds[c] = 0;
      lds_barrier();
      const uint32_t* l32 = reinterpret_cast<const uint32_t*>(lds);
      for (int p = tid; p < nper; p += kBlock) {
        uint32_t s[LP::SW], o[4 * LP::PC];
#pragma unroll
        for (int i = 0; i < LP::SW; ++i) s[i] = l32[p * LP::SW + i];
        LP::emit(s, o);
#pragma unroll
        for (int h = 0; h < LP::PC; ++h)
          if (p * LP::PC + h < nchunk)
            st_stream(qr + (p * LP::PC + h) * 16, o[4 * h], o[4 * h + 1], o[4 * h + 2], o[4 * h + 3]);
      }
      lds_barrier();  // the LDS row is rewritten for the next row
    }
    if constexpr (PIPE) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) cur[i] = nxt[i];
      ctail = ntail;
    } else if (rn < M) {
      load(cur, ctail, rn);
    }
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
  // output position kp = 4(n-1) g + 4 w + j takes the code of X[2n g + 2w + j] (zero past K)
  const int64_t gb = 4 * (n - 1);  // output bytes per group
  for (int64_t kp = threadIdx.x; kp < Kc; kp += kBlock) {
    const int64_t g = kp / gb, rem = kp - g * gb;
    const int64_t src = 2 * n * g + 2 * (rem >> 2) + (rem & 3);
    qr[kp] = (src < K && !zero_row) ? Qz::code(V::scalar(xr + src), inv) : 0;
  }
}

template <typename TIn, bool FP8, int N>
hipError_t launch_n(const TIn* X, int64_t ldx, int64_t M, int64_t K, uint8_t* Xq, int64_t ldq, int64_t Kc, float* sx,
                    hipStream_t st) {
  constexpr int E = InVec<TIn>::E;
  const int64_t vpt = (K / E + kBlock - 1) / kBlock;
  const int64_t kpad = (K + 2 * N - 1) / (2 * N) * (2 * N);
  // codes staged in LDS for the gather, except without a lift and for 6:8 from bf16 with whole 8-groups
  const bool reg_lift = N == 4 && E == 8 && K % 8 == 0;
  using LP = LiftPeriod<N < 3 ? 3 : N>;
  const int64_t nper = (Kc / 16 + LP::PC - 1) / LP::PC;  // periods of the lift pattern covering the row
  const size_t lds = (N == 2 || reg_lift) ? 0 : (size_t)((std::max<int64_t>(nper * LP::SB, kpad) + 15) / 16 * 16);
  const bool fits = K < (1 << 30) && Kc < (1 << 30) && M < (1 << 30) && lds <= 64 * 1024 && vpt <= 12;
  if (!fits) {
    hipLaunchKernelGGL((quant_lift_long_kernel<TIn, FP8>), dim3((unsigned)M), dim3(kBlock), 0, st, X, ldx, K, N, Xq, ldq, Kc, sx);
    return hipGetLastError();
  }
  // One row per workgroup keeps the most loads in flight for batches up to a few
  // thousand rows; larger batches use persistent workgroups that prefetch, as many per CU as fit at once
  // (registers and LDS; at most 8): a grid larger than what fits runs its last workgroups as a partly filled
  // extra round (a fixed 8 per CU was 1.02x slower on 16384 x 14336, 1.07x on the 6:8 lift at 16384 tokens).
  const bool pipe = M > 16 * (int64_t)num_cus_p();
  const int m = (int)M, k = (int)K, kc = (int)Kc;
#define SS_QL(V_) \
  do { if (pipe) hipLaunchKernelGGL((quant_lift_kernel<TIn, FP8, N, V_, true>), dim3((unsigned)(std::min(occupancy_p((const void*)quant_lift_kernel<TIn, FP8, N, V_, true>, kBlock, lds), 8) * num_cus_p())), dim3(kBlock), lds, st, X, ldx, m, k, Xq, ldq, kc, sx); else hipLaunchKernelGGL((quant_lift_kernel<TIn, FP8, N, V_, false>), dim3((unsigned)M), dim3(kBlock), lds, st, X, ldx, m, k, Xq, ldq, kc, sx); } while (0)
  if (vpt <= 1) SS_QL(1);
  else if (vpt <= 2) SS_QL(2);
  else if (vpt <= 4) SS_QL(4);
  else if (vpt <= 8) SS_QL(8);
  else SS_QL(12);
#undef SS_QL
  return hipGetLastError();
}

template <typename TIn, bool FP8>
hipError_t launch_ql(const TIn* X, int64_t ldx, int64_t M, int64_t K, int n, uint8_t* Xq, int64_t ldq, int64_t Kc,
                     float* sx, hipStream_t st) {
  switch (n) {
    case 2: return launch_n<TIn, FP8, 2>(X, ldx, M, K, Xq, ldq, Kc, sx, st);
    case 3: return launch_n<TIn, FP8, 3>(X, ldx, M, K, Xq, ldq, Kc, sx, st);
    case 4: return launch_n<TIn, FP8, 4>(X, ldx, M, K, Xq, ldq, Kc, sx, st);
    case 5: return launch_n<TIn, FP8, 5>(X, ldx, M, K, Xq, ldq, Kc, sx, st);
    case 6: return launch_n<TIn, FP8, 6>(X, ldx, M, K, Xq, ldq, Kc, sx, st);
    case 7: return launch_n<TIn, FP8, 7>(X, ldx, M, K, Xq, ldq, Kc, sx, st);
    default: return launch_n<TIn, FP8, 8>(X, ldx, M, K, Xq, ldq, Kc, sx, st);
  }
}

// Block-scaled FP8 activations (LLM Compressor guide, W8A8-FP8_BLOCK: one dynamic scale per token and
// group of 128 positions along K): 16 lanes per group, 8 positions per lane, the group absmax reduced
// across the 16 lanes; a workgroup covers 16 groups of one token (1-D grid: token-major). Positions past
// K read as zero, so groups wholly past K (the padding up to Kc) get zero codes and scale 0.
template <typename TIn>
__global__ __launch_bounds__(kBlock) void quant_group_kernel(const TIn* __restrict__ X, int64_t ldx, int K, int G,
                                                             int gblocks, uint8_t* __restrict__ Xq, int64_t ldq,
                                                             float* __restrict__ sx) {
  using V = InVec<TIn>;
  const int64_t m = blockIdx.x / gblocks;
  const int g = (blockIdx.x % gblocks) * (kBlock / 16) + (threadIdx.x >> 4), l = threadIdx.x & 15;
  if (g >= G) return;  // whole 16-lane groups leave together
  const int k0 = g * 128 + l * 8;
  const TIn* xr = X + m * ldx;
  float v[8];
  if (k0 + 8 <= K) {
#pragma unroll
    for (int h = 0; h < 8 / V::E; ++h) {
      const uint4 q = reinterpret_cast<const uint4*>(xr + k0)[h];
#pragma unroll
      for (int i = 0; i < V::E; ++i) v[h * V::E + i] = V::get(q, i);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (k0 + i < K) ? V::scalar(xr + k0 + i) : 0.0f;
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 16));
  const bool zero = a == 0.0f;
  const float inv = zero ? 0.0f : Quant<true>::Q / a;
  uint2 c = make_uint2(0u, 0u);
  if (!zero) c = make_uint2(Quant<true>::pack4(v[0], v[1], v[2], v[3], inv), Quant<true>::pack4(v[4], v[5], v[6], v[7], inv));
  *reinterpret_cast<uint2*>(Xq + m * ldq + k0) = c;
  if (l == 0) sx[m * G + g] = zero ? 0.0f : a / Quant<true>::Q;
}

}  // namespace

hipError_t launch_quant_group(bool x_bf16, const void* X, int64_t ldx, int64_t M, int64_t K, void* Xq, int64_t ldq,
                              int64_t Kc, float* sx, hipStream_t st) {
  const int G = (int)(Kc / 128), gblocks = (G + kBlock / 16 - 1) / (kBlock / 16);
  const dim3 grid((unsigned)(M * gblocks));
  uint8_t* q = static_cast<uint8_t*>(Xq);
  if (x_bf16)
    hipLaunchKernelGGL(quant_group_kernel<uint16_t>, grid, dim3(kBlock), 0, st, static_cast<const uint16_t*>(X), ldx,
                       (int)K, G, gblocks, q, ldq, sx);
  else
    hipLaunchKernelGGL(quant_group_kernel<float>, grid, dim3(kBlock), 0, st, static_cast<const float*>(X), ldx, (int)K,
                       G, gblocks, q, ldq, sx);
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
