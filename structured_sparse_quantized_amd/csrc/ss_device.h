// Device-side helpers shared by the gfx950 kernels: element codecs, the
// per-row symmetric quantiser, the 2:4 selection network and block reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

constexpr int kBlock = 256;  // threads per workgroup for the streaming kernels

// ---- element codecs --------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float32 -> bfloat16, nearest with ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two float32 -> two bfloat16 in one word (lo in the low half) by gfx950's packed conversion instruction:
// nearest with ties to even, equal to f32_to_bf16 on every non-NaN input (denormals included); a NaN leaves
// as a quiet NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Magnitude key: for finite floats the unsigned order of the bits without the
// sign is the order of |v|, and +0 / -0 share key 0.
__device__ __forceinline__ uint32_t mag_key_f32(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }
__device__ __forceinline__ uint32_t mag_key_bf16(uint16_t b) { return (uint32_t)(b & 0x7FFFu); }

// ---- per-row symmetric quantisation ----------------------------------------
// Q = 127 (INT8) or 448 (FP8 E4M3FN). inv = Q / a is correctly rounded (HIP's
// default single-precision division); products use __fmul_rn so nothing fuses.
template <bool FP8> struct Quant {
  static constexpr float Q = FP8 ? 448.0f : 127.0f;
  __device__ __forceinline__ static uint8_t code(float v, float inv) {
    float t = __fmul_rn(v, inv);
    if constexpr (FP8) {
      t = fminf(fmaxf(t, -448.0f), 448.0f);
      // OCP E4M3FN, nearest-even (gfx950 conversion unit)
      return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(t, 0.0f, 0, false) & 0xFF);
    } else {
      float r = rintf(t);  // ties to even
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      return (uint8_t)(int8_t)(int)r;
    }
  }
  // Four codes packed little-endian, the same bytes as code(). INT8: clamp to
  // +-127 (integers, so clamping before rounding is the same), then add
  // 1.5 * 2^23: the sum's low mantissa bits hold rint(t) in two's complement.
  // FP8: two conversions of two values each. A zero row (inv = 0) gives zero
  // INT8 codes but FP8 -0 codes (0x80) for negative zeros: the caller masks it.
  __device__ __forceinline__ static uint32_t pack4(float a, float b, float c, float d, float inv) {
    if constexpr (FP8) {
      auto t = [&](float v) { return __builtin_amdgcn_fmed3f(__fmul_rn(v, inv), -448.0f, 448.0f); };
      const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(t(a), t(b), 0, false);
      return __builtin_amdgcn_cvt_pk_fp8_f32(t(c), t(d), lo, true);
    } else {
      auto t = [&](float v) {
        return __float_as_uint(__builtin_amdgcn_fmed3f(__fmul_rn(v, inv), -127.0f, 127.0f) + 12582912.0f);
      };
      return __builtin_amdgcn_perm(t(b), t(a), 0x0C0C0400u) | __builtin_amdgcn_perm(t(d), t(c), 0x04000C0Cu);
    }
  }
};

// ---- 2:4 selection ----------------------------------------------------------
// Keep the two largest keys of a 4-group; equal keys keep the lower index.
// Returns the nibble idx0 | idx1 << 2 with idx0 < idx1.
__device__ __forceinline__ uint32_t top2_nibble(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3) {
  // rank = number of elements that outrank this one
  const int r0 = (k1 > k0) + (k2 > k0) + (k3 > k0);
  const int r1 = (k0 >= k1) + (k2 > k1) + (k3 > k1);
  const int r2 = (k0 >= k2) + (k1 >= k2) + (k3 > k2);
  const int r3 = (k0 >= k3) + (k1 >= k3) + (k2 >= k3);
  const uint32_t m = (uint32_t)(r0 < 2) | ((uint32_t)(r1 < 2) << 1) | ((uint32_t)(r2 < 2) << 2) |
                     ((uint32_t)(r3 < 2) << 3);
  const uint32_t i0 = __builtin_ctz(m);
  const uint32_t i1 = __builtin_ctz(m & (m - 1));
  return i0 | (i1 << 2);
}

// ---- activation lift by periods ---------------------------------------------------
// The lift writes window w of 2n-group g as four codes, X'[4(n-1)g + 4w + j] = X[2n g + 2w + j] (SlideSparse
// article, activation lifting; SlideSparse blog, section 3.2). Its byte pattern is periodic: PC output chunks
// of 16 bytes (4 windows each) hold whole groups and come from SB consecutive source bytes (SB a multiple of
// 4, so a period starts on a word). A thread that owns a period reads its SW source words once and forms the
// 4 PC output words with shifts whose amounts are compile-time constants.
// chunks per period for pattern n (n >= 3): the fewest whole groups that fill whole chunks from whole words
__host__ __device__ constexpr int lift_period_chunks(int n) {
  int p = 1;
  while ((4 * p) % (n - 1) != 0 || (2 * n * (4 * p / (n - 1))) % 4 != 0) ++p;
  return p;
}
__host__ __device__ constexpr int lift_period_bytes(int n) { return 2 * n * (4 * lift_period_chunks(n) / (n - 1)); }
template <int N> struct LiftPeriod {
  static constexpr int WPG = N - 1;                 // windows per group
  static constexpr int PC = lift_period_chunks(N);  // output chunks per period
  static constexpr int SB = lift_period_bytes(N);   // source bytes per period
  static constexpr int SW = SB / 4;                // source words per period
  // first source byte of output word u of the period: window u lies in group u / WPG at position u % WPG
  static constexpr int src(int u) { return 2 * N * (u / WPG) + 2 * (u % WPG); }
  __device__ __forceinline__ static void emit(const uint32_t* s, uint32_t* out) {
#pragma unroll
    for (int u = 0; u < 4 * PC; ++u) {
      const int b = src(u);  // even: a window starts on a byte pair
      out[u] = (b & 2) ? ((s[b >> 2] >> 16) | (s[(b >> 2) + 1] << 16)) : s[b >> 2];
    }
  }
};

// ---- tiled-layout row order ---------------------------------------------------
// Workgroups are dealt to the 8 XCDs round-robin by index. Kernels that write
// one row of the tiled operand per workgroup (or per persistent iteration i)
// take row xcd_row(i, n) so that the 16 rows of a 16-row block, whose 16-byte
// pieces share 128-byte lines, are written through one XCD's L2 and leave it
// as whole lines. A bijection on [0, n): blocks of 128 indices map within
// themselves, the tail (n % 128) maps to itself.
__device__ __forceinline__ int xcd_row(int i, int n) {
  if (i >= (n & ~127)) return i;
  const int x = i & 7, j = i >> 3;
  return ((((j >> 4) << 3) + x) << 4) + (j & 15);
}

// ---- reductions ---------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Workgroup barrier that orders LDS accesses only. A full __syncthreads() also
// waits for every global load in flight (vmcnt(0)), which would stall a row
// prefetched into registers before the barrier; this one waits for LDS
// operations (lgkmcnt) alone. Use it where the barrier guards LDS data only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Block-wide max over kBlock threads; every thread gets the result.
__device__ __forceinline__ float block_max(float v, float* red /* >= kBlock/64 floats */) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = v;
  lds_barrier();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kBlock / 64; ++i) r = fmaxf(r, red[i]);
  lds_barrier();
  return r;
}

}  // namespace ss
