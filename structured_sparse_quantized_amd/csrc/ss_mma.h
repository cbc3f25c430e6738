// The gfx950 structured-sparse matrix instructions behind one interface, shared by the product kernels
// (internal to the library). One instruction multiplies a 16-row block of the compressed operand (two of
// every four positions along K kept, a 2-bit position each; Deep reading of arXiv 2610.28947, introduction)
// by 16 rows of the dense operand: 128 positions of K for 8-bit codes (v_smfmac_*_16x16x128), 64 for bf16
// (v_smfmac_f32_16x16x64_bf16).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ss {
namespace tiled {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v16bf __attribute__((ext_vector_type(16)));

// AB: 0 = int8, 1 = fp8 (16x16x128), 2 = bf16 (16x16x64; HALF selects the 16-bit index half)
template <int AB> struct Mma;
template <> struct Mma<0> {
  using Acc = v4i;
  template <int HALF> __device__ static Acc run(v4i a, v4i b0, v4i b1, Acc c, int idx) {
    return __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), c, idx, 0, 0);
  }
};
template <> struct Mma<1> {
  using Acc = v4f;
  template <int HALF> __device__ static Acc run(v4i a, v4i b0, v4i b1, Acc c, int idx) {
    return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), c, idx,
                                                          0, 0);
  }
};
template <> struct Mma<2> {
  using Acc = v4f;
  template <int HALF> __device__ static Acc run(v4i a, v4i b0, v4i b1, Acc c, int idx) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
        __builtin_bit_cast(v8bf, a), __builtin_bit_cast(v16bf, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7)), c,
        idx, 0, HALF);
  }
};

// Per element size: index bytes per lane per step, and the block of one row block's 4-step index group.
template <int AB> struct Meta {
  static constexpr int ES = AB == 2 ? 2 : 1;  // value bytes
  static constexpr int WB = 4 / ES;           // index bytes per lane per step
  static constexpr int BLOCK = 256 * WB;      // bytes of one row block's 4-step group
  using V = typename std::conditional<AB == 2, v2i, v4i>::type;
  // the 32-bit word holding step q's index (bf16: two steps per word)
  __device__ static int word(const V& m, int q) { return AB == 2 ? m[q >> 1] : m[q]; }
};
// one instruction with step q's index
template <int AB, int Q, typename Acc>
__device__ __forceinline__ Acc mma_step(v4i a, v4i b0, v4i b1, Acc c, const typename Meta<AB>::V& m) {
  return Mma<AB>::template run<AB == 2 ? (Q & 1) : 0>(a, b0, b1, c, Meta<AB>::word(m, Q));
}

// B rows in LDS: 8 rows x 128 bytes per 1 KB block; chunk c of row r sits at chunk position c ^ (r % 8).
__device__ __forceinline__ int swz(int c, int r16) { return c ^ (r16 & 7); }


}  // namespace tiled
}  // namespace ss
