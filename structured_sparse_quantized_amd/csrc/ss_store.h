// Epilogue store shared by the product kernels (internal to the library).
#pragma once
#include "ss_device.h"

namespace ss {

// Store one lane's 4 results: rows ar..ar+3 of the sparse operand, one dense row bc.
template <int YT, bool SIDE_X>
__device__ __forceinline__ void store_out(void* Y, int64_t ldy, int64_t ar, int64_t bc, int64_t R, const float* y,
                                          const int32_t* yi) {
  if (!SIDE_X && (ldy & 3) == 0 && ar + 3 < R) {  // Y[bc][ar .. ar+3] is one aligned vector
    if constexpr (YT == 0) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Y) + bc * ldy + ar) =
          make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
    } else if constexpr (YT == 1) {
      *reinterpret_cast<float4*>(static_cast<float*>(Y) + bc * ldy + ar) = make_float4(y[0], y[1], y[2], y[3]);
    } else {
      *reinterpret_cast<int4*>(static_cast<int32_t*>(Y) + bc * ldy + ar) = make_int4(yi[0], yi[1], yi[2], yi[3]);
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (ar + q >= R) break;
    const int64_t off = SIDE_X ? (ar + q) * ldy + bc : bc * ldy + ar + q;
    if constexpr (YT == 0) static_cast<uint16_t*>(Y)[off] = f32_to_bf16(y[q]);
    else if constexpr (YT == 1) static_cast<float*>(Y)[off] = y[q];
    else static_cast<int32_t*>(Y)[off] = yi[q];
  }
}

}  // namespace ss
