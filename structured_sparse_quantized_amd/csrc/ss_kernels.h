// Host-callable launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

// Compute units of the current device (cached).
int num_cus_p();
// Raise a kernel's dynamic-LDS limit to `bytes` on the current device (the runtime call runs once per device,
// kernel and larger size).
hipError_t lds_limit(const void* kern, int bytes);
// Resident workgroups per CU (cached per device, kernel, block size and LDS bytes; at least 1).
int occupancy_p(const void* kern, int block, size_t lds);

hipError_t launch_quant_lift(bool x_bf16, bool fp8, const void* X, int64_t ldx, int64_t M, int64_t K, int n,
                             void* Xq, int64_t ldq, int64_t Kc, float* sx, hipStream_t st);

// out: 0 = int8, 1 = fp8, 2 = bf16
hipError_t launch_prune24(bool in_bf16, int out, const void* X, int64_t ldx, int64_t M, int64_t K, void* vals,
                          int64_t ldv_bytes, uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st);

hipError_t launch_slide(bool in_bf16, int out, const void* W, int64_t ldw, int64_t rows, int64_t K, int n, void* vals,
                        int64_t ldv_bytes, uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st);

// ab: 0 = int8, 1 = fp8, 2 = bf16; yt: 0 = bf16, 1 = f32, 2 = i32
hipError_t launch_spgemm(bool side_x, int ab, int yt, int64_t R, int64_t C, int64_t Kc, const void* av,
                         int64_t lda_bytes, const uint8_t* am, int64_t ldm, const void* bd, int64_t ldb_bytes,
                         const float* sx, const float* sw, void* Y, int64_t ldy, hipStream_t st);

// Online 2:4 prune of bf16 activations written in the tiled layout (out: 0 = int8, 1 = fp8, 2 = bf16).
hipError_t launch_prune24_act_tiled(int out, const void* X, int64_t ldx, int64_t M, int64_t K, int64_t Kc, void* tv,
                                    uint8_t* tm, float* sx, hipStream_t st);

// Weight preparation written in the tiled layout: 2:4 (F32 / BF16 input) and the (2n-2):2n decomposition.
hipError_t launch_prune24_tiled(bool in_bf16, int out, const void* W, int64_t ldw, int64_t rows, int64_t K, int64_t Kc,
                                void* tv, uint8_t* tm, float* scale, hipStream_t st);
hipError_t launch_slide_tiled(bool in_bf16, int out, const void* W, int64_t ldw, int64_t rows, int64_t K, int n,
                              int64_t Kc, void* tv, uint8_t* tm, float* scale, hipStream_t st);

// Tiled sparse operand and the product that reads it. es = value bytes (1: int8/fp8, 2: bf16).
int64_t tiled_vals_bytes(int64_t rows, int64_t Kc, int es);
int64_t tiled_meta_bytes(int64_t rows, int64_t Kc, int es);
hipError_t launch_pack_tiled(int es, const uint8_t* vals, int64_t ldv_bytes, const uint8_t* meta, int64_t ldm,
                             int64_t rows, int64_t Kc, uint8_t* tv, uint8_t* tm, hipStream_t st);
// ab: 0 = int8, 1 = fp8, 2 = bf16; yt: 0 = bf16, 1 = f32, 2 = i32
// ws: workspace of spgemm_tiled_workspace_bytes bytes, or NULL (no split-K path)
hipError_t launch_spgemm_tiled(bool side_x, int ab, int yt, int64_t R, int64_t C, int64_t Kc, const uint8_t* tv,
                               const uint8_t* tm, const void* bd, int64_t ldb_bytes, const float* sx, const float* sw,
                               void* Y, int64_t ldy, void* ws, hipStream_t st);
int64_t spgemm_tiled_workspace_bytes(bool side_x, int ab, int64_t R, int64_t C, int64_t Kc);
// The prefill kernel of k_spgemm_wide.hip with 256 x bn tiles (bn = 256: one workgroup per CU, weight-sparse
// side only, eight waves for reductions of at most 64 steps and four beyond; bn = 128: two workgroups of four
// waves); R = rows of the sparse operand, C = rows of the dense one, KS = steps of 64 value bytes, ldb in
// bytes; launch_spgemm_tiled routes the larger prefill problems to it.
hipError_t launch_spgemm_wide(int bn, bool side_x, int ab, int yt, int R, int C, int KS, const uint8_t* tv,
                              const uint8_t* tm, const uint8_t* bd, int ldb, const float* sx, const float* sw, void* Y,
                              int ldy, hipStream_t st);

// A batch of same-shaped tiled products (one launch; blockIdx.y = problem); strides in bytes for the tiled
// operand and the dense operand, in elements for the scales and Y.
hipError_t launch_spgemm_tiled_batched(bool side_x, int ab, int yt, int64_t batch, int64_t R, int64_t C, int64_t Kc,
                                       const uint8_t* tv, int64_t s_tv, const uint8_t* tm, int64_t s_tm, const void* bd,
                                       int64_t ldb_bytes, int64_t s_bd, const float* sx, int64_t s_sx, const float* sw,
                                       int64_t s_sw, void* Y, int64_t ldy, int64_t s_y, hipStream_t st);

// Few-token quant+lift fused into the weight-sparse row-block product (ab: 0 = int8, 1 = fp8; yt as above).
bool quant_lift_spgemm_fits(bool x_bf16, int64_t M, int64_t K, int64_t Kc);
hipError_t launch_quant_lift_spgemm(bool x_bf16, int ab, int yt, const void* X, int64_t ldx, int64_t M, int64_t K, int n,
                                    int64_t N, int64_t Kc, const uint8_t* tv, const uint8_t* tm, const float* sw,
                                    void* Y, int64_t ldy, float* sx_out, hipStream_t st);

// Prefill with the per-token quantisation inside the product (2:4 weights, K % 128 == 0, bf16 X): absmax
// into sx, the product coding X into its LDS stages, then sx = a / Q. ab: 0 = int8, 1 = fp8; yt: 0 = bf16,
// 1 = f32.
hipError_t launch_quant_spgemm_prefill(int ab, int yt, const uint16_t* X, int64_t ldx, int64_t M, int64_t K,
                                       const uint8_t* tv, const uint8_t* tm, const float* sw, int64_t N, void* Y,
                                       int64_t ldy, float* sx, hipStream_t st);

// Block-scaled FP8 (128 x 128 weight blocks, per-token groups of 128; 2:4 weights, K' = K = Kc):
// weight prep into the tiled operand with scales [ceil(rows / 128)][Kc / 128], activation codes [M][Kc] with
// scales [M][Kc / 128], and the weight-sparse product (yt: 0 = bf16, 1 = f32).
hipError_t launch_prune24_block(bool in_bf16, const void* W, int64_t ldw, int64_t rows, int64_t K, int64_t Kc,
                                void* tv, uint8_t* tm, float* sw, hipStream_t st);
hipError_t launch_quant_group(bool x_bf16, const void* X, int64_t ldx, int64_t M, int64_t K, void* Xq, int64_t ldq,
                              int64_t Kc, float* sx, hipStream_t st);
hipError_t launch_spgemm_tiled_block(int yt, int64_t R, int64_t C, int64_t Kc, const uint8_t* tv, const uint8_t* tm,
                                     const void* bd, int64_t ldb_bytes, const float* sx, const float* sw, void* Y,
                                     int64_t ldy, hipStream_t st);

}  // namespace ss
