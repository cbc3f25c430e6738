// C ABI of the library: host-side argument validation, then one kernel launch
// per call on the caller's stream. Nothing is enqueued when validation fails.
#include <hip/hip_runtime.h>
#include <stdarg.h>

#include <atomic>
#include <stdio.h>
#include <string.h>

#include "ss.h"
#include "ss_kernels.h"

namespace {

thread_local char g_err[512] = "";

ss_status fail(ss_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

ss_status ok() {
  g_err[0] = 0;
  return SS_OK;
}

ss_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int esize(ss_dtype t) {
  switch (t) {
    case SS_F32: case SS_I32: return 4;
    case SS_BF16: return 2;
    case SS_I8: case SS_FP8E4M3: return 1;
  }
  return 0;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Row starts of a [rows x cols] matrix with leading dimension ld (elements).
ss_status check_mat(const char* name, const void* p, int64_t rows, int64_t cols, int64_t ld, int es) {
  if (!p) return fail(SS_ERR_NULL, "%s is NULL", name);
  if (ld < cols) return fail(SS_ERR_SHAPE, "%s: leading dimension %lld < %lld columns", name, (long long)ld, (long long)cols);
  if (!aligned16(p)) return fail(SS_ERR_ALIGN, "%s is not 16-byte aligned", name);
  if (rows > 1 && (ld * es) % 16 != 0)
    return fail(SS_ERR_ALIGN, "%s: row stride of %lld bytes is not a multiple of 16", name, (long long)(ld * es));
  return SS_OK;
}

int out_code(ss_dtype t) { return t == SS_I8 ? 0 : t == SS_FP8E4M3 ? 1 : 2; }

}  // namespace

extern "C" {

int64_t ss_lifted_k_logical(int64_t K, int n) {
  if (K < 0 || n < 2 || n > 8) return -1;
  return (K + 2 * n - 1) / (2 * n) * 4 * (n - 1);
}

int64_t ss_lifted_k(int64_t K, int n) {
  const int64_t k = ss_lifted_k_logical(K, n);
  if (k < 0) return -1;
  return (k + SS_KALIGN - 1) / SS_KALIGN * SS_KALIGN;
}

const char* ss_status_string(int s) {
  switch (s) {
    case SS_OK: return "SS_OK";
    case SS_ERR_NULL: return "SS_ERR_NULL";
    case SS_ERR_SHAPE: return "SS_ERR_SHAPE";
    case SS_ERR_ALIGN: return "SS_ERR_ALIGN";
    case SS_ERR_DTYPE: return "SS_ERR_DTYPE";
    case SS_ERR_PATTERN: return "SS_ERR_PATTERN";
    case SS_ERR_UNSUPPORTED: return "SS_ERR_UNSUPPORTED";
    case SS_ERR_HIP: return "SS_ERR_HIP";
  }
  return "unknown status";
}

const char* ss_last_error(void) { return g_err; }
int ss_version(void) { return SS_VERSION; }

static ss_status check_weight_prep(const void* W, ss_dtype w_dt, int64_t rows, int64_t K, int64_t ldw,
                                   ss_dtype out_dt, void* vals, int64_t ldv, uint8_t* meta, int64_t ldm,
                                   float* scale, int64_t Kc) {
  if (w_dt != SS_F32 && w_dt != SS_BF16) return fail(SS_ERR_DTYPE, "input must be F32 or BF16");
  if (out_dt != SS_I8 && out_dt != SS_FP8E4M3 && out_dt != SS_BF16)
    return fail(SS_ERR_DTYPE, "output must be I8, FP8E4M3 or BF16");
  if (rows < 0 || K < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (rows > 0x7FFFFFFF) return fail(SS_ERR_SHAPE, "too many rows");
  if (rows == 0 || K == 0) return SS_OK;
  ss_status s;
  if ((s = check_mat("input", W, rows, K, ldw, esize(w_dt))) != SS_OK) return s;
  if ((s = check_mat("vals", vals, rows, Kc / 2, ldv, esize(out_dt))) != SS_OK) return s;
  if ((s = check_mat("meta", meta, rows, Kc / 8, ldm, 1)) != SS_OK) return s;
  if (out_dt == SS_BF16) {
    if (scale) return fail(SS_ERR_DTYPE, "BF16 output takes no scale (pass NULL)");
  } else if (!scale) {
    return fail(SS_ERR_NULL, "scale is NULL");
  }
  return SS_OK;
}

ss_status ss_prune24(const void* W, ss_dtype w_dt, int64_t rows, int64_t K, int64_t ldw, ss_dtype out_dt,
                     void* vals, int64_t ldv, uint8_t* meta, int64_t ldm, float* scale, void* stream) {
  if (K % 4 != 0) return fail(SS_ERR_SHAPE, "K=%lld is not a multiple of 4", (long long)K);
  const int64_t Kc = ss_lifted_k(K, 2);
  ss_status s = check_weight_prep(W, w_dt, rows, K, ldw, out_dt, vals, ldv, meta, ldm, scale, Kc);
  if (s != SS_OK) return s;
  if (rows == 0 || K == 0) return ok();
  return hip_status(ss::launch_prune24(w_dt == SS_BF16, out_code(out_dt), W, ldw, rows, K, vals, ldv * esize(out_dt),
                                       meta, ldm, Kc, scale, (hipStream_t)stream),
                    "ss_prune24 launch");
}

ss_status ss_slide_decompose(const void* W, ss_dtype w_dt, int64_t rows, int64_t K, int64_t ldw, int n,
                             ss_dtype out_dt, void* vals, int64_t ldv, uint8_t* meta, int64_t ldm, float* scale,
                             void* stream) {
  if (n < 2 || n > 8) return fail(SS_ERR_PATTERN, "n=%d outside 2..8", n);
  const int64_t Kc = ss_lifted_k(K, n);
  ss_status s = check_weight_prep(W, w_dt, rows, K, ldw, out_dt, vals, ldv, meta, ldm, scale, Kc);
  if (s != SS_OK) return s;
  if (rows == 0 || K == 0) return ok();
  return hip_status(ss::launch_slide(w_dt == SS_BF16, out_code(out_dt), W, ldw, rows, K, n, vals, ldv * esize(out_dt),
                                     meta, ldm, Kc, scale, (hipStream_t)stream),
                    "ss_slide_decompose launch");
}

ss_status ss_quant_lift_act(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx, int n, ss_dtype q_dt,
                            void* Xq, int64_t ldq, float* sx, void* stream) {
  if (n < 2 || n > 8) return fail(SS_ERR_PATTERN, "n=%d outside 2..8", n);
  if (x_dt != SS_F32 && x_dt != SS_BF16) return fail(SS_ERR_DTYPE, "input must be F32 or BF16");
  if (q_dt != SS_I8 && q_dt != SS_FP8E4M3) return fail(SS_ERR_DTYPE, "output must be I8 or FP8E4M3");
  if (M < 0 || K < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (M > 0x7FFFFFFF) return fail(SS_ERR_SHAPE, "too many rows");
  if (M == 0 || K == 0) return ok();
  const int64_t Kc = ss_lifted_k(K, n);
  ss_status s;
  if ((s = check_mat("X", X, M, K, ldx, esize(x_dt))) != SS_OK) return s;
  if ((s = check_mat("Xq", Xq, M, Kc, ldq, 1)) != SS_OK) return s;
  if (!sx) return fail(SS_ERR_NULL, "sx is NULL");
  return hip_status(ss::launch_quant_lift(x_dt == SS_BF16, q_dt == SS_FP8E4M3, X, ldx, M, K, n, Xq, ldq, Kc, sx,
                                          (hipStream_t)stream),
                    "ss_quant_lift_act launch");
}

ss_status ss_prune24_act(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx, ss_dtype out_dt, void* vals,
                         int64_t ldv, uint8_t* meta, int64_t ldm, float* sx, void* stream) {
  if (x_dt != SS_BF16) return fail(SS_ERR_DTYPE, "activations must be BF16");
  if (K % 4 != 0) return fail(SS_ERR_SHAPE, "K=%lld is not a multiple of 4", (long long)K);
  const int64_t Kc = ss_lifted_k(K, 2);
  ss_status s = check_weight_prep(X, x_dt, M, K, ldx, out_dt, vals, ldv, meta, ldm, sx, Kc);
  if (s != SS_OK) return s;
  if (M == 0 || K == 0) return ok();
  return hip_status(ss::launch_prune24(true, out_code(out_dt), X, ldx, M, K, vals, ldv * esize(out_dt), meta, ldm, Kc,
                                       sx, (hipStream_t)stream),
                    "ss_prune24_act launch");
}

ss_status ss_spgemm(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt, const void* sp_vals, int64_t ldsv,
                    const uint8_t* sp_meta, int64_t ldsm, const void* dense, int64_t ldd, const float* sx,
                    const float* sw, ss_dtype y_dt, void* Y, int64_t ldy, void* stream) {
  if (side != SS_SPARSE_W && side != SS_SPARSE_X) return fail(SS_ERR_SHAPE, "bad side");
  if (ab_dt != SS_I8 && ab_dt != SS_FP8E4M3 && ab_dt != SS_BF16)
    return fail(SS_ERR_DTYPE, "operands must be I8, FP8E4M3 or BF16");
  if (y_dt != SS_BF16 && y_dt != SS_F32 && y_dt != SS_I32) return fail(SS_ERR_DTYPE, "output must be BF16, F32 or I32");
  if (y_dt == SS_I32 && ab_dt != SS_I8) return fail(SS_ERR_DTYPE, "I32 output needs I8 operands");
  if (M < 0 || N < 0 || Kc < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (Kc % SS_KALIGN != 0) return fail(SS_ERR_SHAPE, "Kc=%lld is not a multiple of %d", (long long)Kc, SS_KALIGN);
  if (M > 0x7FFFFFFFLL * 128 || N > 0x7FFFFFFFLL * 128) return fail(SS_ERR_SHAPE, "too many rows");
  if (M == 0 || N == 0) return ok();
  const bool sx_side = (side == SS_SPARSE_X);
  const int64_t R = sx_side ? M : N, C = sx_side ? N : M;
  const int es = esize(ab_dt);
  ss_status s;
  if ((s = check_mat("sp_vals", sp_vals, R, Kc / 2, ldsv, es)) != SS_OK) return s;
  if ((s = check_mat("sp_meta", sp_meta, R, Kc / 8, ldsm, 1)) != SS_OK) return s;
  if ((s = check_mat("dense", dense, C, Kc, ldd, es)) != SS_OK) return s;
  // Y needs only an aligned base; rows are stored with vector writes when
  // ldy % 4 == 0 and element by element otherwise
  if ((s = check_mat("Y", Y, 1, N, ldy, esize(y_dt))) != SS_OK) return s;
  if (ab_dt != SS_BF16 && y_dt != SS_I32 && (!sx || !sw))
    return fail(SS_ERR_NULL, "INT8/FP8 products need both scales");
  const int ab = ab_dt == SS_I8 ? 0 : ab_dt == SS_FP8E4M3 ? 1 : 2;
  const int yt = y_dt == SS_BF16 ? 0 : y_dt == SS_F32 ? 1 : 2;
  return hip_status(ss::launch_spgemm(sx_side, ab, yt, R, C, Kc, sp_vals, ldsv * es, sp_meta, ldsm, dense, ldd * es,
                                      y_dt == SS_I32 ? nullptr : sx, y_dt == SS_I32 ? nullptr : sw, Y, ldy,
                                      (hipStream_t)stream),
                    "ss_spgemm launch");
}

int64_t ss_tiled_vals_bytes(int64_t rows, int64_t Kc, ss_dtype dt) {
  if (rows < 0 || Kc < 0 || Kc % SS_KALIGN != 0 || (dt != SS_I8 && dt != SS_FP8E4M3 && dt != SS_BF16)) return -1;
  return ss::tiled_vals_bytes(rows, Kc, esize(dt));
}

int64_t ss_tiled_meta_bytes(int64_t rows, int64_t Kc, ss_dtype dt) {
  if (rows < 0 || Kc < 0 || Kc % SS_KALIGN != 0 || (dt != SS_I8 && dt != SS_FP8E4M3 && dt != SS_BF16)) return -1;
  return ss::tiled_meta_bytes(rows, Kc, esize(dt));
}

ss_status ss_pack_sparse(int64_t rows, int64_t Kc, ss_dtype dt, const void* vals, int64_t ldv, const uint8_t* meta,
                         int64_t ldm, void* tvals, uint8_t* tmeta, void* stream) {
  if (dt != SS_I8 && dt != SS_FP8E4M3 && dt != SS_BF16) return fail(SS_ERR_DTYPE, "values must be I8, FP8E4M3 or BF16");
  if (rows < 0 || Kc < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (Kc % SS_KALIGN != 0) return fail(SS_ERR_SHAPE, "Kc=%lld is not a multiple of %d", (long long)Kc, SS_KALIGN);
  if (rows > 0x7FFFFFF0LL || Kc / 64 > 0x7FFFFFF0LL) return fail(SS_ERR_SHAPE, "too large");
  if (rows == 0 || Kc == 0) return ok();
  const int es = esize(dt);
  ss_status s;
  if ((s = check_mat("vals", vals, rows, Kc / 2, ldv, es)) != SS_OK) return s;
  if ((s = check_mat("meta", meta, rows, Kc / 8, ldm, 1)) != SS_OK) return s;
  if (!tvals || !tmeta) return fail(SS_ERR_NULL, "tiled outputs are NULL");
  if (!aligned16(tvals) || !aligned16(tmeta)) return fail(SS_ERR_ALIGN, "tiled outputs are not 16-byte aligned");
  return hip_status(ss::launch_pack_tiled(es, static_cast<const uint8_t*>(vals), ldv * es, meta, ldm, rows, Kc,
                                          static_cast<uint8_t*>(tvals), tmeta, (hipStream_t)stream),
                    "ss_pack_sparse launch");
}

ss_status ss_prune24_act_tiled(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx, ss_dtype out_dt,
                               void* tvals, uint8_t* tmeta, float* sx, void* stream) {
  if (x_dt != SS_BF16) return fail(SS_ERR_DTYPE, "activations must be BF16");
  if (out_dt != SS_I8 && out_dt != SS_FP8E4M3 && out_dt != SS_BF16) return fail(SS_ERR_DTYPE, "bad output type");
  if (M < 0 || K < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (K % 4 != 0) return fail(SS_ERR_SHAPE, "K=%lld is not a multiple of 4", (long long)K);
  if (M > 0x7FFFFFF0LL || K > 0x3FFFFFF0LL) return fail(SS_ERR_SHAPE, "too large");
  if (M == 0 || K == 0) return ok();
  ss_status s;
  if ((s = check_mat("X", X, M, K, ldx, 2)) != SS_OK) return s;
  if (!tvals || !tmeta) return fail(SS_ERR_NULL, "tiled outputs are NULL");
  if (!aligned16(tvals) || !aligned16(tmeta)) return fail(SS_ERR_ALIGN, "tiled outputs are not 16-byte aligned");
  if (out_dt == SS_BF16 && sx) return fail(SS_ERR_DTYPE, "BF16 output takes no scale");
  if (out_dt != SS_BF16 && !sx) return fail(SS_ERR_NULL, "quantised output needs sx");
  const int64_t Kc = ss_lifted_k(K, 2);
  return hip_status(ss::launch_prune24_act_tiled(out_code(out_dt), X, ldx, M, K, Kc, tvals, tmeta, sx,
                                                 (hipStream_t)stream),
                    "ss_prune24_act_tiled launch");
}

ss_status ss_slide_decompose_tiled(const void* W, ss_dtype w_dt, int64_t rows, int64_t K, int64_t ldw, int n,
                                   ss_dtype out_dt, void* tvals, uint8_t* tmeta, float* scale, void* stream) {
  if (n < 2 || n > 8) return fail(SS_ERR_PATTERN, "n=%d outside 2..8", n);
  if (w_dt != SS_F32 && w_dt != SS_BF16) return fail(SS_ERR_DTYPE, "input must be F32 or BF16");
  if (out_dt != SS_I8 && out_dt != SS_FP8E4M3 && out_dt != SS_BF16)
    return fail(SS_ERR_DTYPE, "output must be I8, FP8E4M3 or BF16");
  if (rows < 0 || K < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (rows > 0x7FFFFFF0LL || K > 0x3FFFFFF0LL) return fail(SS_ERR_SHAPE, "too large");
  if (rows == 0 || K == 0) return ok();
  ss_status s;
  if ((s = check_mat("input", W, rows, K, ldw, esize(w_dt))) != SS_OK) return s;
  if (!tvals || !tmeta) return fail(SS_ERR_NULL, "tiled outputs are NULL");
  if (!aligned16(tvals) || !aligned16(tmeta)) return fail(SS_ERR_ALIGN, "tiled outputs are not 16-byte aligned");
  if (out_dt == SS_BF16 && scale) return fail(SS_ERR_DTYPE, "BF16 output takes no scale (pass NULL)");
  if (out_dt != SS_BF16 && !scale) return fail(SS_ERR_NULL, "scale is NULL");
  const int64_t Kc = ss_lifted_k(K, n);
  return hip_status(ss::launch_slide_tiled(w_dt == SS_BF16, out_code(out_dt), W, ldw, rows, K, n, Kc, tvals, tmeta,
                                           scale, (hipStream_t)stream),
                    "ss_slide_decompose_tiled launch");
}

// Checks shared by ss_spgemm_tiled and ss_spgemm_tiled_ws; sets *run = false for an empty problem.
static ss_status check_spgemm_tiled(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt, const void* tvals,
                                    const uint8_t* tmeta, const void* dense, int64_t ldd, const float* sx,
                                    const float* sw, ss_dtype y_dt, void* Y, int64_t ldy, bool* run) {
  *run = false;
  if (side != SS_SPARSE_W && side != SS_SPARSE_X) return fail(SS_ERR_SHAPE, "bad side");
  if (ab_dt != SS_I8 && ab_dt != SS_FP8E4M3 && ab_dt != SS_BF16)
    return fail(SS_ERR_DTYPE, "operands must be I8, FP8E4M3 or BF16");
  if (y_dt != SS_BF16 && y_dt != SS_F32 && y_dt != SS_I32) return fail(SS_ERR_DTYPE, "output must be BF16, F32 or I32");
  if (y_dt == SS_I32 && ab_dt != SS_I8) return fail(SS_ERR_DTYPE, "I32 output needs I8 operands");
  if (M < 0 || N < 0 || Kc < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (Kc % SS_KALIGN != 0) return fail(SS_ERR_SHAPE, "Kc=%lld is not a multiple of %d", (long long)Kc, SS_KALIGN);
  if (M == 0 || N == 0) return SS_OK;
  if (Kc == 0) return fail(SS_ERR_SHAPE, "Kc must be positive");
  const bool sx_side = (side == SS_SPARSE_X);
  const int64_t R = sx_side ? M : N, C = sx_side ? N : M;
  if (R > 0x7FFFFFF0LL || C > 0x7FFFFFF0LL || ldy > 0x7FFFFFFFLL || Kc / 64 > 0x7FFFFFF0LL)
    return fail(SS_ERR_SHAPE, "too large");
  const int es = esize(ab_dt);
  ss_status s;
  if ((s = check_mat("dense", dense, C, Kc, ldd, es)) != SS_OK) return s;
  // the kernel addresses the dense operand with 32-bit byte offsets
  if ((uint64_t)(C - 1) * (uint64_t)ldd * es + (uint64_t)Kc * es > 0xFFFFFFFFull)
    return fail(SS_ERR_UNSUPPORTED, "dense operand spans more than 4 GiB");
  if ((s = check_mat("Y", Y, 1, N, ldy, esize(y_dt))) != SS_OK) return s;
  if (!tvals || !tmeta) return fail(SS_ERR_NULL, "tiled operand is NULL");
  if (!aligned16(tvals) || !aligned16(tmeta)) return fail(SS_ERR_ALIGN, "tiled operand is not 16-byte aligned");
  if (ab_dt != SS_BF16 && y_dt != SS_I32 && (!sx || !sw)) return fail(SS_ERR_NULL, "INT8/FP8 products need both scales");
  *run = true;
  return SS_OK;
}

static ss_status run_spgemm_tiled(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt, const void* tvals,
                                  const uint8_t* tmeta, const void* dense, int64_t ldd, const float* sx,
                                  const float* sw, ss_dtype y_dt, void* Y, int64_t ldy, void* ws, void* stream) {
  const bool sx_side = (side == SS_SPARSE_X);
  const int64_t R = sx_side ? M : N, C = sx_side ? N : M;
  const int ab = ab_dt == SS_I8 ? 0 : ab_dt == SS_FP8E4M3 ? 1 : 2;
  const int yt = y_dt == SS_BF16 ? 0 : y_dt == SS_F32 ? 1 : 2;
  return hip_status(ss::launch_spgemm_tiled(sx_side, ab, yt, R, C, Kc, static_cast<const uint8_t*>(tvals), tmeta, dense,
                                            ldd * esize(ab_dt), y_dt == SS_I32 ? nullptr : sx,
                                            y_dt == SS_I32 ? nullptr : sw, Y, ldy, ws, (hipStream_t)stream),
                    "ss_spgemm_tiled launch");
}

ss_status ss_spgemm_tiled(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt, const void* tvals,
                          const uint8_t* tmeta, const void* dense, int64_t ldd, const float* sx, const float* sw,
                          ss_dtype y_dt, void* Y, int64_t ldy, void* stream) {
  bool run = false;
  const ss_status s = check_spgemm_tiled(side, M, N, Kc, ab_dt, tvals, tmeta, dense, ldd, sx, sw, y_dt, Y, ldy, &run);
  if (s != SS_OK) return s;
  if (!run) return ok();
  return run_spgemm_tiled(side, M, N, Kc, ab_dt, tvals, tmeta, dense, ldd, sx, sw, y_dt, Y, ldy, nullptr, stream);
}

int64_t ss_spgemm_tiled_workspace_bytes(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt) {
  if (side != SS_SPARSE_W && side != SS_SPARSE_X) return -1;
  if (ab_dt != SS_I8 && ab_dt != SS_FP8E4M3 && ab_dt != SS_BF16) return -1;
  if (M < 0 || N < 0 || Kc < 0 || Kc % SS_KALIGN != 0) return -1;
  if (M == 0 || N == 0 || Kc == 0 || M > 0x7FFFFFF0LL || N > 0x7FFFFFF0LL) return 0;
  const bool sx_side = (side == SS_SPARSE_X);
  const int ab = ab_dt == SS_I8 ? 0 : ab_dt == SS_FP8E4M3 ? 1 : 2;
  return ss::spgemm_tiled_workspace_bytes(sx_side, ab, sx_side ? M : N, sx_side ? N : M, Kc);
}

// The allocation-free variant's split-K workspace: a static array in the code object (one copy per GPU), and
// its device address per GPU, looked up once with that GPU current. Host code must use the looked-up
// address: the array's name on the host is only a stand-in for the symbol.
static __device__ __align__(256) uint8_t scratch[SS_NOALLOC_SCRATCH_BYTES];
namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

ss_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SS_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                                                 kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(SS_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SS_OK;
}
}  // namespace

ss_status ss_spgemm_tiled_noalloc(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt, const void* tvals,
                                  const uint8_t* tmeta, const void* dense, int64_t ldd, const float* sx,
                                  const float* sw, ss_dtype y_dt, void* Y, int64_t ldy, void* stream) {
  bool run = false;
  ss_status s = check_spgemm_tiled(side, M, N, Kc, ab_dt, tvals, tmeta, dense, ldd, sx, sw, y_dt, Y, ldy, &run);
  if (s != SS_OK) return s;
  if (!run) return ok();
  const int64_t need = ss_spgemm_tiled_workspace_bytes(side, M, N, Kc, ab_dt);
  if (need > SS_NOALLOC_SCRATCH_BYTES)
    return fail(SS_ERR_UNSUPPORTED, "workspace of %lld bytes exceeds the %d-byte static scratch", (long long)need,
                SS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0 && (s = scratch_ptr(&ws)) != SS_OK) return s;
  return run_spgemm_tiled(side, M, N, Kc, ab_dt, tvals, tmeta, dense, ldd, sx, sw, y_dt, Y, ldy, ws, stream);
}

ss_status ss_quant_spgemm_prefill(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx, ss_dtype q_dt,
                                  const void* tvals, const uint8_t* tmeta, const float* sw, int64_t N, ss_dtype y_dt,
                                  void* Y, int64_t ldy, float* sx, void* stream) {
  if (x_dt != SS_BF16) return fail(SS_ERR_DTYPE, "X must be BF16");
  if (q_dt != SS_I8 && q_dt != SS_FP8E4M3) return fail(SS_ERR_DTYPE, "codes must be I8 or FP8E4M3");
  if (y_dt != SS_BF16 && y_dt != SS_F32) return fail(SS_ERR_DTYPE, "output must be BF16 or F32");
  if (M < 0 || N < 0 || K < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (K % 128 != 0) return fail(SS_ERR_SHAPE, "K=%lld is not a multiple of 128", (long long)K);
  if (M == 0 || N == 0) return ok();
  if (K == 0) return fail(SS_ERR_SHAPE, "K must be positive");
  if (M > 0x7FFFFFF0LL || N > 0x7FFFFFF0LL || K > 0x7FFFFF00LL || ldy > 0x7FFFFFFFLL || ldx > 0x7FFFFFFFLL)
    return fail(SS_ERR_SHAPE, "too large");
  ss_status s;
  if ((s = check_mat("X", X, M, K, ldx, 2)) != SS_OK) return s;
  // (output rows need no 16-byte alignment: the stores fall back to single elements)
  if ((s = check_mat("Y", Y, 1, N, ldy, esize(y_dt))) != SS_OK) return s;
  if (!tvals || !tmeta || !sw || !sx) return fail(SS_ERR_NULL, "tvals, tmeta, sw and sx are required");
  if (!aligned16(tvals) || !aligned16(tmeta)) return fail(SS_ERR_ALIGN, "tiled operand is not 16-byte aligned");
  return hip_status(ss::launch_quant_spgemm_prefill(q_dt == SS_I8 ? 0 : 1, y_dt == SS_BF16 ? 0 : 1,
                                                    static_cast<const uint16_t*>(X), ldx, M, K,
                                                    static_cast<const uint8_t*>(tvals), tmeta, sw, N, Y, ldy, sx,
                                                    (hipStream_t)stream),
                    "ss_quant_spgemm_prefill launch");
}

ss_status ss_spgemm_tiled_ws(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt, const void* tvals,
                             const uint8_t* tmeta, const void* dense, int64_t ldd, const float* sx, const float* sw,
                             ss_dtype y_dt, void* Y, int64_t ldy, void* workspace, int64_t ws_bytes, void* stream) {
  bool run = false;
  const ss_status s = check_spgemm_tiled(side, M, N, Kc, ab_dt, tvals, tmeta, dense, ldd, sx, sw, y_dt, Y, ldy, &run);
  if (s != SS_OK) return s;
  if (ws_bytes < 0) return fail(SS_ERR_SHAPE, "negative workspace size");
  if (!run) return ok();
  const int64_t need = ss_spgemm_tiled_workspace_bytes(side, M, N, Kc, ab_dt);
  if (need > 0) {
    if (!workspace) return fail(SS_ERR_NULL, "workspace is NULL (%lld bytes needed)", (long long)need);
    if (!aligned16(workspace)) return fail(SS_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (ws_bytes < need) return fail(SS_ERR_SHAPE, "workspace of %lld bytes, %lld needed", (long long)ws_bytes,
                                     (long long)need);
  }
  return run_spgemm_tiled(side, M, N, Kc, ab_dt, tvals, tmeta, dense, ldd, sx, sw, y_dt, Y, ldy,
                          need > 0 ? workspace : nullptr, stream);
}

ss_status ss_prune24_block(const void* W, ss_dtype w_dt, int64_t rows, int64_t K, int64_t ldw, void* tvals,
                           uint8_t* tmeta, float* sw, void* stream) {
  if (w_dt != SS_F32 && w_dt != SS_BF16) return fail(SS_ERR_DTYPE, "input must be F32 or BF16");
  if (rows < 0 || K < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (K % 4 != 0) return fail(SS_ERR_SHAPE, "K=%lld is not a multiple of 4", (long long)K);
  if (rows > 0x7FFFFFF0LL || K > 0x3FFFFFF0LL) return fail(SS_ERR_SHAPE, "too large");
  if (rows == 0 || K == 0) return ok();
  ss_status s;
  if ((s = check_mat("input", W, rows, K, ldw, esize(w_dt))) != SS_OK) return s;
  if (!tvals || !tmeta) return fail(SS_ERR_NULL, "tiled outputs are NULL");
  if (!aligned16(tvals) || !aligned16(tmeta)) return fail(SS_ERR_ALIGN, "tiled outputs are not 16-byte aligned");
  if (!sw) return fail(SS_ERR_NULL, "sw is NULL");
  const int64_t Kc = ss_lifted_k(K, 2);
  return hip_status(ss::launch_prune24_block(w_dt == SS_BF16, W, ldw, rows, K, Kc, tvals, tmeta, sw,
                                             (hipStream_t)stream),
                    "ss_prune24_block launch");
}

ss_status ss_quant_group_act(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx, void* Xq, int64_t ldq,
                             float* sx, void* stream) {
  if (x_dt != SS_F32 && x_dt != SS_BF16) return fail(SS_ERR_DTYPE, "input must be F32 or BF16");
  if (M < 0 || K < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (M > 0x7FFFFFF0LL || K > 0x3FFFFFF0LL) return fail(SS_ERR_SHAPE, "too large");
  if (M == 0 || K == 0) return ok();
  const int64_t Kc = ss_lifted_k(K, 2);
  if (M * ((Kc / 128 + 15) / 16) > 0x7FFFFFFFLL) return fail(SS_ERR_SHAPE, "too large");
  ss_status s;
  if ((s = check_mat("X", X, M, K, ldx, esize(x_dt))) != SS_OK) return s;
  if ((s = check_mat("Xq", Xq, M, Kc, ldq, 1)) != SS_OK) return s;
  if (!sx) return fail(SS_ERR_NULL, "sx is NULL");
  return hip_status(ss::launch_quant_group(x_dt == SS_BF16, X, ldx, M, K, Xq, ldq, Kc, sx, (hipStream_t)stream),
                    "ss_quant_group_act launch");
}

ss_status ss_spgemm_tiled_block(int64_t M, int64_t N, int64_t Kc, const void* tvals, const uint8_t* tmeta,
                                const void* dense, int64_t ldd, const float* sx, const float* sw, ss_dtype y_dt,
                                void* Y, int64_t ldy, void* stream) {
  if (y_dt != SS_BF16 && y_dt != SS_F32) return fail(SS_ERR_DTYPE, "output must be BF16 or F32");
  if (M < 0 || N < 0 || Kc < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (Kc % SS_KALIGN != 0) return fail(SS_ERR_SHAPE, "Kc=%lld is not a multiple of %d", (long long)Kc, SS_KALIGN);
  if (M == 0 || N == 0) return ok();
  if (Kc == 0) return fail(SS_ERR_SHAPE, "Kc must be positive");
  if (M > 0x7FFFFFF0LL || N > 0x7FFFFFF0LL || ldy > 0x7FFFFFFFLL || Kc / 64 > 0x7FFFFFF0LL)
    return fail(SS_ERR_SHAPE, "too large");
  ss_status s;
  if ((s = check_mat("dense", dense, M, Kc, ldd, 1)) != SS_OK) return s;
  if ((uint64_t)(M - 1) * (uint64_t)ldd + (uint64_t)Kc > 0xFFFFFFFFull)
    return fail(SS_ERR_UNSUPPORTED, "dense operand spans more than 4 GiB");
  if ((s = check_mat("Y", Y, 1, N, ldy, esize(y_dt))) != SS_OK) return s;
  if (!tvals || !tmeta) return fail(SS_ERR_NULL, "tiled operand is NULL");
  if (!aligned16(tvals) || !aligned16(tmeta)) return fail(SS_ERR_ALIGN, "tiled operand is not 16-byte aligned");
  if (!sx || !sw) return fail(SS_ERR_NULL, "block-scaled products need both scale arrays");
  return hip_status(ss::launch_spgemm_tiled_block(y_dt == SS_BF16 ? 0 : 1, N, M, Kc, static_cast<const uint8_t*>(tvals),
                                                  tmeta, dense, ldd, sx, sw, Y, ldy, (hipStream_t)stream),
                    "ss_spgemm_tiled_block launch");
}

ss_status ss_spgemm_tiled_batched(ss_side side, int64_t batch, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt,
                                  const void* tvals, int64_t tvals_stride, const uint8_t* tmeta, int64_t tmeta_stride,
                                  const void* dense, int64_t ldd, int64_t dense_stride, const float* sx,
                                  int64_t sx_stride, const float* sw, int64_t sw_stride, ss_dtype y_dt, void* Y,
                                  int64_t ldy, int64_t y_stride, void* stream) {
  if (batch < 0) return fail(SS_ERR_SHAPE, "negative batch");
  bool run = false;
  const ss_status s = check_spgemm_tiled(side, M, N, Kc, ab_dt, tvals, tmeta, dense, ldd, sx, sw, y_dt, Y, ldy, &run);
  if (s != SS_OK) return s;
  if (!run || batch == 0) return ok();
  if (batch > 65535) return fail(SS_ERR_SHAPE, "batch=%lld exceeds 65535", (long long)batch);
  if (tvals_stride < 0 || tmeta_stride < 0 || dense_stride < 0 || sx_stride < 0 || sw_stride < 0 || y_stride < 0)
    return fail(SS_ERR_SHAPE, "negative stride");
  const int es = esize(ab_dt);
  if (tvals_stride % 16 || tmeta_stride % 16 || (dense_stride * es) % 16 || (y_stride * esize(y_dt)) % 16)
    return fail(SS_ERR_ALIGN, "operand strides must keep every problem 16-byte aligned");
  const bool sx_side = (side == SS_SPARSE_X);
  const int64_t R = sx_side ? M : N, C = sx_side ? N : M;
  const int ab = ab_dt == SS_I8 ? 0 : ab_dt == SS_FP8E4M3 ? 1 : 2;
  const int yt = y_dt == SS_BF16 ? 0 : y_dt == SS_F32 ? 1 : 2;
  return hip_status(ss::launch_spgemm_tiled_batched(sx_side, ab, yt, batch, R, C, Kc, static_cast<const uint8_t*>(tvals),
                                                    tvals_stride, tmeta, tmeta_stride, dense, ldd * es, dense_stride * es,
                                                    y_dt == SS_I32 ? nullptr : sx, sx_stride,
                                                    y_dt == SS_I32 ? nullptr : sw, sw_stride, Y, ldy, y_stride,
                                                    (hipStream_t)stream),
                    "ss_spgemm_tiled_batched launch");
}

ss_status ss_quant_lift_spgemm_decode(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx, int n,
                                      ss_dtype q_dt, const void* tvals, const uint8_t* tmeta, const float* sw, int64_t N,
                                      ss_dtype y_dt, void* Y, int64_t ldy, float* sx_out, void* stream) {
  if (n < 2 || n > 8) return fail(SS_ERR_PATTERN, "n=%d outside 2..8", n);
  if (x_dt != SS_F32 && x_dt != SS_BF16) return fail(SS_ERR_DTYPE, "input must be F32 or BF16");
  if (q_dt != SS_I8 && q_dt != SS_FP8E4M3) return fail(SS_ERR_DTYPE, "codes must be I8 or FP8E4M3");
  if (y_dt != SS_BF16 && y_dt != SS_F32 && y_dt != SS_I32) return fail(SS_ERR_DTYPE, "output must be BF16, F32 or I32");
  if (y_dt == SS_I32 && q_dt != SS_I8) return fail(SS_ERR_DTYPE, "I32 output needs I8 codes");
  if (M < 0 || K < 0 || N < 0) return fail(SS_ERR_SHAPE, "negative size");
  if (M == 0 || N == 0) return ok();
  if (K == 0) return fail(SS_ERR_SHAPE, "K must be positive");
  if (N > 0x7FFFFFF0LL || K > 0x3FFFFFF0LL || ldy > 0x7FFFFFFFLL) return fail(SS_ERR_SHAPE, "too large");
  const int64_t Kc = ss_lifted_k(K, n);
  if (!ss::quant_lift_spgemm_fits(x_dt == SS_BF16, M, K, Kc))
    return fail(SS_ERR_UNSUPPORTED, "M=%lld, K=%lld: the fused path takes 1..4 tokens with M*K' <= 131072 and K <= %d",
                (long long)M, (long long)K, x_dt == SS_BF16 ? 20480 : 16384);
  ss_status s;
  if ((s = check_mat("X", X, M, K, ldx, esize(x_dt))) != SS_OK) return s;
  if ((s = check_mat("Y", Y, 1, N, ldy, esize(y_dt))) != SS_OK) return s;
  if (!tvals || !tmeta) return fail(SS_ERR_NULL, "tiled operand is NULL");
  if (!aligned16(tvals) || !aligned16(tmeta)) return fail(SS_ERR_ALIGN, "tiled operand is not 16-byte aligned");
  if (!sw) return fail(SS_ERR_NULL, "sw is NULL");
  return hip_status(ss::launch_quant_lift_spgemm(x_dt == SS_BF16, q_dt == SS_I8 ? 0 : 1,
                                                 y_dt == SS_BF16 ? 0 : y_dt == SS_F32 ? 1 : 2, X, ldx, M, K, n, N, Kc,
                                                 static_cast<const uint8_t*>(tvals), tmeta, sw, Y, ldy, sx_out,
                                                 (hipStream_t)stream),
                    "ss_quant_lift_spgemm_decode launch");
}

}  // extern "C"
