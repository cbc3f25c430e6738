/* ss.h -- C ABI of the structured-sparse quantised linear-layer library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes the N:M structured-sparse, quantised matrix product of
 * an LLM linear layer, Y = X W^T, with one operand in 2:4 form:
 *   - weights: 2:4 magnitude prune along K into values plus 2-bit positions,
 *     or a (2n-2):2n magnitude prune followed by the SlideSparse sliding-window
 *     decomposition into n-1 overlapping stride-2 width-4 windows that each
 *     satisfy 2:4, over an expanded K';
 *   - activations: per-token dynamic INT8/FP8 quantisation fused with the
 *     lift to K', or an online 2:4 prune and compress;
 *   - the 2:4 product on the gfx950 structured-sparse matrix cores with a
 *     per-token x per-channel rescale epilogue.
 *
 * Sources (page title, then section): "Deep reading of arXiv 2610.28947"
 * (paper-daily.com) for 2:4 along the accumulate axis, the online pruning of
 * activations and the bits accounting; "SlideSparse: layout sparse boundary"
 * (MSRA article, 66bd.net) for the (2n-2):2n patterns, the window
 * decomposition and activation lifting; the SlideSparse blog (omica.com.cn),
 * sections 2.1-3.2, for the pattern table and the fused quantise-and-slide
 * kernel; the LLM Compressor "compression schemes" guide for per-channel
 * weight and dynamic per-token activation scales.
 *
 * Conventions shared by every call
 *   Pointers: device pointers unless stated; 16-byte aligned. Matrices are
 *   row-major with a leading dimension in ELEMENTS (metadata: in bytes); every
 *   row start must be 16-byte aligned (ld * element size % 16 == 0).
 *   Ownership: the caller allocates and owns every buffer; the library keeps no
 *   device memory and no state between calls. Calls are re-entrant.
 *   Streams: `stream` is a hipStream_t (NULL = the default stream). Work is
 *   enqueued on it; no call synchronises.
 *   Errors: arguments are checked on the host before anything is enqueued; on
 *   failure nothing is launched, the status is returned and ss_last_error()
 *   (per thread) describes it. SS_ERR_HIP reports a failed launch. Faults
 *   inside a kernel surface at the caller's next synchronisation.
 *   Empty problems (a zero row or column count) return SS_OK and launch
 *   nothing.
 *   Inputs must be finite (not checked).
 *
 * Pattern parameter n: (2n-2):2n, so n=2 is 2:4, n=3 is 4:6, n=4 is 6:8,
 * n=5 is 8:10; 2 <= n <= 8.
 *
 * Compressed 2:4 layout (every sparse operand):
 *   vals [rows][Kc/2] in the storage type: each 4-group of K keeps two slots,
 *     stored in ascending position order; slots holding a zero store +0;
 *   meta [rows][Kc/8] bytes: a group's nibble is idx0 | idx1 << 2 (idx0 <
 *     idx1, positions 0..3 within the group); byte j holds group 2j in bits
 *     0-3 and group 2j+1 in bits 4-7. Groups with fewer than two nonzeros fill
 *     the second slot with the lowest free position; all-zero groups use
 *     positions (0, 1). This is exactly the index operand of the gfx950
 *     v_smfmac instructions, so the product reads it unchanged.
 *   Kc = ss_lifted_k(K, n): K' rounded up to SS_KALIGN; the padding is
 *     zero groups.
 *
 * Per-row symmetric quantisation (weights per output channel, activations per
 * token), all in float32 with one rounding per step:
 *   a = max|v| of the row; inv = Q / a (correctly rounded); t = v * inv; INT8 q = clamp(rint(t), -127, 127) (ties to even),
 *   FP8 q = E4M3FN(clamp(t, -448, 448)) (OCP E4M3FN, nearest-even);
 *   scale = a / Q; Q = 127 (INT8) or 448 (FP8). A zero row gives scale 0 and
 *   zero codes.
 */
#ifndef SS_H
#define SS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SS_VERSION 1
#define SS_KALIGN 256 /* Kc of every sparse operand is a multiple of this */

typedef enum {
  SS_OK = 0,
  SS_ERR_NULL = 1,        /* a required pointer is NULL */
  SS_ERR_SHAPE = 2,       /* a size or leading dimension is invalid */
  SS_ERR_ALIGN = 3,       /* a pointer or row start is not 16-byte aligned */
  SS_ERR_DTYPE = 4,       /* unsupported data-type combination */
  SS_ERR_PATTERN = 5,     /* n outside 2..8 */
  SS_ERR_UNSUPPORTED = 6, /* valid request the library does not implement */
  SS_ERR_HIP = 7          /* a HIP call or kernel launch failed */
} ss_status;

typedef enum { SS_F32 = 0, SS_BF16 = 1, SS_I8 = 2, SS_FP8E4M3 = 3, SS_I32 = 4 } ss_dtype;

typedef enum {
  SS_SPARSE_W = 0, /* compressed operand = weights W' [N][Kc]; dense = activations [M][Kc] */
  SS_SPARSE_X = 1  /* compressed operand = activations [M][Kc]; dense = weights W [N][Kc] */
} ss_side;

/* Kc for K original columns and pattern n: ceil(K/2n)*4(n-1) rounded up to
 * SS_KALIGN (n = 2 gives K rounded up). Returns -1 for K < 0 or a bad n.
 * SlideSparse article, sliding-window section (8 positions become 12). */
int64_t ss_lifted_k(int64_t K, int n);
/* The same without the SS_KALIGN rounding: ceil(K/2n)*4(n-1). */
int64_t ss_lifted_k_logical(int64_t K, int n);

const char* ss_status_string(int status);
/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* ss_last_error(void);
int ss_version(void);

/* ss_prune24 -- offline 2:4 weight preparation.
 * Deep reading of arXiv 2610.28947 (introduction, section 2.3: magnitude
 * pruning of the weight operand; 2:4 keeps two of every four consecutive
 * elements along K) and the LLM Compressor guide (2:4 row: per-channel
 * weight quantisation).
 * W [rows][K] (F32 or BF16, row stride ldw elements), K % 4 == 0.
 * Keeps the two largest |w| of every 4-group (ties keep the lower index),
 * then per row: out_dt I8 / FP8E4M3 -> codes + scale[rows]; BF16 -> the kept
 * values rounded to bf16 (from F32) or copied (from BF16), scale must be NULL.
 * Outputs: vals [rows][Kc/2] (ldv elements), meta [rows][Kc/8] (ldm bytes),
 * Kc = ss_lifted_k(K, 2). */
ss_status ss_prune24(const void* W, ss_dtype w_dt, int64_t rows, int64_t K, int64_t ldw,
                     ss_dtype out_dt, void* vals, int64_t ldv, uint8_t* meta, int64_t ldm,
                     float* scale, void* stream);

/* ss_slide_decompose -- offline (2n-2):2n weight preparation.
 * SlideSparse article (sliding-window decomposition section; figure 2) and
 * SlideSparse blog sections 2.2-2.3: zero-pad K to a multiple of 2n, keep the
 * 2n-2 largest |w| of every 2n-group (ties keep the lower index), give each
 * nonzero to one of the n-1 windows spanning positions 2w..2w+3 (each window,
 * in order, takes the not yet taken nonzeros of its span in ascending position
 * until it holds two), and write window w of group g as the 4-group
 * (n-1)g + w of W' [rows][K']. Then per-row quantisation and 2:4 compression
 * as in ss_prune24 (I8 / FP8E4M3 / BF16). n = 2 gives the same bytes as
 * ss_prune24. Outputs span Kc = ss_lifted_k(K, n). Any K >= 1. */
ss_status ss_slide_decompose(const void* W, ss_dtype w_dt, int64_t rows, int64_t K, int64_t ldw,
                             int n, ss_dtype out_dt, void* vals, int64_t ldv, uint8_t* meta,
                             int64_t ldm, float* scale, void* stream);

/* ss_quant_lift_act -- online activation preparation (one fused pass).
 * SlideSparse article (activation lifting is an index map fused into the
 * per-token quantisation kernel) and SlideSparse blog section 3.2 (absmax,
 * scale, quantise, clamp, slide and pack in one kernel; window base
 * 2n*group + 2*offset). LLM Compressor guide: dynamic per-token scales.
 * X [M][K] (BF16 or F32, ldx elements) -> per-token absmax over the original
 * K, scale sx[M] (float32), codes q_dt (I8 or FP8E4M3) lifted to
 * Xq [M][Kc] (ldq elements), Kc = ss_lifted_k(K, n):
 *   Xq[m][4(n-1)g + 4w + j] = q(X[m][2n g + 2w + j]), sources >= K and the
 *   padding columns are 0. n = 2 is plain per-token quantisation (no lift). */
ss_status ss_quant_lift_act(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx, int n,
                            ss_dtype q_dt, void* Xq, int64_t ldq, float* sx, void* stream);

/* ss_prune24_act -- online 2:4 prune and compress of activations.
 * Deep reading of arXiv 2610.28947, section 1 (activations are produced at
 * run time and must be pruned and compressed before every product; that time
 * counts) and section 2.3. X [M][K] BF16, K % 4 == 0: keep the two largest
 * bf16 magnitudes of every 4-group (ties keep the lower index). out_dt BF16:
 * values copied, sx must be NULL; I8 / FP8E4M3: per-token scale sx[M] from
 * the row absmax and the kept values quantised. Outputs span
 * Kc = ss_lifted_k(K, 2). */
ss_status ss_prune24_act(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                         ss_dtype out_dt, void* vals, int64_t ldv, uint8_t* meta, int64_t ldm,
                         float* sx, void* stream);

/* ss_spgemm -- the 2:4 sparse product with the rescale epilogue.
 * Deep reading of arXiv 2610.28947 (introduction: one operand keeps two of
 * every four along the accumulate axis; section 3.1: sparse-weight and
 * sparse-activation cases) and SlideSparse blog section 2.2 step 3; the
 * rescale follows the LLM Compressor W8A8 scheme.
 *   side SS_SPARSE_W: sp = W' vals/meta [N][Kc], dense = X' [M][Kc].
 *   side SS_SPARSE_X: sp = X vals/meta [M][Kc], dense = W [N][Kc].
 *   acc[m][n] = sum_k X'[m][k] W'[n][k]  (i32 for I8; f32 for FP8E4M3/BF16)
 *   Y[m][n] = fl32(fl32(float(acc) * sx[m]) * sw[n]) rounded to y_dt (BF16:
 *   nearest-even); a NULL sx or sw skips that factor. y_dt SS_I32 (I8 only)
 *   stores the raw accumulator and ignores sx/sw.
 * ab_dt: I8, FP8E4M3 or BF16 for both operands. Kc % SS_KALIGN == 0.
 * Y [M][N] with ldy elements; Y itself must be 16-byte aligned, its rows need
 * not be. M, N may be any size >= 0. */
ss_status ss_spgemm(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt,
                    const void* sp_vals, int64_t ldsv, const uint8_t* sp_meta, int64_t ldsm,
                    const void* dense, int64_t ldd, const float* sx, const float* sw,
                    ss_dtype y_dt, void* Y, int64_t ldy, void* stream);

/* Tiled sparse operand -- the layout ss_spgemm_tiled streams.
 * A re-arrangement of a compressed operand (same values, same 2:4 positions)
 * into the lane order of the gfx950 structured-sparse instructions
 * (16x16x128 for I8/FP8E4M3, 16x16x64 for BF16), so that each wave's share of
 * a K step is one contiguous 1 KB block. A step is 64 compressed bytes of a
 * row: 128 K positions for 8-bit values, 64 for BF16. With
 * KS = Kc*es/128 (es = value bytes), G = ceil(KS/4), RB = ceil(rows/16):
 *   tvals: RB*4G blocks of 1024 bytes; block (b, s) at byte (b*4G + s)*1024;
 *     its bytes 16l..16l+15 (l = 0..63) are bytes 64s + 16(l/16) .. +15 of
 *     row 16b + l%16 of vals (row-major, in bytes); rows >= rows and steps
 *     s >= KS hold zeros.
 *   tmeta, 8-bit values: RB*G blocks of 1024 bytes; block (b, g) at byte
 *     (b*G + g)*1024; its 32-bit word 4l + q is meta[16b + l%16][16(4g+q) +
 *     4(l/16) .. +3] as a little-endian word (the 16x16x128 index operand of
 *     lane l); padding words 0x44444444.
 *   tmeta, BF16 values: RB*G blocks of 512 bytes; block (b, g) at byte
 *     (b*G + g)*512; its 16-bit word 4l + q is meta[16b + l%16][8(4g+q) +
 *     2(l/16) .. +1] (the 16x16x64 index of lane l); padding 0x4444.
 * Return the byte sizes of the two buffers for value type dt (I8, FP8E4M3 or
 * BF16); -1 for a bad argument. */
int64_t ss_tiled_vals_bytes(int64_t rows, int64_t Kc, ss_dtype dt);
int64_t ss_tiled_meta_bytes(int64_t rows, int64_t Kc, ss_dtype dt);

/* ss_pack_sparse -- compressed operand (row-major, as written by ss_prune24,
 * ss_slide_decompose or ss_prune24_act) -> tiled operand. A layout change
 * only (deep reading of arXiv 2610.28947, section 2.3: values plus 2-bit
 * positions). dt: I8, FP8E4M3 or BF16. vals [rows][Kc/2] (ldv elements),
 * meta [rows][Kc/8] (ldm bytes); tvals / tmeta: ss_tiled_vals_bytes /
 * ss_tiled_meta_bytes bytes, 16-byte aligned, written completely.
 * Kc % SS_KALIGN == 0. */
ss_status ss_pack_sparse(int64_t rows, int64_t Kc, ss_dtype dt, const void* vals, int64_t ldv,
                         const uint8_t* meta, int64_t ldm, void* tvals, uint8_t* tmeta, void* stream);

/* ss_prune24_act_tiled -- ss_prune24_act with its output written directly in
 * the tiled layout (one pass instead of ss_prune24_act + ss_pack_sparse; the
 * bytes are identical to that pair). Same sources as ss_prune24_act. X [M][K]
 * BF16 (ldx elements), K % 4 == 0; out_dt I8 / FP8E4M3 (sx[M] per-token
 * scales) or BF16 (sx NULL); tvals / tmeta sized by ss_tiled_vals_bytes /
 * ss_tiled_meta_bytes for (M, ss_lifted_k(K, 2), out_dt), 16-byte aligned,
 * written completely. */
ss_status ss_prune24_act_tiled(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx,
                               ss_dtype out_dt, void* tvals, uint8_t* tmeta, float* sx, void* stream);

/* ss_slide_decompose_tiled -- ss_slide_decompose with its output written
 * directly in the tiled layout (one pass instead of ss_slide_decompose +
 * ss_pack_sparse; the bytes are identical to that pair). Same sources as
 * ss_slide_decompose; n = 2 is the 2:4 prune of ss_prune24 (any K: the last
 * 4-group is zero-padded). W [rows][K] F32 or BF16 (ldw elements); out_dt
 * I8 / FP8E4M3 (scale[rows] per-channel scales) or BF16 (scale NULL);
 * tvals / tmeta sized by ss_tiled_vals_bytes / ss_tiled_meta_bytes for
 * (rows, ss_lifted_k(K, n), out_dt), 16-byte aligned, written completely. */
ss_status ss_slide_decompose_tiled(const void* W, ss_dtype w_dt, int64_t rows, int64_t K, int64_t ldw, int n,
                                   ss_dtype out_dt, void* tvals, uint8_t* tmeta, float* scale, void* stream);

/* ss_spgemm_tiled -- ss_spgemm on a tiled sparse operand.
 * Same product, scales, sides and output rules as ss_spgemm (same sources).
 * The sparse operand is tvals/tmeta of ss_pack_sparse for its rows (N for
 * side SS_SPARSE_W, M for SS_SPARSE_X), Kc and ab_dt; dense [rows][Kc] with
 * ldd elements of ab_dt. 0 < Kc, Kc % SS_KALIGN == 0; the dense operand must
 * span less than 4 GiB (else SS_ERR_UNSUPPORTED); Y as in ss_spgemm. I8 and
 * FP8E4M3 products need both sx and sw unless y_dt is SS_I32; for BF16 a NULL
 * scale skips that factor. Side SS_SPARSE_W with at most 64 tokens and too few
 * 256-row tiles to fill the GPU runs a row-block kernel (same results; FP8 and
 * BF16 sums in a different order). */
ss_status ss_spgemm_tiled(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt,
                          const void* tvals, const uint8_t* tmeta, const void* dense, int64_t ldd,
                          const float* sx, const float* sw, ss_dtype y_dt, void* Y, int64_t ldy,
                          void* stream);

/* ss_spgemm_tiled_workspace_bytes -- bytes of device workspace that
 * ss_spgemm_tiled_ws uses for this problem on the current device; 0 when the
 * problem takes no workspace (then ss_spgemm_tiled_ws equals
 * ss_spgemm_tiled); -1 for invalid arguments. Today: side SS_SPARSE_W with
 * 17..64 tokens and too few 256-row tiles to fill the GPU (the decode regime
 * of the SlideSparse blog, section 5.1). */
int64_t ss_spgemm_tiled_workspace_bytes(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt);

/* ss_spgemm_tiled_ws -- ss_spgemm_tiled with a caller-owned workspace that
 * lets few-token products split K across workgroups: each writes a partial
 * tile (int32 for I8 -- exact; fp32 otherwise) and a second kernel sums the
 * splits in a fixed order before the same epilogue (FP8/BF16 sums in a
 * different order than ss_spgemm_tiled, within the same 1e-2 bound).
 * workspace: device memory, 16-byte aligned, ws_bytes >= the query above
 * (SS_ERR_NULL / SS_ERR_ALIGN / SS_ERR_SHAPE otherwise); NULL with ws_bytes 0
 * is accepted when the query returns 0. Its contents need no initialisation
 * and are undefined afterwards; calls that share a workspace must be
 * stream-ordered. Other arguments and errors as ss_spgemm_tiled. */
ss_status ss_spgemm_tiled_ws(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt, const void* tvals,
                             const uint8_t* tmeta, const void* dense, int64_t ldd, const float* sx, const float* sw,
                             ss_dtype y_dt, void* Y, int64_t ldy, void* workspace, int64_t ws_bytes, void* stream);

/* ss_spgemm_tiled_noalloc -- ss_spgemm_tiled_ws for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the split-K partial tiles go to the
 * library's own static device array of SS_NOALLOC_SCRATCH_BYTES (8 MiB) on
 * the current GPU instead of a caller workspace. The array is part of the
 * library's code object: each GPU the library runs on holds its own copy
 * until the process ends; its address is looked up (hipGetSymbolAddress) on
 * the first call on each device and kept. The call allocates nothing (no
 * hipMalloc / hipFree, no allocating library routine). No part of the array
 * needs clearing: every split writes its whole partial tile before the
 * reduction reads it. Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (different streams or threads) race: order them.
 * A problem whose workspace (ss_spgemm_tiled_workspace_bytes) exceeds the
 * array returns SS_ERR_UNSUPPORTED with nothing launched (the split-K plan
 * needs at most 32 KiB per compute unit: 8 MiB on a 256-CU GPU). Arguments,
 * results (bit for bit) and other errors as ss_spgemm_tiled_ws. */
#define SS_NOALLOC_SCRATCH_BYTES (8 << 20)
ss_status ss_spgemm_tiled_noalloc(ss_side side, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt, const void* tvals,
                                  const uint8_t* tmeta, const void* dense, int64_t ldd, const float* sx,
                                  const float* sw, ss_dtype y_dt, void* Y, int64_t ldy, void* stream);

/* ss_quant_spgemm_prefill -- a prefill layer with the per-token quantisation
 * inside the sparse product (the SlideSparse blog, section 3.2, fuses the
 * activation lift into the per-token quantisation kernel; here both move into
 * the product's prologue, so the coded activations never go through HBM):
 * Y [M, N] = X W'^T with X [M, K] bf16 (ldx elements, rows 16-byte aligned),
 * K % 128 == 0 (SS_ERR_SHAPE otherwise), q_dt I8 or FP8E4M3, the 2:4 weights
 * as ss_slide_decompose_tiled(W, 2, q_dt) writes them (tvals, tmeta, sw [N]),
 * y_dt BF16 or F32. sx [M] (float) receives the per-token scales. Three
 * launches: per-token absmax into sx, the product (which codes X with
 * fl32(Q / absmax) into its LDS stages), then sx = absmax / Q. Codes, scales
 * and outputs equal ss_quant_lift_act(X, n = 2) followed by
 * ss_spgemm_tiled bit for bit. No scratch memory. */
ss_status ss_quant_spgemm_prefill(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx, ss_dtype q_dt,
                                  const void* tvals, const uint8_t* tmeta, const float* sw, int64_t N, ss_dtype y_dt,
                                  void* Y, int64_t ldy, float* sx, void* stream);

/* ss_spgemm_tiled_batched -- `batch` independent ss_spgemm_tiled products of
 * one shape in one launch (the prefill kernel; problem b reads tvals + b *
 * tvals_stride and tmeta + b * tmeta_stride (bytes), dense + b * dense_stride,
 * sx + b * sx_stride, sw + b * sw_stride and writes Y + b * y_stride (all in
 * elements)). For the online 2:4 operand roles of attention (deep reading,
 * introduction: either operand of a product can be the 2:4 one, pruned on the
 * fly), one problem per head: side SS_SPARSE_X with the pruned Q against K
 * (reduction over the head dimension) or the pruned probabilities P against
 * V^T (reduction over the keys; the dense operand's rows run along the
 * reduction, so V is passed transposed). A tiled operand prepared in one pass
 * for all problems (ss_prune24_act_tiled on the stacked rows) splits into
 * problems when M is a multiple of 16: tvals_stride = ss_tiled_vals_bytes(M,
 * Kc, ab_dt), tmeta_stride = ss_tiled_meta_bytes(M, Kc, ab_dt). Strides must
 * keep each problem 16-byte aligned (SS_ERR_ALIGN); 0 <= batch <= 65535; other
 * arguments and errors as ss_spgemm_tiled (a stride of 0 repeats an operand). */
ss_status ss_spgemm_tiled_batched(ss_side side, int64_t batch, int64_t M, int64_t N, int64_t Kc, ss_dtype ab_dt,
                                  const void* tvals, int64_t tvals_stride, const uint8_t* tmeta, int64_t tmeta_stride,
                                  const void* dense, int64_t ldd, int64_t dense_stride, const float* sx,
                                  int64_t sx_stride, const float* sw, int64_t sw_stride, ss_dtype y_dt, void* Y,
                                  int64_t ldy, int64_t y_stride, void* stream);

/* ss_quant_lift_spgemm_decode -- few-token layer in one launch: ss_quant_lift_act
 * (per-token codes, lift to K' = ss_lifted_k(K, n)) followed by the
 * weight-sparse ss_spgemm_tiled, with the quantisation and the lift done by
 * every workgroup of the product into LDS (the SlideSparse blog, section 3.2,
 * fuses the lift into the quantisation; here both move into the product). The
 * results equal the two calls bit for bit (INT8 and FP8: the same arithmetic
 * and the same sum order as the few-token product). X [M][K] F32 or BF16 (ldx
 * elements); q_dt I8 or FP8E4M3; tvals / tmeta / sw: the weight operand of
 * ss_slide_decompose_tiled for N rows, K' and q_dt; y_dt BF16, F32 or I32 (I8
 * only: the raw accumulator); Y [M][N] (ldy elements) as in ss_spgemm;
 * sx_out: NULL or M floats that receive the per-token scales. Limits:
 * 1 <= M <= 4, M * K' <= 131072, K <= 20480 (BF16) / 16384 (F32), else
 * SS_ERR_UNSUPPORTED (then use the two calls). Every workgroup repeats the
 * quantisation, so the call pays off where launches dominate: one or two
 * tokens on layers with a short weight stream (measured ~2x on
 * Qwen2.5-7B-shaped qkv at 1-2 tokens, 1.05-1.1x on gate_up and even on down
 * at 1 token); with long K and more tokens the two calls are faster. */
ss_status ss_quant_lift_spgemm_decode(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx, int n,
                                      ss_dtype q_dt, const void* tvals, const uint8_t* tmeta, const float* sw, int64_t N,
                                      ss_dtype y_dt, void* Y, int64_t ldy, float* sx_out, void* stream);

/* ---- Block-scaled FP8 -------------------------------------------------------
 * The W8A8-FP8_BLOCK scheme of the LLM Compressor "compression schemes" guide:
 * FP8 weights with one scale per block of 128 output channels x 128 positions
 * along K, FP8 activations with one dynamic scale per token and group of 128
 * positions. Here on 2:4-sparse weights (plain pattern, K' = K): Kc =
 * ss_lifted_k(K, 2), G = Kc / 128 scale groups (a multiple of 2). Each block
 * or group is quantised as a row of ss_prune24 / ss_quant_lift_act is:
 * a = max |v| over it, codes E4M3FN(clamp(fl32(v * fl32(448 / a)))), scale
 * fl32(a / 448); an all-zero block or group (including the padding groups past
 * K) has scale 0 and zero codes. */

/* ss_prune24_block -- block-scaled weight prep, written in the tiled layout.
 * W [rows][K] F32 or BF16 (ldw elements), K % 4 == 0: 2:4 magnitude prune along
 * K on the raw values (as ss_prune24; the prune keeps every block maximum),
 * then the kept values coded with the scale of their block.
 * tvals / tmeta: ss_tiled_vals_bytes / ss_tiled_meta_bytes(rows, Kc,
 * SS_FP8E4M3) bytes, 16-byte aligned, written completely. sw: ceil(rows / 128)
 * x G floats, row-major: sw[b][g] scales rows 128b .. 128b + 127 and K
 * positions 128g .. 128g + 127. */
ss_status ss_prune24_block(const void* W, ss_dtype w_dt, int64_t rows, int64_t K, int64_t ldw, void* tvals,
                           uint8_t* tmeta, float* sw, void* stream);

/* ss_quant_group_act -- block-scaled activation prep. X [M][K] F32 or BF16
 * (ldx elements), any K >= 0; Xq [M][Kc] FP8E4M3 codes (ldq bytes, zero past
 * K); sx: M x G floats, row-major (sx[m][g] for positions 128g .. 128g + 127
 * of token m). */
ss_status ss_quant_group_act(const void* X, ss_dtype x_dt, int64_t M, int64_t K, int64_t ldx, void* Xq, int64_t ldq,
                             float* sx, void* stream);

/* ss_spgemm_tiled_block -- the weight-sparse block-scaled product:
 *   Y[m][n] = sum over g of acc_g[m][n] * fl32(sx[m][g] * sw[n / 128][g]),
 *   acc_g = sum over the 128 positions of group g of Xq[m][k] W'[n][k] (float32),
 * accumulated in float32 in group order and rounded to y_dt (BF16 nearest-even
 * or F32). tvals / tmeta from ss_prune24_block for N rows and Kc; dense = Xq
 * [M][Kc] FP8E4M3 (ldd bytes); sx, sw as written by the two calls above.
 * 0 < Kc, Kc % SS_KALIGN == 0; the dense operand must span less than 4 GiB;
 * Y [M][N] (ldy elements) as in ss_spgemm. Any M >= 0 (the prefill kernel
 * serves every size). */
ss_status ss_spgemm_tiled_block(int64_t M, int64_t N, int64_t Kc, const void* tvals, const uint8_t* tmeta,
                                const void* dense, int64_t ldd, const float* sx, const float* sw, ss_dtype y_dt,
                                void* Y, int64_t ldy, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SS_H */
