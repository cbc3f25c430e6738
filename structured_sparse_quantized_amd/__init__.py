"""Python binding of ``libss.so``, the gfx950 structured-sparse quantised GEMM library.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in ``include/ss.h``. PyTorch supplies device memory and the current
stream. There is no CPU fallback: importing this package raises if the
library has not been built, and every call raises ``SSError`` on a non-OK
status.

Functions keep the names of the C entry points:

    lifted_k(K, n)                          -> Kc (K' rounded up to KALIGN)
    prune24(W, out_dtype)                   -> (vals, meta, scale | None)
    slide_decompose(W, n, out_dtype)        -> (vals, meta, scale | None)
    quant_lift_act(X, n, q_dtype)           -> (Xq, sx)
    prune24_act(X, out_dtype)               -> (vals, meta, sx | None)
    spgemm(side, M, N, Kc, vals, meta, dense, sx, sw, y_dtype) -> Y [M, N]
    tiled_bytes(rows, Kc, dtype)            -> (tvals bytes, tmeta bytes)
    pack_sparse(vals, meta)                 -> (tvals, tmeta)  tiled operand
    prune24_act_tiled(X, out_dtype)         -> (tvals, tmeta, sx | None)
    slide_decompose_tiled(W, n, out_dtype)  -> (tvals, tmeta, scale | None)
    spgemm_tiled(side, M, N, Kc, tvals, tmeta, dense, sx, sw, y_dtype) -> Y [M, N]
        (takes a workspace from torch when ss_spgemm_tiled_workspace_bytes asks for one)
    spgemm_tiled_workspace_bytes(side, M, N, Kc, dtype) -> int
    spgemm_tiled_noalloc(side, M, N, Kc, tvals, tmeta, dense, sx, sw, y_dtype) -> Y  (static scratch, no workspace)
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libss.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with structured_sparse_quantized_amd.build.build()")
lib = ctypes.CDLL(_LIB_PATH)

SS_OK, SS_ERR_NULL, SS_ERR_SHAPE, SS_ERR_ALIGN, SS_ERR_DTYPE, SS_ERR_PATTERN, SS_ERR_UNSUPPORTED, SS_ERR_HIP = range(8)
SS_F32, SS_BF16, SS_I8, SS_FP8E4M3, SS_I32 = range(5)
SS_SPARSE_W, SS_SPARSE_X = 0, 1
KALIGN = 256

_i64, _int, _vp, _fp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
lib.ss_lifted_k.argtypes = [_i64, _int]
lib.ss_lifted_k.restype = _i64
lib.ss_lifted_k_logical.argtypes = [_i64, _int]
lib.ss_lifted_k_logical.restype = _i64
lib.ss_status_string.argtypes = [_int]
lib.ss_status_string.restype = ctypes.c_char_p
lib.ss_last_error.argtypes = []
lib.ss_last_error.restype = ctypes.c_char_p
lib.ss_version.restype = _int
lib.ss_prune24.argtypes = [_vp, _int, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _fp, _vp]
lib.ss_slide_decompose.argtypes = [_vp, _int, _i64, _i64, _i64, _int, _int, _vp, _i64, _vp, _i64, _fp, _vp]
lib.ss_quant_lift_act.argtypes = [_vp, _int, _i64, _i64, _i64, _int, _int, _vp, _i64, _fp, _vp]
lib.ss_prune24_act.argtypes = [_vp, _int, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _fp, _vp]
lib.ss_spgemm.argtypes = [_int, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _fp, _fp, _int, _vp, _i64, _vp]
lib.ss_tiled_vals_bytes.argtypes = [_i64, _i64, _int]
lib.ss_tiled_vals_bytes.restype = _i64
lib.ss_tiled_meta_bytes.argtypes = [_i64, _i64, _int]
lib.ss_tiled_meta_bytes.restype = _i64
lib.ss_pack_sparse.argtypes = [_i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _vp, _vp]
lib.ss_prune24_act_tiled.argtypes = [_vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _fp, _vp]
lib.ss_slide_decompose_tiled.argtypes = [_vp, _int, _i64, _i64, _i64, _int, _int, _vp, _vp, _fp, _vp]
lib.ss_spgemm_tiled.argtypes = [_int, _i64, _i64, _i64, _int, _vp, _vp, _vp, _i64, _fp, _fp, _int, _vp, _i64, _vp]
lib.ss_spgemm_tiled_workspace_bytes.argtypes = [_int, _i64, _i64, _i64, _int]
lib.ss_spgemm_tiled_workspace_bytes.restype = _i64
lib.ss_spgemm_tiled_ws.argtypes = [_int, _i64, _i64, _i64, _int, _vp, _vp, _vp, _i64, _fp, _fp, _int, _vp, _i64, _vp,
                                   _i64, _vp]
lib.ss_spgemm_tiled_noalloc.argtypes = [_int, _i64, _i64, _i64, _int, _vp, _vp, _vp, _i64, _fp, _fp, _int, _vp, _i64,
                                        _vp]
lib.ss_quant_spgemm_prefill.argtypes = [_vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _fp, _i64, _int, _vp, _i64, _fp,
                                        _vp]
lib.ss_prune24_block.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _vp, _fp, _vp]
lib.ss_quant_group_act.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _i64, _fp, _vp]
lib.ss_spgemm_tiled_block.argtypes = [_i64, _i64, _i64, _vp, _vp, _vp, _i64, _fp, _fp, _int, _vp, _i64, _vp]
lib.ss_spgemm_tiled_batched.argtypes = [_int, _i64, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _fp,
                                        _i64, _fp, _i64, _int, _vp, _i64, _i64, _vp]
lib.ss_quant_lift_spgemm_decode.argtypes = [_vp, _int, _i64, _i64, _i64, _int, _int, _vp, _vp, _fp, _i64, _int, _vp, _i64,
                                            _fp, _vp]
for _f in ("ss_prune24", "ss_slide_decompose", "ss_quant_lift_act", "ss_prune24_act", "ss_spgemm", "ss_pack_sparse",
           "ss_prune24_act_tiled", "ss_slide_decompose_tiled", "ss_spgemm_tiled", "ss_spgemm_tiled_ws",
           "ss_spgemm_tiled_noalloc", "ss_prune24_block", "ss_quant_group_act", "ss_spgemm_tiled_block",
           "ss_quant_lift_spgemm_decode", "ss_spgemm_tiled_batched", "ss_quant_spgemm_prefill"):
    getattr(lib, _f).restype = _int

EXPORTS = ("ss_lifted_k", "ss_lifted_k_logical", "ss_status_string", "ss_last_error", "ss_version",
           "ss_prune24", "ss_slide_decompose", "ss_quant_lift_act", "ss_prune24_act", "ss_spgemm",
           "ss_tiled_vals_bytes", "ss_tiled_meta_bytes", "ss_pack_sparse", "ss_prune24_act_tiled",
           "ss_slide_decompose_tiled", "ss_spgemm_tiled", "ss_spgemm_tiled_workspace_bytes", "ss_spgemm_tiled_ws",
           "ss_spgemm_tiled_noalloc", "ss_prune24_block", "ss_quant_group_act", "ss_spgemm_tiled_block",
           "ss_quant_lift_spgemm_decode", "ss_spgemm_tiled_batched", "ss_quant_spgemm_prefill")


class SSError(RuntimeError):
    def __init__(self, status: int, detail: str | None = None):
        self.status = status
        msg = lib.ss_status_string(status).decode()
        if detail is None:
            detail = lib.ss_last_error().decode()
        super().__init__(f"{msg}: {detail}")


# Size checks made before a call reaches the C ABI: the library validates sizes, strides and alignment, but
# it cannot see how large a tensor behind a pointer is. A tensor smaller than the region a call reads or
# writes raises SSError(SS_ERR_SHAPE), a host tensor SSError(SS_ERR_UNSUPPORTED), before anything launches.
def _bytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _need_bytes(t, nbytes: int, name: str) -> None:
    if t is None:
        return
    if not t.is_contiguous() or _bytes(t) < nbytes:
        raise SSError(SS_ERR_SHAPE, f"{name}: needs {nbytes} contiguous bytes, has {_bytes(t)}"
                      f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def _need_mat(t, rows: int, cols: int, name: str) -> None:
    """A row-major matrix of at least rows x cols elements (rows may be padded: a larger leading dimension)."""
    if t is None:
        return
    if t.dim() != 2 or t.shape[0] < rows or t.shape[1] < cols or (t.shape[0] > 0 and t.stride(1) != 1):
        raise SSError(SS_ERR_SHAPE, f"{name}: needs a row-major [{rows}, >= {cols}] matrix, has "
                      f"{list(t.shape)} with strides {list(t.stride())}")


def _need_vec(t, n: int, name: str) -> None:
    if t is None:
        return
    if t.numel() < n or (t.dim() == 1 and t.stride(0) != 1):
        raise SSError(SS_ERR_SHAPE, f"{name}: needs {n} contiguous elements, has {t.numel()}")


def _need_dtype(t, dt, name: str) -> None:
    if t is not None and t.dtype != dt:
        raise SSError(SS_ERR_DTYPE, f"{name}: needs {dt}, has {t.dtype}")


def _on_gpu(*ts) -> None:
    for t in ts:
        if t is not None and t.device.type != "cuda":
            raise SSError(SS_ERR_UNSUPPORTED, f"tensor on {t.device}: the library runs on the GPU only")


def _check(status: int) -> None:
    if status != SS_OK:
        raise SSError(status)


_TORCH = {
    SS_F32: torch.float32, SS_BF16: torch.bfloat16, SS_I8: torch.int8,
    SS_FP8E4M3: torch.float8_e4m3fn, SS_I32: torch.int32,
}
_NAMES = {"f32": SS_F32, "bf16": SS_BF16, "i8": SS_I8, "fp8": SS_FP8E4M3, "i32": SS_I32}
_FROM_TORCH = {v: k for k, v in _TORCH.items()}


def dtype_code(d) -> int:
    if isinstance(d, int):
        return d
    if isinstance(d, str):
        return _NAMES[d]
    return _FROM_TORCH[d]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ld(t: torch.Tensor) -> int:
    assert t.dim() == 2 and t.stride(1) == 1, "row-major 2-D tensor expected"
    return t.stride(0)


def lifted_k(K: int, n: int) -> int:
    return int(lib.ss_lifted_k(K, n))


def lifted_k_logical(K: int, n: int) -> int:
    return int(lib.ss_lifted_k_logical(K, n))


def _alloc_sparse(rows, Kc, out, device):
    vals = torch.empty((rows, Kc // 2), dtype=_TORCH[out], device=device)
    meta = torch.empty((rows, Kc // 8), dtype=torch.uint8, device=device)
    scale = None if out == SS_BF16 else torch.empty(rows, dtype=torch.float32, device=device)
    return vals, meta, scale


def _check_sparse_out(vals, meta, scale, rows, Kc, o):
    _need_mat(vals, rows, Kc // 2, "vals")
    _need_mat(meta, rows, Kc // 8, "meta")
    _need_vec(scale, rows, "scale")
    _need_dtype(vals, _TORCH[o], "vals")
    _need_dtype(meta, torch.uint8, "meta")
    _on_gpu(vals, meta, scale)


def prune24(W: torch.Tensor, out_dtype="i8", out=None):
    """Offline 2:4 weight prune + per-channel quantisation + compression."""
    o = dtype_code(out_dtype)
    rows, K = W.shape
    Kc = lifted_k(K, 2)
    vals, meta, scale = out if out is not None else _alloc_sparse(rows, Kc, o, W.device)
    _check_sparse_out(vals, meta, scale, rows, Kc, o)
    _on_gpu(W)
    _check(lib.ss_prune24(_ptr(W), dtype_code(W.dtype), rows, K, _ld(W), o, _ptr(vals), _ld(vals), _ptr(meta),
                          _ld(meta), _ptr(scale), _stream(W.device)))
    return vals, meta, scale


def slide_decompose(W: torch.Tensor, n: int, out_dtype="i8", out=None):
    """Offline (2n-2):2n prune + sliding-window decomposition to 2:4 over K'."""
    o = dtype_code(out_dtype)
    rows, K = W.shape
    Kc = lifted_k(K, n)
    vals, meta, scale = out if out is not None else _alloc_sparse(rows, Kc, o, W.device)
    _check_sparse_out(vals, meta, scale, rows, Kc, o)
    _on_gpu(W)
    _check(lib.ss_slide_decompose(_ptr(W), dtype_code(W.dtype), rows, K, _ld(W), n, o, _ptr(vals), _ld(vals),
                                  _ptr(meta), _ld(meta), _ptr(scale), _stream(W.device)))
    return vals, meta, scale


def quant_lift_act(X: torch.Tensor, n: int = 2, q_dtype="i8", out=None):
    """Fused per-token quantisation and lift to K' (n = 2: no lift)."""
    q = dtype_code(q_dtype)
    M, K = X.shape
    Kc = lifted_k(K, n)
    if out is None:
        Xq = torch.empty((M, Kc), dtype=_TORCH[q], device=X.device)
        sx = torch.empty(M, dtype=torch.float32, device=X.device)
    else:
        Xq, sx = out
        _need_mat(Xq, M, Kc, "Xq")
        _need_vec(sx, M, "sx")
        _need_dtype(Xq, _TORCH[q], "Xq")
    _on_gpu(X, Xq, sx)
    _check(lib.ss_quant_lift_act(_ptr(X), dtype_code(X.dtype), M, K, _ld(X), n, q, _ptr(Xq), _ld(Xq), _ptr(sx),
                                 _stream(X.device)))
    return Xq, sx


def prune24_act(X: torch.Tensor, out_dtype="bf16", out=None):
    """Online 2:4 prune + compress of bf16 activations (optionally quantised)."""
    o = dtype_code(out_dtype)
    M, K = X.shape
    Kc = lifted_k(K, 2)
    vals, meta, sx = out if out is not None else _alloc_sparse(M, Kc, o, X.device)
    _check_sparse_out(vals, meta, sx, M, Kc, o)
    _on_gpu(X)
    _check(lib.ss_prune24_act(_ptr(X), dtype_code(X.dtype), M, K, _ld(X), o, _ptr(vals), _ld(vals), _ptr(meta),
                              _ld(meta), _ptr(sx), _stream(X.device)))
    return vals, meta, sx


def spgemm(side: int, M: int, N: int, Kc: int, vals: torch.Tensor, meta: torch.Tensor, dense: torch.Tensor,
           sx=None, sw=None, y_dtype="bf16", out=None):
    """Y [M, N] = sparse x dense product with the per-token x per-channel rescale."""
    y = dtype_code(y_dtype)
    rows, dn = (M, N) if side == SS_SPARSE_X else (N, M)
    _need_mat(vals, rows, Kc // 2, "vals")
    _need_mat(meta, rows, Kc // 8, "meta")
    _need_mat(dense, dn, Kc, "dense")
    _need_vec(sx, M, "sx")
    _need_vec(sw, N, "sw")
    if out is not None:
        _need_mat(out, M, N, "out")
    _need_dtype(out, _TORCH[y], "out")
    _on_gpu(vals, meta, dense, sx, sw, out)
    Y = out if out is not None else torch.empty((M, N), dtype=_TORCH[y], device=dense.device)
    _check(lib.ss_spgemm(side, M, N, Kc, dtype_code(vals.dtype), _ptr(vals), _ld(vals), _ptr(meta), _ld(meta),
                         _ptr(dense), _ld(dense), _ptr(sx), _ptr(sw), y, _ptr(Y), _ld(Y), _stream(dense.device)))
    return Y


def tiled_bytes(rows: int, Kc: int, dtype="i8"):
    d = dtype_code(dtype)
    return int(lib.ss_tiled_vals_bytes(rows, Kc, d)), int(lib.ss_tiled_meta_bytes(rows, Kc, d))


def pack_sparse(vals: torch.Tensor, meta: torch.Tensor, out=None):
    """Row-major compressed operand -> tiled operand (flat uint8 tensors)."""
    rows, half = vals.shape
    Kc = 2 * half
    if out is None:
        nv, nm = tiled_bytes(rows, Kc, vals.dtype)
        if nv < 0:
            raise SSError(SS_ERR_SHAPE)
        tv = torch.empty(nv, dtype=torch.uint8, device=vals.device)
        tm = torch.empty(nm, dtype=torch.uint8, device=vals.device)
    else:
        tv, tm = out
        nv, nm = tiled_bytes(rows, Kc, vals.dtype)
        _need_bytes(tv, nv, "tvals")
        _need_bytes(tm, nm, "tmeta")
    _on_gpu(vals, meta, tv, tm)
    _check(lib.ss_pack_sparse(rows, Kc, dtype_code(vals.dtype), _ptr(vals), _ld(vals), _ptr(meta), _ld(meta),
                              _ptr(tv), _ptr(tm), _stream(vals.device)))
    return tv, tm


def _check_tiled_product(side, M, N, Kc, ab, tvals, tmeta, dense, sx, sw, out, y, batch=1):
    rows, dn = (M, N) if side == SS_SPARSE_X else (N, M)  # sparse rows, dense rows
    nv, nm = tiled_bytes(rows, Kc, ab)
    _need_bytes(tvals, batch * nv if batch > 1 else nv, "tvals")
    _need_bytes(tmeta, batch * nm if batch > 1 else nm, "tmeta")
    if batch == 1:
        _need_mat(dense, dn, Kc, "dense")
        _need_vec(sx, M, "sx")
        _need_vec(sw, N, "sw")
        if out is not None:
            _need_mat(out, M, N, "out")
    _need_dtype(out, _TORCH[y], "out")
    _need_dtype(sx, torch.float32, "sx")
    _need_dtype(sw, torch.float32, "sw")
    _on_gpu(tvals, tmeta, dense, sx, sw, out)


def spgemm_tiled_workspace_bytes(side: int, M: int, N: int, Kc: int, dtype="i8") -> int:
    return int(lib.ss_spgemm_tiled_workspace_bytes(side, M, N, Kc, dtype_code(dtype)))


def spgemm_tiled(side: int, M: int, N: int, Kc: int, tvals: torch.Tensor, tmeta: torch.Tensor, dense: torch.Tensor,
                 sx=None, sw=None, y_dtype="bf16", out=None, workspace=None):
    """Y [M, N] = tiled-sparse x dense product with the per-token x per-channel rescale.

    Few-token weight-sparse products split K when given a workspace; with workspace=None one is taken from
    torch's allocator when the library asks for it (pass workspace=False to run without)."""
    y = dtype_code(y_dtype)
    ab = dtype_code(dense.dtype)
    _check_tiled_product(side, M, N, Kc, ab, tvals, tmeta, dense, sx, sw, out, y)
    Y = out if out is not None else torch.empty((M, N), dtype=_TORCH[y], device=dense.device)
    if workspace is False:
        _check(lib.ss_spgemm_tiled(side, M, N, Kc, ab, _ptr(tvals), _ptr(tmeta), _ptr(dense), _ld(dense), _ptr(sx),
                                   _ptr(sw), y, _ptr(Y), _ld(Y), _stream(dense.device)))
        return Y
    else:
        need = int(lib.ss_spgemm_tiled_workspace_bytes(side, M, N, Kc, ab)) if workspace is None else -1
        if workspace is None:
            ws = torch.empty(max(need, 0), dtype=torch.uint8, device=dense.device) if need > 0 else None
        else:
            ws = workspace
            _need_bytes(ws, int(lib.ss_spgemm_tiled_workspace_bytes(side, M, N, Kc, ab)), "workspace")
            _on_gpu(ws)
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.ss_spgemm_tiled_ws(side, M, N, Kc, ab, _ptr(tvals), _ptr(tmeta), _ptr(dense), _ld(dense),
                                  _ptr(sx), _ptr(sw), y, _ptr(Y), _ld(Y), _ptr(ws), nbytes, _stream(dense.device)))
    return Y


def spgemm_tiled_noalloc(side: int, M: int, N: int, Kc: int, tvals: torch.Tensor, tmeta: torch.Tensor,
                         dense: torch.Tensor, sx=None, sw=None, y_dtype="bf16", out=None):
    """spgemm_tiled for callers that cannot allocate: a few-token product that splits K keeps its partial
    tiles in the library's static per-GPU scratch (no workspace argument). Pass ``out`` to allocate nothing
    at all on the Python side either."""
    y = dtype_code(y_dtype)
    _check_tiled_product(side, M, N, Kc, dtype_code(dense.dtype), tvals, tmeta, dense, sx, sw, out, y)
    Y = out if out is not None else torch.empty((M, N), dtype=_TORCH[y], device=dense.device)
    _check(lib.ss_spgemm_tiled_noalloc(side, M, N, Kc, dtype_code(dense.dtype), _ptr(tvals), _ptr(tmeta), _ptr(dense),
                                       _ld(dense), _ptr(sx), _ptr(sw), y, _ptr(Y), _ld(Y), _stream(dense.device)))
    return Y


def spgemm_tiled_batched(side: int, batch: int, M: int, N: int, Kc: int, tvals: torch.Tensor, tmeta: torch.Tensor,
                         dense: torch.Tensor, sx=None, sw=None, y_dtype="bf16", out=None, strides=None):
    """`batch` same-shaped tiled products in one launch. ``dense`` is [batch, rows, Kc] (or any 3-D view with
    row-major rows); ``tvals`` / ``tmeta`` hold the problems' tiled operands back to back (stride = the bytes of
    one problem unless ``strides`` = (tv, tm) bytes is given); sx / sw are [batch, n] or None.
    Returns Y [batch, M, N]."""
    y = dtype_code(y_dtype)
    ab = dtype_code(dense.dtype)
    Y = out if out is not None else torch.empty((batch, M, N), dtype=_TORCH[y], device=dense.device)
    rows = M if side == SS_SPARSE_X else N
    if strides is None:
        nv, nm = tiled_bytes(rows, Kc, ab)
        strides = (nv, nm)
    nv, nm = tiled_bytes(rows, Kc, ab)
    dn = N if side == SS_SPARSE_X else M
    _need_bytes(tvals, (batch - 1) * strides[0] + nv, "tvals")
    _need_bytes(tmeta, (batch - 1) * strides[1] + nm, "tmeta")
    if dense.dim() != 3 or dense.shape[0] < batch or dense.shape[1] < dn or dense.shape[2] < Kc or dense.stride(2) != 1:
        raise SSError(SS_ERR_SHAPE, f"dense: needs [{batch}, {dn}, >= {Kc}] with unit stride, has {list(dense.shape)}")
    if Y.dim() != 3 or Y.shape[0] < batch or Y.shape[1] < M or Y.shape[2] < N or Y.stride(2) != 1:
        raise SSError(SS_ERR_SHAPE, f"out: needs [{batch}, {M}, {N}] with unit stride, has {list(Y.shape)}")
    for t, n, name in ((sx, M, "sx"), (sw, N, "sw")):  # [batch, n] per problem, or [n] shared by all
        if t is not None and not ((t.dim() == 2 and t.shape[0] >= batch and t.shape[1] >= n and t.stride(1) == 1)
                                  or (t.dim() == 1 and t.numel() >= n and t.stride(0) == 1)):
            raise SSError(SS_ERR_SHAPE, f"{name}: needs [{batch}, >= {n}] or [>= {n}], has {list(t.shape)}")
    _on_gpu(tvals, tmeta, dense, sx, sw, Y)
    def _s(t):
        return 0 if t is None else (t.stride(0) if t.dim() == 2 else 0)
    _check(lib.ss_spgemm_tiled_batched(side, batch, M, N, Kc, ab, _ptr(tvals), strides[0], _ptr(tmeta), strides[1],
                                       _ptr(dense), dense.stride(1), dense.stride(0), _ptr(sx), _s(sx), _ptr(sw),
                                       _s(sw), y, _ptr(Y), Y.stride(1), Y.stride(0), _stream(dense.device)))
    return Y


def quant_spgemm_prefill(X: torch.Tensor, tvals: torch.Tensor, tmeta: torch.Tensor, sw: torch.Tensor, N: int,
                         q_dtype="fp8", y_dtype="bf16", out=None, sx_out=None):
    """Prefill layer with the per-token quantisation inside the product (2:4 weights, K % 128 == 0): returns
    (Y [M, N], sx [M]); equal bit for bit to quant_lift_act(X, 2, q) followed by spgemm_tiled."""
    M, K = X.shape
    y, q = dtype_code(y_dtype), dtype_code(q_dtype)
    Kc = lifted_k(K, 2)
    nv, nm = tiled_bytes(N, Kc, q)
    _need_bytes(tvals, nv, "tvals")
    _need_bytes(tmeta, nm, "tmeta")
    _need_vec(sw, N, "sw")
    _need_vec(sx_out, M, "sx_out")
    if out is not None:
        _need_mat(out, M, N, "out")
    _need_dtype(out, _TORCH[y], "out")
    _on_gpu(X, tvals, tmeta, sw, out, sx_out)
    Y = out if out is not None else torch.empty((M, N), dtype=_TORCH[y], device=X.device)
    sx = sx_out if sx_out is not None else torch.empty(M, dtype=torch.float32, device=X.device)
    _check(lib.ss_quant_spgemm_prefill(_ptr(X), dtype_code(X.dtype), M, K, _ld(X), q, _ptr(tvals), _ptr(tmeta),
                                       _ptr(sw), N, y, _ptr(Y), _ld(Y), _ptr(sx), _stream(X.device)))
    return Y, sx


def quant_lift_spgemm_decode(X: torch.Tensor, n: int, tvals: torch.Tensor, tmeta: torch.Tensor, sw: torch.Tensor,
                             N: int, q_dtype="i8", y_dtype="bf16", out=None, sx_out=None):
    """Few tokens (1..4): quant+lift and the weight-sparse product in one launch; Y [M, N]."""
    M, K = X.shape
    y = dtype_code(y_dtype)
    q = dtype_code(q_dtype)
    Kc = lifted_k(K, n) if n >= 2 else 0
    nv, nm = tiled_bytes(N, Kc, q) if Kc > 0 else (0, 0)
    _need_bytes(tvals, nv, "tvals")
    _need_bytes(tmeta, nm, "tmeta")
    _need_vec(sw, N, "sw")
    _need_vec(sx_out, M, "sx_out")
    if out is not None:
        _need_mat(out, M, N, "out")
    _need_dtype(out, _TORCH[y], "out")
    _on_gpu(X, tvals, tmeta, sw, out, sx_out)
    Y = out if out is not None else torch.empty((M, N), dtype=_TORCH[y], device=X.device)
    _check(lib.ss_quant_lift_spgemm_decode(_ptr(X), dtype_code(X.dtype), M, K, _ld(X), n, dtype_code(q_dtype),
                                           _ptr(tvals), _ptr(tmeta), _ptr(sw), N, y, _ptr(Y), _ld(Y), _ptr(sx_out),
                                           _stream(X.device)))
    return Y


def prune24_act_tiled(X: torch.Tensor, out_dtype="fp8", out=None):
    """Online 2:4 prune + compress of bf16 activations, written in the tiled layout."""
    o = dtype_code(out_dtype)
    M, K = X.shape
    Kc = lifted_k(K, 2)
    if out is None:
        nv, nm = tiled_bytes(M, Kc, o)
        tv = torch.empty(nv, dtype=torch.uint8, device=X.device)
        tm = torch.empty(nm, dtype=torch.uint8, device=X.device)
        sx = None if o == SS_BF16 else torch.empty(M, dtype=torch.float32, device=X.device)
    else:
        tv, tm, sx = out
        nv, nm = tiled_bytes(M, Kc, o)
        _need_bytes(tv, nv, "tvals")
        _need_bytes(tm, nm, "tmeta")
        _need_vec(sx, M, "sx")
    _on_gpu(X, tv, tm, sx)
    _check(lib.ss_prune24_act_tiled(_ptr(X), dtype_code(X.dtype), M, K, _ld(X), o, _ptr(tv), _ptr(tm), _ptr(sx),
                                    _stream(X.device)))
    return tv, tm, sx


def slide_decompose_tiled(W: torch.Tensor, n: int, out_dtype="i8", out=None):
    """Offline (2n-2):2n prune + decomposition (n = 2: the 2:4 prune), written in the tiled layout."""
    o = dtype_code(out_dtype)
    rows, K = W.shape
    Kc = lifted_k(K, n)
    if out is None:
        nv, nm = tiled_bytes(rows, Kc, o)
        tv = torch.empty(nv, dtype=torch.uint8, device=W.device)
        tm = torch.empty(nm, dtype=torch.uint8, device=W.device)
        scale = None if o == SS_BF16 else torch.empty(rows, dtype=torch.float32, device=W.device)
    else:
        tv, tm, scale = out
        nv, nm = tiled_bytes(rows, Kc, o)
        _need_bytes(tv, nv, "tvals")
        _need_bytes(tm, nm, "tmeta")
        _need_vec(scale, rows, "scale")
    _on_gpu(W, tv, tm, scale)
    _check(lib.ss_slide_decompose_tiled(_ptr(W), dtype_code(W.dtype), rows, K, _ld(W), n, o, _ptr(tv), _ptr(tm),
                                        _ptr(scale), _stream(W.device)))
    return tv, tm, scale


# ---- block-scaled FP8 (128 x 128 weight blocks, per-token groups of 128) -------------------------------------

BLOCK = 128


def prune24_block(W: torch.Tensor, out=None):
    """Offline 2:4 prune with FP8 codes scaled per 128 x 128 block, written in the tiled layout.
    Returns (tvals, tmeta, sw [ceil(rows / 128), Kc / 128])."""
    rows, K = W.shape
    Kc = lifted_k(K, 2)
    if out is None:
        nv, nm = tiled_bytes(rows, Kc, SS_FP8E4M3)
        tv = torch.empty(nv, dtype=torch.uint8, device=W.device)
        tm = torch.empty(nm, dtype=torch.uint8, device=W.device)
        sw = torch.empty(((rows + BLOCK - 1) // BLOCK, Kc // BLOCK), dtype=torch.float32, device=W.device)
    else:
        tv, tm, sw = out
        nv, nm = tiled_bytes(rows, Kc, SS_FP8E4M3)
        _need_bytes(tv, nv, "tvals")
        _need_bytes(tm, nm, "tmeta")
        _need_mat(sw, (rows + BLOCK - 1) // BLOCK, Kc // BLOCK, "sw")
    _on_gpu(W, tv, tm, sw)
    _check(lib.ss_prune24_block(_ptr(W), dtype_code(W.dtype), rows, K, _ld(W), _ptr(tv), _ptr(tm), _ptr(sw),
                                _stream(W.device)))
    return tv, tm, sw


def quant_group_act(X: torch.Tensor, out=None):
    """Online FP8 codes with one scale per token and group of 128 positions.
    Returns (Xq [M, Kc] float8_e4m3fn, sx [M, Kc / 128])."""
    M, K = X.shape
    Kc = lifted_k(K, 2)
    if out is None:
        Xq = torch.empty((M, Kc), dtype=torch.float8_e4m3fn, device=X.device)
        sx = torch.empty((M, Kc // BLOCK), dtype=torch.float32, device=X.device)
    else:
        Xq, sx = out
        _need_mat(Xq, M, Kc, "Xq")
        _need_mat(sx, M, Kc // BLOCK, "sx")
    _on_gpu(X, Xq, sx)
    _check(lib.ss_quant_group_act(_ptr(X), dtype_code(X.dtype), M, K, _ld(X), _ptr(Xq), _ld(Xq), _ptr(sx),
                                  _stream(X.device)))
    return Xq, sx


def spgemm_tiled_block(M: int, N: int, Kc: int, tvals: torch.Tensor, tmeta: torch.Tensor, dense: torch.Tensor,
                       sx: torch.Tensor, sw: torch.Tensor, y_dtype="bf16", out=None):
    """Y [M, N]: the weight-sparse block-scaled FP8 product."""
    y = dtype_code(y_dtype)
    nv, nm = tiled_bytes(N, Kc, SS_FP8E4M3)
    _need_bytes(tvals, nv, "tvals")
    _need_bytes(tmeta, nm, "tmeta")
    _need_mat(dense, M, Kc, "dense")
    _need_mat(sx, M, Kc // BLOCK, "sx")
    _need_mat(sw, (N + BLOCK - 1) // BLOCK, Kc // BLOCK, "sw")
    if out is not None:
        _need_mat(out, M, N, "out")
    _on_gpu(tvals, tmeta, dense, sx, sw, out)
    Y = out if out is not None else torch.empty((M, N), dtype=_TORCH[y], device=dense.device)
    _check(lib.ss_spgemm_tiled_block(M, N, Kc, _ptr(tvals), _ptr(tmeta), _ptr(dense), _ld(dense), _ptr(sx), _ptr(sw),
                                     y, _ptr(Y), _ld(Y), _stream(dense.device)))
    return Y
