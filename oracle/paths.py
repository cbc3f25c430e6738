"""The five library calls, each as a plain composition of the oracle steps.

Test infrastructure only (see the package docstring). Inputs are float32
arrays or raw bf16 bits (uint16). Every sparse output is padded along K to
``lifted_k_alloc(K, n)`` with zero groups whose metadata is positions (0, 1).
"""
from __future__ import annotations

import numpy as np

from .prune import prune_nm, compress24, pack_meta
from .slide import lifted_k_alloc, slide_decompose_dense, lift
from .quant import quant_rows, bf16_bits_to_f32, f32_to_bf16_bits_rne


def _as_f32(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v)
    if v.dtype == np.uint16:
        return bf16_bits_to_f32(v)
    return v.astype(np.float32)


def _pad_cols(v: np.ndarray, width: int) -> np.ndarray:
    out = np.zeros((v.shape[0], width), dtype=v.dtype)
    out[:, : v.shape[1]] = v
    return out


def _compress_and_code(dense_f: np.ndarray, Kalloc: int, out_dt: str):
    """Compress a <=2-per-4 float matrix, then code the kept values.

    Zero values (either sign) are stored as +0. For INT8/FP8 the kept values
    of each row are quantised with that row's absmax (which equals the absmax
    of the row before pruning, since a magnitude prune always keeps the
    largest element of each group).
    """
    vals, nib = compress24(_pad_cols(dense_f.astype(np.float32), Kalloc))
    vals = np.where(vals == 0, np.float32(0), vals).astype(np.float32)
    meta = pack_meta(nib)
    if out_dt in ("i8", "fp8"):
        codes, s = quant_rows(vals, out_dt)
        return codes, meta, s
    if out_dt == "bf16":
        return f32_to_bf16_bits_rne(vals), meta, None
    raise ValueError(out_dt)


def prune24(W: np.ndarray, out_dt: str):
    """Offline weight prep for plain 2:4: magnitude prune along K, per-channel
    quantisation, compression. Returns ``(vals, meta, scale)``."""
    w = _as_f32(W)
    K = w.shape[1]
    assert K % 4 == 0
    return _compress_and_code(prune_nm(w, 4, 2), lifted_k_alloc(K, 2), out_dt)


def slide_decompose(W: np.ndarray, n: int, out_dt: str):
    """Offline weight prep for (2n-2):2n: prune, sliding-window decomposition
    into 2:4 windows over K', per-channel quantisation, compression."""
    w = _as_f32(W)
    rows, K = w.shape
    Kp = -(-K // (2 * n)) * 2 * n
    wpad = _pad_cols(w, Kp)
    pruned = prune_nm(wpad, 2 * n, 2 * n - 2)
    wprime = slide_decompose_dense(pruned, n).astype(np.float32)  # exact copies
    return _compress_and_code(wprime, lifted_k_alloc(K, n), out_dt)


def quant_lift_act(X: np.ndarray, n: int, q: str):
    """Online activation prep: per-token quantisation over the original K, then
    the lift to K' and zero padding to K'_alloc. Returns ``(Xq, sx)``."""
    x = _as_f32(X)
    K = x.shape[1]
    codes, s = quant_rows(x, q)
    lifted = lift(codes, n)
    return _pad_cols(lifted, lifted_k_alloc(K, n)), s


def dense_quant_rows(X: np.ndarray, q: str):
    """Per-row quantisation of a dense operand (n = 2, i.e. no lift)."""
    return quant_lift_act(X, 2, q)


def prune24_act(X: np.ndarray, out_dt: str):
    """Online activation 2:4 prune and compress along K (bf16 magnitudes),
    optionally quantised per token. Returns ``(vals, meta, sx)``."""
    x = _as_f32(X)
    K = x.shape[1]
    assert K % 4 == 0
    return _compress_and_code(prune_nm(x, 4, 2), lifted_k_alloc(K, 2), out_dt)
