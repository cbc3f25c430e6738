"""Sparse matrix product and the per-token x per-channel rescale epilogue.

Test infrastructure only (see the package docstring).

The plain definition: decompress the 2:4 operand to dense and take the
ordinary matrix product in float64. For INT8 codes every partial sum is an
integer well below 2^53, and for E4M3FN codes every product is a multiple of
2^-18 below 2^17.6, so with at most 2^15 terms every partial sum fits in 51
significant bits: both products are exact. bf16 products are exact too
(16-bit significands), and their sums are exact to float64 rounding.
"""
from __future__ import annotations

import numpy as np

from .prune import decompress24
from .quant import e4m3_decode, bf16_bits_to_f32, f32_to_bf16_bits_rne


def _decode(codes: np.ndarray, ab: str) -> np.ndarray:
    if ab == "i8":
        return np.asarray(codes, dtype=np.int8).astype(np.float64)
    if ab == "fp8":
        return e4m3_decode(codes)
    if ab == "bf16":
        return bf16_bits_to_f32(codes).astype(np.float64)
    raise ValueError(ab)


def spgemm_acc(side: str, sp_vals, sp_meta, dense, Kc: int, ab: str) -> np.ndarray:
    """Accumulator [M, N] of one 2:4 product, in float64.

    side "W": the compressed operand is the weight W' [N, Kc] (rows are output
    channels) and ``dense`` is the activation X' [M, Kc]; Y = X' W'^T.
    side "X": the compressed operand is the activation X [M, Kc] and ``dense``
    is the weight W [N, Kc]; Y = X W^T. Which operand is sparse follows the
    W and X columns of the deep reading's speed table (section 3.1).
    """
    A = decompress24(_decode(sp_vals, ab)[:, : Kc // 2], sp_meta, Kc)
    B = _decode(dense, ab)[:, :Kc]
    if side == "W":
        acc = B @ A.T
    elif side == "X":
        acc = A @ B.T
    else:
        raise ValueError(side)
    if ab == "i8":
        assert np.all(np.abs(acc) <= 2 ** 31 - 1), "int32 accumulator overflow"
    return acc


def epilogue(acc: np.ndarray, sx, sw, y_dt: str, ab: str) -> np.ndarray:
    """y = fl32(fl32(fl32(acc) * s_x[m]) * s_w[n]), then to ``y_dt``.

    The per-token and per-channel scales are those of the LLM Compressor
    W8A8 scheme. ``acc`` is rounded once to float32 (nearest even). bf16
    operands carry no scales. ``y_dt`` "i32" returns the raw INT8 accumulator;
    "bf16" returns uint16 bits rounded to nearest even.
    """
    if y_dt == "i32":
        assert ab == "i8"
        return acc.astype(np.int64).astype(np.int32)
    y = acc.astype(np.float32)
    if sx is not None:
        y = (y * np.asarray(sx, np.float32)[:, None]).astype(np.float32)
    if sw is not None:
        y = (y * np.asarray(sw, np.float32)[None, :]).astype(np.float32)
    if y_dt == "f32":
        return y
    if y_dt == "bf16":
        return f32_to_bf16_bits_rne(y)
    raise ValueError(y_dt)


def spgemm(side, sp_vals, sp_meta, dense, Kc, ab, sx, sw, y_dt):
    return epilogue(spgemm_acc(side, sp_vals, sp_meta, dense, Kc, ab), sx, sw, y_dt, ab)
