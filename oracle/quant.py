"""Per-row symmetric INT8 / FP8-E4M3FN quantisation and the E4M3FN codec.

Test infrastructure only (see the package docstring). Scheme: per output
channel for weights and dynamic per token for activations (LLM Compressor
guide, W8A8-INT8 and W8A8-FP8 rows). The pages do not fix the arithmetic;
this reading is used throughout (float32 steps, each rounded once):

    a   = max |v| over the row               (exact)
    inv = fl32(Q / a),  Q = 127 (INT8) or 448 (E4M3FN)
    t   = fl32(v * inv)
    q   = clamp(rint(t), -127, 127)          (INT8, ties to even)
    q   = E4M3FN(clamp(t, -448, 448))        (FP8, nearest, ties to even)
    s   = fl32(a / Q)
    an all-zero row gives s = 0 and q = 0.
"""
from __future__ import annotations

import numpy as np

QMAX = {"i8": 127.0, "fp8": 448.0}


def e4m3_values() -> np.ndarray:
    """The 127 non-negative finite E4M3FN values, indexed by their code 0..126.

    E4M3FN (OCP 8-bit float): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
    exponent field 0 is subnormal (m * 2^-9); code 0x7F is NaN, so the largest
    finite value is 1.75 * 2^8 = 448. There are no infinities.
    """
    vals = np.empty(127)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3_values()


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8)
    mag = code & 0x7F
    assert not np.any(mag == 0x7F), "NaN code"
    v = _E4M3[mag.astype(np.int64)]
    return np.where(code & 0x80, -v, v)


def e4m3_encode(t: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code (ties to the even code), saturating at +-448.

    Negative inputs, including those that round to zero, keep the sign bit.
    """
    t = np.asarray(t, dtype=np.float64)
    a = np.minimum(np.abs(t), 448.0)
    hi = np.searchsorted(_E4M3, a, side="left")  # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3[lo]
    d_hi = _E4M3[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _E4M3[hi], hi, code).astype(np.uint8)
    sign = np.signbit(t)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def quant_rows(v: np.ndarray, q: str):
    """Quantise each row of float32 ``v`` [rows, K]. Returns ``(codes, scales)``.

    INT8 codes are int8; FP8 codes are uint8 E4M3FN bit patterns.
    """
    v = np.asarray(v, dtype=np.float32)
    Q = np.float32(QMAX[q])
    a = np.max(np.abs(v), axis=1) if v.shape[1] else np.zeros(v.shape[0], np.float32)
    zero = a == 0
    a_safe = np.where(zero, np.float32(1), a).astype(np.float32)
    inv = (Q / a_safe).astype(np.float32)
    t = (v * inv[:, None]).astype(np.float32)
    if q == "i8":
        codes = np.clip(np.rint(t), -127, 127).astype(np.int8)
        codes[zero] = 0
    elif q == "fp8":
        codes = e4m3_encode(np.clip(t, -448.0, 448.0))
        codes[zero] = 0
    else:
        raise ValueError(q)
    s = (a / Q).astype(np.float32)
    s[zero] = 0
    return codes, s


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits_rne(x))


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 of each float32, ties to even, as raw uint16 bits.

    Written from the definition: the 16 dropped bits decide the rounding; a
    remainder above half rounds up, exactly half rounds to an even result.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)
    upper = u >> 16
    rem = u & 0xFFFF
    up = (rem > 0x8000) | ((rem == 0x8000) & ((upper & 1) == 1))
    return (upper + up).astype(np.uint16)
