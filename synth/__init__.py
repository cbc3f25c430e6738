"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws and stores inputs. It holds none of the method's
arithmetic (no pruning, quantisation, lifting or matrix products), so the CPU
oracle and the HIP path can both take their operands from here without sharing
any step of the computation.

Recipe (one numpy PCG64 stream per call, ``default_rng(seed)``):

* draws are float64 ``standard_normal`` values, multiplied by the stated
  standard deviation in float64 and cast to float32 (round to nearest even);
* bf16 tensors are those float32 values rounded to bfloat16 (nearest even) and
  kept as their raw 16-bit patterns (``numpy.uint16``);
* draw order inside one workload: X first, then W, then any outlier columns;
* outlier channels: ``round(0.01*K)`` distinct columns from ``rng.choice``;
  those columns of X are multiplied by 20 before the bf16 rounding.

The shapes stand in for the projection layers of Llama-3.1-8B and Qwen2.5-7B
that the pages benchmark; no dataset or model weight is involved.
"""
from __future__ import annotations

import numpy as np

W_STD = 0.02


def normal_f32(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """float64 N(0, std^2) draws cast once to float32."""
    return (rng.standard_normal(size=shape) * std).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return raw uint16 bits.

    Input preparation only (finite values assumed)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations_bf16(seed: int, M: int, K: int, outlier_frac: float = 0.0,
                     outlier_scale: float = 20.0) -> np.ndarray:
    """X [M, K] as bf16 bits: N(0,1), optional outlier columns scaled before rounding."""
    rng = np.random.default_rng(seed)
    x = normal_f32(rng, (M, K))
    if outlier_frac > 0:
        cols = rng.choice(K, int(round(outlier_frac * K)), replace=False)
        x[:, cols] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(x)


def workload(seed: int, M: int, N: int, K: int, x_kind: str = "bf16",
             outlier_frac: float = 0.0, w_std: float = W_STD):
    """Draw X [M, K] then W [N, K] (float32, std ``w_std``) from one stream.

    ``x_kind`` is ``"bf16"`` (X returned as uint16 bf16 bits) or ``"f32"``.
    Returns ``(X, W, outlier_cols)``; ``outlier_cols`` is None without outliers.
    """
    rng = np.random.default_rng(seed)
    x = normal_f32(rng, (M, K))
    w = normal_f32(rng, (N, K), w_std)
    cols = None
    if outlier_frac > 0:
        cols = np.sort(rng.choice(K, int(round(outlier_frac * K)), replace=False))
        x[:, cols] *= np.float32(20.0)
    if x_kind == "bf16":
        x = f32_to_bf16_bits(x)
    elif x_kind != "f32":
        raise ValueError(x_kind)
    return x, w, cols


# The five workloads (shapes of the pages' benchmarks; every tensor synthetic).
LLAMA31_8B_LINEARS = {  # name: (K, N_out)
    "qkv": (4096, 6144),
    "o": (4096, 4096),
    "gate_up": (4096, 28672),
    "down": (14336, 4096),
}
QWEN25_7B_LINEARS = {
    "qkv": (3584, 4608),
    "gate_up": (3584, 37888),
    "down": (18944, 3584),
}

CFG_SMALL_24_INT8 = dict(M=64, N=256, K=512, n=2, x_kind="f32", q="i8", seed=0)
CFG_68_INT8 = dict(M=2048, N=4096, K=4096, n=4, x_kind="bf16", q="i8", seed=0, outlier_frac=0.01)
CFG_SPARSE_X = dict(M=8192, N=4096, K=4096, seed=0)
LLAMA_M = (2048, 4096, 8192, 16384)
QWEN_M = (1, 16, 64, 4096)
