"""Block-scaled FP8: 128 x 128 weight blocks and per-token groups of 128.

Test infrastructure only (see the package docstring).

Scheme: the W8A8-FP8_BLOCK row of the LLM Compressor "compression schemes"
guide -- weights in FP8 with one scale per block of 128 output channels x 128
positions along K, activations in FP8 with one dynamic scale per token and
group of 128 consecutive positions along K. Here it is applied to a 2:4
weight (the plain pattern, K' = K): the prune runs on the unquantised
weights first, as for the per-channel scheme.

The guide fixes the granularity, not the arithmetic. Reading used here:

* every block (weights) or group (activations) is quantised exactly as one
  row is in ``quant.quant_rows``: a = max |v| over the block, inv = fl32(448/a),
  code = E4M3FN(clamp(fl32(v * inv), +-448)), s = fl32(a / 448); an all-zero
  block has s = 0 and zero codes. Edge blocks are ragged; positions past K
  and the zero padding up to K'_alloc are zeros (padding groups get s = 0).
* the 2:4 selection uses the float magnitudes (as ``paths.prune24``); the kept
  values are then coded with the scale of the block they lie in. Compressed
  column j of a row holds a value from K positions 4(j // 2) .. 4(j // 2) + 3,
  so it lies in group j // 64. A magnitude prune keeps every group maximum,
  so a block's absmax is the same before and after the prune.
* the product: y[m, n] = sum over groups g of acc_g[m, n] * s_x[m, g] *
  s_w[n // 128, g], where acc_g is the exact product of the decoded codes over
  group g's 128 positions. The oracle sums in float64 and rounds once to the
  output type; any summation order in float32 is a valid reading, so parity
  is checked to a relative Frobenius tolerance, as for the other FP8 products.
"""
from __future__ import annotations

import numpy as np

from .prune import prune_nm, compress24, pack_meta, decompress24
from .quant import quant_rows, e4m3_decode, f32_to_bf16_bits_rne, bf16_bits_to_f32
from .slide import lifted_k_alloc

BLOCK = 128  # block edge for weights, group length for activations


def _as_f32(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v)
    if v.dtype == np.uint16:
        return bf16_bits_to_f32(v)
    return v.astype(np.float32)


def _pad_cols(v: np.ndarray, width: int) -> np.ndarray:
    out = np.zeros((v.shape[0], width), dtype=v.dtype)
    out[:, : v.shape[1]] = v
    return out


def n_groups(K: int) -> int:
    """Scale groups along K: K'_alloc / 128 (K'_alloc is a multiple of 256)."""
    return lifted_k_alloc(K, 2) // BLOCK


def quant_group_act(X: np.ndarray):
    """Online activation prep: per token and group of 128 positions along K,
    FP8 codes with one scale each. Returns ``(codes [M, K'_alloc] uint8,
    scales [M, K'_alloc / 128] float32)``."""
    x = _as_f32(X)
    M, K = x.shape
    Kalloc = lifted_k_alloc(K, 2)
    xp = _pad_cols(x, Kalloc)
    codes = np.zeros((M, Kalloc), np.uint8)
    scales = np.zeros((M, Kalloc // BLOCK), np.float32)
    for g in range(Kalloc // BLOCK):
        cols = slice(g * BLOCK, (g + 1) * BLOCK)
        codes[:, cols], scales[:, g] = quant_rows(xp[:, cols], "fp8")
    return codes, scales


def prune24_block(W: np.ndarray):
    """Offline weight prep: 2:4 magnitude prune along K, compression, FP8 codes
    with one scale per 128 x 128 block. Returns ``(vals [rows, K'_alloc / 2]
    uint8, meta [rows, K'_alloc / 8] uint8, scales [ceil(rows / 128),
    K'_alloc / 128] float32)``."""
    w = _as_f32(W)
    rows, K = w.shape
    assert K % 4 == 0
    Kalloc = lifted_k_alloc(K, 2)
    vals, nib = compress24(_pad_cols(prune_nm(w, 4, 2), Kalloc))
    vals = np.where(vals == 0, np.float32(0), vals).astype(np.float32)
    nrb, ng = -(-rows // BLOCK), Kalloc // BLOCK
    codes = np.zeros(vals.shape, np.uint8)
    scales = np.zeros((nrb, ng), np.float32)
    half = BLOCK // 2  # compressed columns per group
    for b in range(nrb):
        r = slice(b * BLOCK, min((b + 1) * BLOCK, rows))
        for g in range(ng):
            c = slice(g * half, (g + 1) * half)
            blk = vals[r, c]
            q, s = quant_rows(blk.reshape(1, -1), "fp8")
            codes[r, c] = q.reshape(blk.shape)
            scales[b, g] = s[0]
    return codes, pack_meta(nib), scales


def spgemm_block_f64(sp_vals, sp_meta, dense, Kc: int, sx, sw) -> np.ndarray:
    """y [M, N] in float64 for the weight-sparse FP8 block-scaled product
    (before rounding to the output type)."""
    A = decompress24(e4m3_decode(sp_vals)[:, : Kc // 2], sp_meta, Kc)  # W' [N, Kc]
    B = e4m3_decode(dense)[:, :Kc]  # X' [M, Kc]
    sx = np.asarray(sx, np.float32).astype(np.float64)
    sw = np.asarray(sw, np.float32).astype(np.float64)
    N = A.shape[0]
    wblock = np.arange(N) // BLOCK
    y = np.zeros((B.shape[0], N))
    for g in range(Kc // BLOCK):
        cols = slice(g * BLOCK, (g + 1) * BLOCK)
        acc = B[:, cols] @ A[:, cols].T  # exact (see gemm.py)
        y += acc * (sx[:, g][:, None] * sw[wblock, g][None, :])
    return y


def spgemm_block(sp_vals, sp_meta, dense, Kc: int, sx, sw, y_dt: str) -> np.ndarray:
    """The block-scaled product rounded once to ``y_dt`` ("f32", or "bf16" as
    uint16 bits, nearest even via float32)."""
    y = spgemm_block_f64(sp_vals, sp_meta, dense, Kc, sx, sw).astype(np.float32)
    if y_dt == "f32":
        return y
    if y_dt == "bf16":
        return f32_to_bf16_bits_rne(y)
    raise ValueError(y_dt)
