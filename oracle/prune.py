"""Magnitude N:M pruning along K, 2:4 compression, and the energy metric.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def nm_keep_mask(v: np.ndarray, m: int, keep: int) -> np.ndarray:
    """Keep the ``keep`` largest magnitudes of every ``m`` consecutive elements.

    2:4 keeps 2 of each 4 consecutive elements along the accumulate (K) axis
    (deep reading of arXiv 2610.28947, introduction); (2N-2):2N keeps 2N-2 of
    each 2N (SlideSparse article, introduction; SlideSparse blog section 2.1).
    The pages do not say how ties are broken: equal magnitudes keep the lower
    index (a stable descending sort), and +0 and -0 compare equal.

    ``v`` is [..., K] with K a multiple of ``m`` (callers zero-pad).
    """
    v = np.asarray(v)
    K = v.shape[-1]
    assert K % m == 0, "pad K to a multiple of the group size first"
    g = np.abs(v.astype(np.float64)).reshape(-1, m)
    order = np.argsort(-g, axis=1, kind="stable")  # descending; ties in index order
    mask = np.zeros(g.shape, dtype=bool)
    np.put_along_axis(mask, order[:, :keep], True, axis=1)
    return mask.reshape(v.shape)


def prune_nm(v: np.ndarray, m: int, keep: int) -> np.ndarray:
    """Zero every element that :func:`nm_keep_mask` drops (dtype preserved)."""
    mask = nm_keep_mask(v, m, keep)
    out = np.array(v, copy=True)
    out[~mask] = 0
    return out


def compress24(dense: np.ndarray):
    """Compress rows that hold at most 2 nonzeros per 4-group.

    Each group stores two values and a 2-bit position for each (deep reading,
    section 1: every kept value carries a position index). The two slots are
    the group's nonzeros, then its lowest-index zeros, in ascending position;
    a group's nibble is ``idx0 | idx1 << 2`` and row byte j holds groups 2j
    (low nibble) and 2j+1 (high nibble).

    Returns ``(vals [rows, K/2], nibbles [rows, K/4] uint8)``.
    """
    dense = np.asarray(dense)
    rows, K = dense.shape
    assert K % 4 == 0
    g = dense.reshape(rows, K // 4, 4)
    nz = (g != 0)
    assert nz.sum(axis=2).max(initial=0) <= 2, "group with more than 2 nonzeros"
    # slot choice = the same magnitude rule on the group: nonzeros outrank
    # zeros, and among equals the lower index wins
    keep = nm_keep_mask(dense, 4, 2).reshape(rows, K // 4, 4)
    pos = np.nonzero(keep)[2].reshape(rows, K // 4, 2)  # ascending within the group
    vals = np.take_along_axis(g, pos, axis=2).reshape(rows, K // 2)
    nib = (pos[..., 0] | (pos[..., 1] << 2)).astype(np.uint8)
    return vals, nib


def pack_meta(nib: np.ndarray) -> np.ndarray:
    """Two nibbles per byte: group 2j in bits 0-3, group 2j+1 in bits 4-7."""
    nib = np.asarray(nib, dtype=np.uint8)
    assert nib.shape[-1] % 2 == 0
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_meta(meta: np.ndarray) -> np.ndarray:
    meta = np.asarray(meta, dtype=np.uint8)
    out = np.empty(meta.shape[:-1] + (meta.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = meta & 0xF
    out[..., 1::2] = meta >> 4
    return out


def decompress24(vals: np.ndarray, meta: np.ndarray, K: int) -> np.ndarray:
    """Scatter compressed values back to dense [rows, K] (float64)."""
    vals = np.asarray(vals, dtype=np.float64)
    rows = vals.shape[0]
    nib = unpack_meta(meta)[:, : K // 4].astype(np.int64)
    idx0, idx1 = nib & 3, nib >> 2
    assert np.all(idx0 < idx1), "metadata slots must be strictly ascending"
    out = np.zeros((rows, K // 4, 4))
    v = vals[:, : K // 2].reshape(rows, K // 4, 2)
    np.put_along_axis(out, idx0[..., None], v[..., 0:1], axis=2)
    np.put_along_axis(out, idx1[..., None], v[..., 1:2], axis=2)
    return out.reshape(rows, K)


def paired48_keep_mask(v: np.ndarray) -> np.ndarray:
    """Paired 4:8: in each 8-group keep the 2 of 4 adjacent pairs with most energy.

    The sparse FP4 mode the deep reading describes (section 3.3) keeps two
    of the four adjacent pairs in every eight elements. Ties keep the lower
    pair index. Used only for the energy check.
    """
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % 8 == 0
    p = v.reshape(-1, 4, 2)
    e = (p * p).sum(axis=2)
    keep_pairs = nm_keep_mask(e, 4, 2)  # top 2 of 4 by energy, ties to lower pair
    return np.repeat(keep_pairs, 2, axis=1).reshape(v.shape)


def energy_removed(v: np.ndarray, keep: np.ndarray) -> float:
    """Share of the sum of squares that the pruning removes (deep reading, 3.1)."""
    v = np.asarray(v, dtype=np.float64)
    tot = np.sum(v * v)
    return float(np.sum((v * v)[~keep]) / tot)
