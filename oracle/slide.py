"""Sliding-window decomposition of (2n-2):2n blocks and activation lifting.

Test infrastructure only (see the package docstring). Pattern parameter n:
(2n-2):2n, so n=2 is plain 2:4, n=3 is 4:6, n=4 is 6:8 and n=5 is 8:10.
"""
from __future__ import annotations

import numpy as np

# The GEMM consumes K' in steps of this many dense positions; the lifted and
# decomposed operands are zero-padded up to a multiple of it.
KALIGN = 256


def lifted_k(K: int, n: int) -> int:
    """Logical K' for pattern n.

    Each 2n-group becomes n-1 windows of width 4 (SlideSparse article,
    sliding-window section: 8 elements grow to 12 for 6:8), so
    K' = ceil(K/2n) * 4(n-1). K is zero-padded to a multiple of 2n first (the
    pages only state the aligned case).
    """
    assert n >= 2
    return -(-K // (2 * n)) * 4 * (n - 1)


def lifted_k_alloc(K: int, n: int) -> int:
    """K' rounded up to a multiple of KALIGN (zero columns)."""
    kp = lifted_k(K, n)
    return -(-kp // KALIGN) * KALIGN


def window_claims(nonzero: np.ndarray, n: int) -> np.ndarray:
    """Assign each nonzero of each 2n-group to one of the n-1 windows.

    Window w spans local positions 2w..2w+3 (width 4, stride 2; for 6:8 the
    windows are 0-3, 2-5 and 4-7 per the SlideSparse article). Windows are
    visited in order; each takes the not yet assigned nonzeros in its span in
    ascending position until it holds two, so a window's overflow stays in the
    overlap it shares with the next window, which takes it (the article's
    pigeonhole argument). Returns, per position, the window index or -1 for
    zeros. Raises if a nonzero is left over, which would contradict the
    article's claim that n-1 windows always suffice.

    ``nonzero`` is bool [G, 2n].
    """
    G, width = nonzero.shape
    assert width == 2 * n
    owner = np.full((G, width), -1, dtype=np.int64)
    for w in range(n - 1):
        taken = np.zeros(G, dtype=np.int64)
        for j in range(4):
            p = 2 * w + j
            take = nonzero[:, p] & (owner[:, p] < 0) & (taken < 2)
            owner[take, p] = w
            taken += take
    if np.any(nonzero & (owner < 0)):
        raise AssertionError("nonzero left unassigned by the window cover")
    return owner


def slide_decompose_dense(wp: np.ndarray, n: int) -> np.ndarray:
    """Expand a (2n-2):2n-pruned matrix [rows, K] to W' [rows, K'] (float64).

    W'[r, 4(n-1)g + 4w + j] = W[r, 2n g + 2w + j] when window w owns that
    position, else 0. Every 4-group of W' then has at most two nonzeros.
    """
    wp = np.asarray(wp, dtype=np.float64)
    rows, K = wp.shape
    Kp = -(-K // (2 * n)) * 2 * n
    pad = np.zeros((rows, Kp))
    pad[:, :K] = wp
    G = rows * (Kp // (2 * n))
    blocks = pad.reshape(G, 2 * n)
    owner = window_claims(blocks != 0, n)
    out = np.zeros((G, n - 1, 4))
    for w in range(n - 1):
        span = blocks[:, 2 * w: 2 * w + 4]
        mine = owner[:, 2 * w: 2 * w + 4] == w
        out[:, w, :] = np.where(mine, span, 0.0)
    return out.reshape(rows, lifted_k(K, n))


def lift(x: np.ndarray, n: int) -> np.ndarray:
    """Activation lifting: gather x into the window order of W'.

    X'[m, 4(n-1)g + 4w + j] = X[m, 2n g + 2w + j]; the SlideSparse blog
    (section 3.2) gives the window base as 2N*group + 2*offset with group and
    offset from the flat window index. Source positions past K read 0.
    """
    x = np.asarray(x)
    M, K = x.shape
    Kp = -(-K // (2 * n)) * 2 * n
    pad = np.zeros((M, Kp), dtype=x.dtype)
    pad[:, :K] = x
    groups = Kp // (2 * n)
    src = np.empty(lifted_k(K, n), dtype=np.int64)
    t = 0
    for g in range(groups):
        for w in range(n - 1):
            for j in range(4):
                src[t] = 2 * n * g + 2 * w + j
                t += 1
    return pad[:, src]
