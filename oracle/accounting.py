"""Storage bits per original element and the closed forms of the patterns.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

SCALE_BITS_PER_ELEMENT = 16 / 128  # one FP16 scale per 128 elements


def bits_dense(k: float) -> float:
    """Dense INTk: k bits per element plus the shared scale (deep reading, 2.1)."""
    return k + SCALE_BITS_PER_ELEMENT


def bits_24(k: float, scaled: bool = True) -> float:
    """2:4 + k-bit values: half the elements at k bits, plus a 2-bit position
    per kept value (1 bit per original element), plus the scale share
    (deep reading, 2.1)."""
    return k / 2 + 1 + (SCALE_BITS_PER_ELEMENT if scaled else 0.0)


def bits_slide(k: float, n: int) -> float:
    """(2n-2):2n through the window decomposition: K'/K = 2(n-1)/n times the
    2:4 cost of the expanded row, plus the scale share of the original row.
    Derived here; the pages give no figure for it."""
    return expansion(n) * (k / 2 + 1) + SCALE_BITS_PER_ELEMENT


def expansion(n: int) -> float:
    """K'/K = 2(n-1)/n (SlideSparse article: 8 positions become 12 for 6:8)."""
    return 2 * (n - 1) / n


def theoretical_speedup(n: int) -> float:
    """2x sparse rate over the expanded K': n/(n-1) (SlideSparse article;
    SlideSparse blog section 2.1 table)."""
    return 2.0 / expansion(n)


def density(n: int) -> float:
    """Nonzero share of (2n-2):2n."""
    return (2 * n - 2) / (2 * n)
