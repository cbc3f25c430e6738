"""Pins for the oracle's magnitude prune, 2:4 compression and energy metric."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy import integrate, stats

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rank_rule_keep(group, keep):
    """Independent statement of the keep rule: element i survives iff fewer than
    ``keep`` elements outrank it (larger magnitude, or equal magnitude and a
    lower index)."""
    mag = [abs(float(x)) for x in group]
    out = []
    for i, mi in enumerate(mag):
        better = sum(1 for j, mj in enumerate(mag) if mj > mi or (mj == mi and j < i))
        out.append(better < keep)
    return out


@pytest.mark.parametrize("m,keep", [(4, 2), (6, 4), (8, 6)])
def test_keep_mask_brute_force(m, keep):
    # every group over magnitudes {0,1,2} with both signs: all tie patterns
    vals = [0.0, 1.0, -1.0, 2.0, -2.0] if m == 4 else [0.0, 1.0, -2.0]
    groups = np.array(list(itertools.product(vals, repeat=m)), dtype=np.float32)
    mask = oracle.nm_keep_mask(groups.reshape(1, -1), m, keep).reshape(groups.shape)
    for g, mk in zip(groups, mask):
        assert list(mk) == _rank_rule_keep(g, keep), g


def test_keep_mask_invariants_random():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[:, ::7] = np.round(x[:, ::7])  # plant ties
    for m, keep in [(4, 2), (6, 4), (8, 6), (10, 8)]:
        xx = x[:, : (256 // m) * m]
        mk = oracle.nm_keep_mask(xx, m, keep).reshape(-1, m)
        g = np.abs(xx.reshape(-1, m))
        assert np.all(mk.sum(1) == keep)
        kept_min = np.where(mk, g, np.inf).min(1)
        drop_max = np.where(~mk, g, -np.inf).max(1)
        assert np.all(kept_min >= drop_max)


def test_handworked_prune_and_compress():
    gold = json.load(open(os.path.join(GOLD, "handworked.json")))
    for case in gold["prune24"]:
        got = oracle.nm_keep_mask(np.array([case["row"]], np.float32), 4, 2)[0]
        assert list(got) == case["keep"], case
    c = gold["compress"]
    vals, nib = oracle.compress24(np.array([c["row"]], np.float32))
    assert vals[0].tolist() == c["vals"]
    assert oracle.pack_meta(nib)[0].tolist() == c["meta_bytes"]


def test_compress_roundtrip_and_slots():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((32, 512)).astype(np.float32)
    x[rng.random(x.shape) < 0.2] = 0  # groups with fewer than 2 nonzeros
    p = oracle.prune_nm(x, 4, 2)
    vals, nib = oracle.compress24(p)
    meta = oracle.pack_meta(nib)
    assert meta.shape == (32, 512 // 8)
    back = oracle.decompress24(vals, meta, 512)
    assert np.array_equal(back, p.astype(np.float64))
    idx0, idx1 = nib & 3, nib >> 2
    assert np.all(idx0 < idx1)
    # filler slots: a group with a single nonzero at position q uses the
    # lowest free position for the other slot
    g = p.reshape(32, 128, 4)
    one = (g != 0).sum(2) == 1
    q = np.argmax(g != 0, axis=2)
    other = np.where(idx0 == q, idx1, idx0)
    expect_other = np.where(q == 0, 1, 0)
    assert np.all(other[one] == expect_other[one])


def _halfnormal_24_closed_form():
    """E[sum of squares of the two smallest of four |N(0,1)|] / 4, by
    integrating the order-statistic densities of the half-normal law."""
    F = lambda x: 2 * stats.norm.cdf(x) - 1
    f = lambda x: 2 * stats.norm.pdf(x)
    def dens(k, n, x):  # density of the k-th smallest of n
        from math import comb
        return n * comb(n - 1, k - 1) * F(x) ** (k - 1) * (1 - F(x)) ** (n - k) * f(x)
    e = sum(integrate.quad(lambda x: x * x * dens(k, 4, x), 0, np.inf)[0] for k in (1, 2))
    return e / 4.0


def test_energy_removed_gaussian():
    gold = json.load(open(os.path.join(GOLD, "bits_energy.json")))
    cf24 = _halfnormal_24_closed_form()
    cf48 = 5.0 / 24.0  # pair energies are iid exponential (mean 2): drop the 2 smallest of 4
    # the pages' rounded figures agree with the closed forms
    assert abs(cf24 - gold["energy_24"]) < gold["page_rounding"]
    assert abs(cf48 - gold["energy_paired48"]) < gold["page_rounding"]
    rng = np.random.default_rng(0)
    v = rng.standard_normal((1024, 8192))  # 2M 4-groups, 1M 8-groups
    e24 = oracle.energy_removed(v, oracle.nm_keep_mask(v, 4, 2))
    e48 = oracle.energy_removed(v, oracle.paired48_keep_mask(v))
    assert abs(e24 - cf24) < 2e-3
    assert abs(e48 - cf48) < 2e-3


def test_paired48_mask_structure():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((16, 64))
    mk = oracle.paired48_keep_mask(v).reshape(-1, 4, 2)
    assert np.all(mk[..., 0] == mk[..., 1])  # whole pairs
    assert np.all(mk[..., 0].sum(1) == 2)
    e = (v.reshape(-1, 4, 2) ** 2).sum(2)
    assert np.all(np.where(mk[..., 0], e, np.inf).min(1) >= np.where(~mk[..., 0], e, -np.inf).max(1))
