"""Pins for the sliding-window decomposition and the activation lift."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_68():
    g = json.load(open(os.path.join(GOLD, "slide_68_example.json")))
    n = g["n"]
    block = np.array([g["block"]], np.float64)
    owner = oracle.window_claims(block != 0, n)[0]
    assert owner.tolist() == g["owner"]
    assert oracle.slide_decompose_dense(block, n)[0].tolist() == g["expanded"]
    assert oracle.lifted_k(8, n) == g["expanded_width"]
    # the lift reads each window span of the block in order
    x = np.arange(8, dtype=np.float64)[None, :] + 10
    lifted = oracle.lift(x, n)[0].reshape(n - 1, 4)
    for w, span in enumerate(g["window_spans"]):
        assert lifted[w].tolist() == [10 + p for p in span]


@pytest.mark.parametrize("n", [2, 3, 4, 5, 6])
def test_every_pattern_decomposes_exactly(n):
    """Brute force over every nonzero pattern with at most 2n-2 nonzeros in 2n."""
    width = 2 * n
    pats = [p for p in itertools.product([0, 1], repeat=width) if sum(p) <= width - 2]
    nz = np.array(pats, dtype=bool)
    owner = oracle.window_claims(nz, n)  # raises if a nonzero is left over
    rng = np.random.default_rng(n)
    w = nz * rng.integers(1, 100, size=nz.shape)
    wp = oracle.slide_decompose_dense(w.astype(np.float64), n)
    assert wp.shape == (len(pats), 4 * (n - 1))
    assert np.all((wp.reshape(len(pats), n - 1, 4) != 0).sum(2) <= 2)
    x = rng.integers(-50, 50, size=(3, width)).astype(np.float64)
    lifted = oracle.lift(x, n)
    # exact reconstruction W x == W' lift(x), in integers
    assert np.array_equal(x @ w.T.astype(np.float64), lifted @ wp.T)
    assert np.all((owner >= 0) == nz)


def test_patterns_with_more_nonzeros_are_rejected():
    n = 4
    nz = np.ones((1, 8), dtype=bool)
    nz[0, 3] = False  # 7 nonzeros: more than 6:8 allows
    with pytest.raises(AssertionError):
        oracle.window_claims(nz, n)


def test_pattern_table_closed_forms():
    g = json.load(open(os.path.join(GOLD, "pattern_table.json")))
    for r in g["rows"]:
        n = r["n"]
        assert abs(oracle.density(n) - r["density"]) < 1e-3
        assert abs(oracle.theoretical_speedup(n) - r["speedup"]) < 5e-3
        # the decomposition uses n-1 windows: K' per 2n-group is 4(n-1)
        assert oracle.lifted_k(2 * n, n) == 4 * r["windows"]
        if "k_factor" in r:
            assert abs(oracle.expansion(n) - r["k_factor"]) < 1e-12
    ke = g["k_example"]
    assert oracle.lifted_k(ke["K"], ke["n"]) == ke["K_prime"]


def test_lift_matches_flat_window_iteration():
    """The SlideSparse blog (section 3.2) walks output windows with one flat
    index t: group = t // (N-1), offset = t % (N-1), and reads 4 inputs from
    2N*group + 2*offset."""
    rng = np.random.default_rng(4)
    for n in (2, 3, 4, 5):
        K = 2 * n * 7
        x = rng.standard_normal((5, K))
        lifted = oracle.lift(x, n)
        for t in range(lifted.shape[1] // 4):
            base = 2 * n * (t // (n - 1)) + 2 * (t % (n - 1))
            assert np.array_equal(lifted[:, 4 * t: 4 * t + 4], x[:, base: base + 4])


def test_lift_pads_ragged_k_with_zeros():
    x = np.arange(1, 15, dtype=np.float64)[None, :]  # K = 14, not a multiple of 8
    lifted = oracle.lift(x, 4)
    assert lifted.shape[1] == oracle.lifted_k(14, 4) == 24
    # the second group's sources 14, 15 are past K
    assert lifted[0, 12 + 8: 12 + 12].tolist() == [13.0, 14.0, 0.0, 0.0]


def test_lifted_k_alloc_examples():
    assert oracle.lifted_k_alloc(512, 2) == 512
    assert oracle.lifted_k_alloc(4096, 4) == 6144
    assert oracle.lifted_k(3584, 3) == 4784 and oracle.lifted_k_alloc(3584, 3) == 4864
    assert oracle.lifted_k(18944, 5) == 30320 and oracle.lifted_k_alloc(18944, 5) == 30464
