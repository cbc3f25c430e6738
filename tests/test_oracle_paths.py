"""End-to-end pins for the five calls: bits, reconstruction and invariants."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_bits_accounting():
    g = json.load(open(os.path.join(GOLD, "bits_energy.json")))
    for k, b in g["dense_bits"].items():
        assert oracle.bits_dense(int(k)) == b
    for k24, kd in g["equal_pairs"]:
        assert oracle.bits_24(k24) == oracle.bits_dense(kd)
    assert oracle.bits_24(16, scaled=False) > oracle.bits_dense(8)
    assert oracle.bits_slide(8, 2) == oracle.bits_24(8)


def test_stored_bytes_match_bits():
    """Stored bytes of values + metadata per original element (scale excluded)."""
    K = 4080  # a multiple of 4, 6, 8 and 10, so no group padding
    W = synth.normal_f32(np.random.default_rng(11), (8, K), 0.02)
    for n in (2, 3, 4, 5):
        vals, meta, s = oracle.slide_decompose(W, n, "i8")
        bits = 8 * (vals.nbytes + meta.nbytes) / W.size
        logical = oracle.lifted_k(K, n) / oracle.lifted_k_alloc(K, n)
        assert abs(bits * logical - (oracle.bits_slide(8, n) - 0.125)) < 1e-9


@pytest.mark.parametrize("n", [3, 4, 5])
@pytest.mark.parametrize("K", [240, 250, 4096])
def test_reconstruction_through_paths(n, K):
    """INT8 accumulators through W' and lift(X) equal those of the pruned W and
    X directly, exactly (the decomposition loses nothing)."""
    X, W, _ = synth.workload(12 + n, 7, 33, K, x_kind="bf16")
    vals, meta, sw = oracle.slide_decompose(W, n, "i8")
    xq, sx = oracle.quant_lift_act(X, n, "i8")
    Kc = oracle.lifted_k_alloc(K, n)
    acc = oracle.spgemm_acc("W", vals, meta, xq, Kc, "i8")
    # direct: quantise the pruned W with the same per-row scale, and X over K
    w32 = W.astype(np.float32)
    Kp = -(-K // (2 * n)) * 2 * n
    wpad = np.zeros((33, Kp), np.float32)
    wpad[:, :K] = w32
    wp = oracle.prune_nm(wpad, 2 * n, 2 * n - 2)
    wq, sw2 = oracle.quant_rows(wp, "i8")
    xq2, sx2 = oracle.quant_rows(oracle.bf16_bits_to_f32(X), "i8")
    assert np.array_equal(sw, sw2) and np.array_equal(sx, sx2)
    direct = xq2.astype(np.int64) @ wq[:, :K].astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), direct)


def test_quantise_commutes_with_lift():
    X, _, _ = synth.workload(13, 5, 1, 96, x_kind="bf16")
    x32 = oracle.bf16_bits_to_f32(X)
    for n in (2, 3, 4, 5):
        for q in ("i8", "fp8"):
            a, sa = oracle.quant_lift_act(X, n, q)
            lifted = oracle.lift(x32, n)
            b, sb = oracle.quant_rows(lifted, q)
            assert np.array_equal(sa, sb)
            assert np.array_equal(a[:, : b.shape[1]], b)
            assert not np.any(a[:, b.shape[1]:])


def test_slide_n2_equals_prune24():
    _, W, _ = synth.workload(14, 1, 40, 512)
    for q in ("i8", "fp8", "bf16"):
        a = oracle.slide_decompose(W, 2, q)
        b = oracle.prune24(W, q)
        for u, v in zip(a, b):
            assert (u is None and v is None) or np.array_equal(u, v)


def test_weight_scale_unchanged_by_prune():
    _, W, _ = synth.workload(15, 1, 16, 512)
    for n in (2, 4):
        _, _, s = oracle.slide_decompose(W, n, "i8")
        _, s_full = oracle.quant_rows(W, "i8")
        assert np.array_equal(s, s_full)


def test_prune24_act_fp8_uses_full_row_absmax():
    X, _, _ = synth.workload(16, 9, 1, 256, x_kind="bf16")
    vals, meta, sx = oracle.prune24_act(X, "fp8")
    _, s_full = oracle.quant_rows(oracle.bf16_bits_to_f32(X), "fp8")
    assert np.array_equal(sx, s_full)
    assert vals.shape == (9, 128) and meta.shape == (9, 32)


def test_zero_row_and_padding():
    W = np.zeros((2, 24), np.float32)
    W[1, 5] = 3.0
    vals, meta, s = oracle.slide_decompose(W, 4, "i8")
    assert s[0] == 0 and not vals[0].any()
    assert vals.shape == (2, oracle.lifted_k_alloc(24, 4) // 2)
    # zero groups use positions (0, 1): nibble 0b0100
    assert np.all(oracle.unpack_meta(meta)[0] == 4)
