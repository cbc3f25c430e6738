"""Pins for the sparse product and the epilogue."""
import numpy as np

import oracle
import synth


def _direct_acc(vals, meta, dense, Kc):
    """Product straight from the compressed form: each kept value meets the
    dense element at its recorded position (no decompression)."""
    nib = oracle.unpack_meta(meta)
    rows = vals.shape[0]
    acc = np.zeros((dense.shape[0], rows), dtype=np.int64)
    for r in range(rows):
        for g in range(Kc // 4):
            for s in range(2):
                p = 4 * g + ((int(nib[r, g]) >> (2 * s)) & 3)
                acc[:, r] += int(vals[r, 2 * g + s]) * dense[:, p].astype(np.int64)
    return acc


def test_int8_product_exact_and_direct():
    rng = np.random.default_rng(8)
    W = rng.standard_normal((24, 256)).astype(np.float32)
    X = rng.integers(-127, 128, size=(9, 256)).astype(np.int8)
    vals, meta, sw = oracle.prune24(W, "i8")
    acc = oracle.spgemm_acc("W", vals, meta, X, 256, "i8")
    assert np.array_equal(acc.astype(np.int64), _direct_acc(vals, meta, X, 256))
    dense_w = oracle.decompress24(vals.astype(np.float64), meta, 256).astype(np.int64)
    assert np.array_equal(acc.astype(np.int64), X.astype(np.int64) @ dense_w.T)


def test_fp8_product_exact():
    """float64 sums of E4M3 products are exact: compare with integer arithmetic
    on values scaled by 2^9 (every E4M3 value is a multiple of 2^-9)."""
    rng = np.random.default_rng(9)
    W = rng.standard_normal((16, 512)).astype(np.float32)
    X = rng.standard_normal((8, 512)).astype(np.float32) * 30
    vals, meta, sw = oracle.prune24(W, "fp8")
    xq, sx = oracle.dense_quant_rows(X, "fp8")
    acc = oracle.spgemm_acc("W", vals, meta, xq, 512, "fp8")
    wi = (oracle.decompress24(oracle.e4m3_decode(vals), meta, 512) * 512).astype(np.int64)
    xi = (oracle.e4m3_decode(xq) * 512).astype(np.int64)
    exact = xi @ wi.T
    assert np.array_equal((acc * 2.0 ** 18).astype(np.int64), exact)


def test_side_x_matches_side_w_transposed():
    rng = np.random.default_rng(10)
    X = synth.f32_to_bf16_bits(rng.standard_normal((12, 128)).astype(np.float32))
    Wd = synth.f32_to_bf16_bits(rng.standard_normal((20, 128)).astype(np.float32))
    vals, meta, _ = oracle.prune24_act(X, "bf16")
    acc_x = oracle.spgemm_acc("X", vals, meta, Wd, 128, "bf16")
    acc_w = oracle.spgemm_acc("W", vals, meta, Wd, 128, "bf16")  # roles swapped
    assert np.array_equal(acc_x, acc_w.T)


def test_epilogue_order_and_types():
    acc = np.array([[1000.0, -7.0], [0.0, 2 ** 24 + 1.0]])
    sx = np.array([0.1, 2.0], np.float32)
    sw = np.array([3.0, 0.5], np.float32)
    y = oracle.epilogue(acc, sx, sw, "f32", "i8")
    assert y.dtype == np.float32
    assert y[0, 0] == np.float32(np.float32(np.float32(1000.0) * np.float32(0.1)) * np.float32(3.0))
    assert y[1, 1] == np.float32(2 ** 24) * 2 * np.float32(0.5)  # acc rounds to float32 first
    assert oracle.epilogue(acc, None, None, "i32", "i8")[1, 1] == 2 ** 24 + 1
    yb = oracle.epilogue(acc, sx, sw, "bf16", "i8")
    assert yb.dtype == np.uint16
