"""Pins for the block-scaled FP8 oracle (128 x 128 weight blocks, per-token
groups of 128; LLM Compressor guide, W8A8-FP8_BLOCK row).

Each pin checks the oracle against something other than its own formula: a
special case that is the already pinned per-row quantiser, exact power-of-two
invariances that expose a wrong block index, the E4M3FN error bound, and a
pure-Python loop over single elements for the product.
"""
import numpy as np
import pytest

import oracle


def _ulp_bound(t):
    """Half a unit in the last place of E4M3FN at |t| (3 mantissa bits; subnormal
    spacing 2^-9 below 2^-6)."""
    a = np.abs(t)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * 2.0 ** (e - 3)


def test_group_quant_single_group_is_row_quant():
    """K <= 128: the first group is the whole row, i.e. per-token quantisation."""
    rng = np.random.default_rng(30)
    X = rng.standard_normal((7, 100)).astype(np.float32) * 3
    codes, s = oracle.quant_group_act(X)
    ref_codes, ref_s = oracle.quant_rows(X, "fp8")
    assert codes.shape == (7, 256) and s.shape == (7, 2)
    assert np.array_equal(codes[:, :100], ref_codes) and np.array_equal(s[:, 0], ref_s)
    assert not codes[:, 100:].any() and not s[:, 1].any()  # padding group: zero codes, zero scale


def test_block_quant_single_block_is_tensor_quant():
    """At most 128 rows and 128 positions: one block, i.e. one scale for the
    whole (pruned) matrix, the per-row rule applied to the flattened kept values."""
    rng = np.random.default_rng(31)
    W = rng.standard_normal((50, 128)).astype(np.float32)
    vals, meta, s = oracle.prune24_block(W)
    v24, m24, _ = oracle.prune24(W, "fp8")  # same prune and compression, per-channel scales
    assert np.array_equal(meta, m24)
    kept, _ = oracle.compress24(oracle.prune_nm(W, 4, 2))
    ref_codes, ref_s = oracle.quant_rows(kept.reshape(1, -1), "fp8")
    assert s.shape == (1, 2) and s[0, 0] == ref_s[0] and s[0, 1] == 0
    assert np.array_equal(vals[:, :64], ref_codes.reshape(50, 64))
    assert not vals[:, 64:].any()


@pytest.mark.parametrize("k", [-3, 5])
def test_block_scaling_moves_only_that_block(k):
    """Multiplying one 128 x 128 block by 2^k multiplies its scale by 2^k and
    leaves every code and every other scale unchanged (power-of-two scaling
    is exact in every float32 step). A wrong row-block or group index fails."""
    rng = np.random.default_rng(32)
    W = rng.standard_normal((300, 520)).astype(np.float32)  # ragged in rows and K
    vals, meta, s = oracle.prune24_block(W)
    assert s.shape == (3, 6)  # K_alloc = 768
    W2 = W.copy()
    W2[128:256, 256:384] *= np.float32(2.0 ** k)
    vals2, meta2, s2 = oracle.prune24_block(W2)
    assert np.array_equal(vals2, vals) and np.array_equal(meta2, meta)
    expect = s.copy()
    expect[1, 2] *= np.float32(2.0 ** k)
    assert np.array_equal(s2, expect)


@pytest.mark.parametrize("k", [-4, 6])
def test_group_scaling_moves_only_that_group(k):
    rng = np.random.default_rng(33)
    X = rng.standard_normal((5, 300)).astype(np.float32)
    codes, s = oracle.quant_group_act(X)
    X2 = X.copy()
    X2[3, 128:256] *= np.float32(2.0 ** k)
    codes2, s2 = oracle.quant_group_act(X2)
    assert np.array_equal(codes2, codes)
    expect = s.copy()
    expect[3, 1] *= np.float32(2.0 ** k)
    assert np.array_equal(s2, expect)


def test_block_max_codes_to_448_and_error_bound():
    rng = np.random.default_rng(34)
    W = (rng.standard_normal((256, 384)) * rng.uniform(0.01, 10, (256, 1))).astype(np.float32)
    W[0:128, 0:128] = 0  # an all-zero block
    vals, meta, s = oracle.prune24_block(W)
    assert s[0, 0] == 0 and not vals[0:128, 0:64].any()
    dense_codes = oracle.decompress24(oracle.e4m3_decode(vals), meta, 512)
    pruned = np.zeros((256, 512), np.float32)
    pruned[:, :384] = oracle.prune_nm(W, 4, 2)
    for b in range(2):
        for g in range(4):
            blk = pruned[128 * b:128 * (b + 1), 128 * g:128 * (g + 1)].astype(np.float64)
            q = dense_codes[128 * b:128 * (b + 1), 128 * g:128 * (g + 1)]
            a = np.abs(blk).max()
            if a == 0:
                assert s[b, g] == 0 and not q.any()
                continue
            assert np.abs(q).max() == 448.0  # the block maximum maps to the top code
            t = blk * (448.0 / a)
            assert np.all(np.abs(q - t) <= _ulp_bound(t) * (1 + 1e-6) + 1e-9)


def _loop_product(Wd, Xd, sx, sw):
    """y[m][n] = sum over positions k of x[m][k] w[n][k] sx[m][k // 128]
    sw[n // 128][k // 128], one element at a time."""
    M, K = Xd.shape
    N = Wd.shape[0]
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            t = 0.0
            for k in range(K):
                if Wd[n, k] != 0.0 and Xd[m, k] != 0.0:
                    t += float(Xd[m, k]) * float(Wd[n, k]) * float(sx[m, k // 128]) * float(sw[n // 128, k // 128])
            y[m, n] = t
    return y


def test_block_product_element_loop():
    rng = np.random.default_rng(35)
    M, N, K = 3, 130, 256  # the second weight block holds 2 rows
    W = rng.standard_normal((N, K)).astype(np.float32)
    X = (rng.standard_normal((M, K)) * 4).astype(np.float32)
    vals, meta, sw = oracle.prune24_block(W)
    xq, sx = oracle.quant_group_act(X)
    y = oracle.spgemm_block_f64(vals, meta, xq, K, sx, sw)
    Wd = oracle.decompress24(oracle.e4m3_decode(vals), meta, K)
    Xd = oracle.e4m3_decode(xq)
    ref = _loop_product(Wd, Xd, sx, sw)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_block_product_constant_scales_is_plain_product():
    """Scales constant along K factor out: the product is the plain sparse
    product times s_x[m] s_w[n // 128]."""
    rng = np.random.default_rng(36)
    M, N, K = 6, 200, 640
    W = rng.standard_normal((N, K)).astype(np.float32)
    X = rng.standard_normal((M, K)).astype(np.float32)
    vals, meta, _ = oracle.prune24_block(W)
    xq, _ = oracle.quant_group_act(X)
    Kc = oracle.lifted_k_alloc(K, 2)
    a = rng.uniform(0.5, 2, M).astype(np.float32)
    c = rng.uniform(0.5, 2, 2).astype(np.float32)
    sx = np.repeat(a[:, None], Kc // 128, axis=1)
    sw = np.repeat(c[:, None], Kc // 128, axis=1)
    y = oracle.spgemm_block_f64(vals, meta, xq, Kc, sx, sw)
    acc = oracle.spgemm_acc("W", vals, meta, xq, Kc, "fp8")
    ref = acc * a.astype(np.float64)[:, None] * c.astype(np.float64)[np.arange(N) // 128][None, :]
    assert np.allclose(y, ref, rtol=1e-13, atol=0)


def test_block_output_rounding():
    rng = np.random.default_rng(37)
    W = rng.standard_normal((64, 256)).astype(np.float32)
    X = rng.standard_normal((4, 256)).astype(np.float32)
    vals, meta, sw = oracle.prune24_block(W)
    xq, sx = oracle.quant_group_act(X)
    y64 = oracle.spgemm_block_f64(vals, meta, xq, 256, sx, sw)
    assert np.array_equal(oracle.spgemm_block(vals, meta, xq, 256, sx, sw, "f32"), y64.astype(np.float32))
    yb = oracle.spgemm_block(vals, meta, xq, 256, sx, sw, "bf16")
    assert np.array_equal(yb, oracle.f32_to_bf16_bits_rne(y64.astype(np.float32)))
