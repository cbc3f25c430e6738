"""GPU parity of every C-ABI call against the CPU oracle, on seeded inputs.

Small shapes span several tiles and ragged tails; INT8 results and all
codes, masks, metadata and scales must be bit-exact, FP8/bf16 products are
held to a relative Frobenius error of 1e-2 against the oracle's same-format
result and, element by element, to the matrix core's summation precision
(4e-5 sum|terms| plus one output rounding).
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_product, dev_bf16, dev_codes, dev_f32, dev_u8, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

TOL = 1e-2


@pytest.fixture(scope="module")
def ss():
    import structured_sparse_quantized_amd as m
    return m


def _x(seed, M, K, kind, zero_rows=(), ties=False):
    rng = np.random.default_rng(seed)
    x = synth.normal_f32(rng, (M, K))
    if ties:
        x[:, ::3] = np.round(x[:, ::3] * 2) / 2
    for r in zero_rows:
        if r < M:
            x[r] = 0
    return synth.f32_to_bf16_bits(x) if kind == "bf16" else x


def _dev(x):
    return dev_bf16(x) if x.dtype == np.uint16 else dev_f32(x)


# ---------------------------------------------------------------- quant + lift
QL_SHAPES = [(1, 8), (3, 40), (7, 520), (64, 512), (33, 3584), (5, 4096), (130, 1024), (2, 30000)]


@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("q", ["i8", "fp8"])
@pytest.mark.parametrize("n", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("shape", QL_SHAPES)
def test_quant_lift_act(ss, kind, q, n, shape):
    M, K = shape
    if kind == "f32" and K == 30000:
        K = 20000
    x = _x(100 + M + K + n, M, K, kind, zero_rows=(1,))
    xq, sx = ss.quant_lift_act(_dev(x), n, q)
    exp_q, exp_s = oracle.quant_lift_act(x, n, q)
    assert np.array_equal(host(sx), exp_s)
    got = host(xq)
    assert got.shape == exp_q.shape
    assert np.array_equal(got.view(np.uint8), exp_q.view(np.uint8))


def test_quant_lift_padded_leading_dim(ss):
    x = _x(5, 9, 200, "bf16")
    big = np.zeros((9, 264), np.uint16)
    big[:, :200] = x
    xd = dev_bf16(big)[:, :200]
    xq, sx = ss.quant_lift_act(xd, 4, "i8")
    exp_q, exp_s = oracle.quant_lift_act(x, 4, "i8")
    assert np.array_equal(host(xq), exp_q) and np.array_equal(host(sx), exp_s)


@pytest.mark.parametrize("q", ["i8", "fp8"])
@pytest.mark.parametrize("n", [2, 3, 4, 5])
@pytest.mark.parametrize("K", [203, 1002, 4094])
def test_quant_lift_ragged_k_padded_rows(ss, K, n, q):
    """bf16 rows whose length is not a multiple of 8 (so the last 2n-group is partial and, at 6:8, the
    groups do not line up with 16-byte vectors): rows padded to a 16-byte stride."""
    x = _x(K + n, 11, K, "bf16")
    ld = -(-K // 8) * 8 + 8
    big = np.zeros((11, ld), np.uint16)
    big[:, :K] = x
    xq, sx = ss.quant_lift_act(dev_bf16(big)[:, :K], n, q)
    exp_q, exp_s = oracle.quant_lift_act(x, n, q)
    assert np.array_equal(host(sx), exp_s)
    assert np.array_equal(host(xq).view(np.uint8), exp_q.view(np.uint8))


# ---------------------------------------------------------------- weight prep
W_SHAPES = [(1, 8), (5, 24), (130, 520), (256, 512), (64, 4096), (3, 14336)]


def _w(seed, rows, K, kind, ties=False):
    rng = np.random.default_rng(seed)
    w = synth.normal_f32(rng, (rows, K), 0.02)
    if ties:
        w[:, ::2] = np.round(w[:, ::2] * 100) / 100
        w[:, 1::4] = -w[:, 0::4]
    if rows > 2:
        w[2] = 0
        w[1, : K // 2] = 0
    return synth.f32_to_bf16_bits(w) if kind == "bf16" else w


def _cmp_sparse(got, exp):
    gv, gm, gs = got
    ev, em, es = exp
    assert np.array_equal(host(gm), em)
    assert np.array_equal(host(gv).view(np.uint8), np.ascontiguousarray(ev).view(np.uint8))
    if es is None:
        assert gs is None
    else:
        assert np.array_equal(host(gs), es)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("out", ["i8", "fp8", "bf16"])
@pytest.mark.parametrize("shape", W_SHAPES)
@pytest.mark.parametrize("ties", [False, True])
def test_prune24(ss, kind, out, shape, ties):
    rows, K = shape
    w = _w(7 + rows + K, rows, K, kind, ties)
    _cmp_sparse(ss.prune24(_dev(w), out), oracle.prune24(w, out))


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("out", ["i8", "fp8", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("shape", [(1, 8), (5, 40), (130, 520), (64, 3584), (3, 18944), (2, 60000)])
def test_slide_decompose(ss, kind, out, n, shape):
    rows, K = shape
    w = _w(11 + rows + K + n, rows, K, kind, ties=(n == 4))
    _cmp_sparse(ss.slide_decompose(_dev(w), n, out), oracle.slide_decompose(w, n, out))


@pytest.mark.parametrize("out", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("shape", [(1, 8), (7, 24), (130, 520), (33, 4096), (2, 18944), (3, 100000)])
def test_prune24_act(ss, out, shape):
    M, K = shape
    x = _x(21 + M + K, M, K, "bf16", zero_rows=(1,), ties=True)
    _cmp_sparse(ss.prune24_act(dev_bf16(x), out), oracle.prune24_act(x, out))


# ---------------------------------------------------------------- sparse GEMM
GEMM_SHAPES = [(1, 1, 8), (64, 256, 512), (200, 130, 768), (129, 257, 1024), (17, 300, 40)]


def _gemm_case(seed, M, N, K, n, ab, side):
    """Operands built by the oracle (no HIP step), then fed to the GPU product."""
    X, W, _ = synth.workload(seed, M, N, K, x_kind="bf16")
    if side == "W":
        if n == 2:
            vals, meta, sw = oracle.prune24(W, ab)
        else:
            vals, meta, sw = oracle.slide_decompose(W, n, ab)
        if ab == "bf16":
            dense = oracle.lift(X, n)
            Kc = oracle.lifted_k_alloc(K, n)
            dpad = np.zeros((M, Kc), np.uint16)
            dpad[:, : dense.shape[1]] = dense
            dense, sx, sw = dpad, None, None
        else:
            dense, sx = oracle.quant_lift_act(X, n, ab)
    else:
        if ab == "bf16":
            vals, meta, sx = oracle.prune24_act(X, "bf16")
            Kc = oracle.lifted_k_alloc(K, 2)
            dense = np.zeros((N, Kc), np.uint16)
            dense[:, :K] = synth.f32_to_bf16_bits(W)
            sw = None
        else:
            vals, meta, sx = oracle.prune24_act(X, ab)
            dense, sw = oracle.quant_lift_act(W, 2, ab)
    Kc = meta.shape[1] * 8
    return vals, meta, dense, sx, sw, Kc


@pytest.mark.parametrize("side", ["W", "X"])
@pytest.mark.parametrize("ab", ["i8", "fp8", "bf16"])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_spgemm_against_oracle_operands(ss, side, ab, shape):
    M, N, K = shape
    n = 4 if (side == "W" and K % 8 == 0 and K > 8) else 2
    vals, meta, dense, sx, sw, Kc = _gemm_case(31 + M + N, M, N, K, n, ab, side)
    s = ss.SS_SPARSE_W if side == "W" else ss.SS_SPARSE_X
    args = (dev_codes(vals, ab), dev_u8(meta), dev_codes(dense, ab),
            None if sx is None else dev_f32(sx), None if sw is None else dev_f32(sw))
    for y in (["i32", "f32", "bf16"] if ab == "i8" else ["f32", "bf16"]):
        Y = host(ss.spgemm(s, M, N, Kc, *args, y_dtype=y))
        exp = oracle.spgemm(side, vals, meta, dense, Kc, ab, sx, sw, y)
        assert_product(Y, exp, side, vals, meta, dense, Kc, ab, sx, sw, y, TOL)


@pytest.mark.parametrize("n", [2, 3, 4, 5])
@pytest.mark.parametrize("q", ["i8", "fp8"])
def test_weight_sparse_path_end_to_end(ss, n, q):
    """GPU prune/decompose + GPU quant-lift + GPU product vs the oracle path."""
    M, N, K = 150, 260, 1000
    X, W, _ = synth.workload(41 + n, M, N, K, x_kind="bf16", outlier_frac=0.01)
    wv, wm, sw = (ss.prune24(dev_f32(W), q) if n == 2 else ss.slide_decompose(dev_f32(W), n, q))
    xq, sx = ss.quant_lift_act(dev_bf16(X), n, q)
    Kc = ss.lifted_k(K, n)
    Y = host(ss.spgemm(ss.SS_SPARSE_W, M, N, Kc, wv, wm, xq, sx, sw, "bf16"))
    ov, om, osw = oracle.slide_decompose(W, n, q) if n > 2 else oracle.prune24(W, q)
    oxq, osx = oracle.quant_lift_act(X, n, q)
    exp = oracle.spgemm("W", ov, om, oxq, Kc, q, osx, osw, "bf16")
    assert_product(Y, exp, "W", ov, om, oxq, Kc, q, osx, osw, "bf16", TOL)


@pytest.mark.parametrize("out", ["bf16", "fp8"])
def test_activation_sparse_path_end_to_end(ss, out):
    M, N, K = 300, 200, 512
    X, W, _ = synth.workload(51, M, N, K, x_kind="bf16")
    xv, xm, sx = ss.prune24_act(dev_bf16(X), out)
    if out == "bf16":
        wd, sw = dev_bf16(synth.f32_to_bf16_bits(W)), None
        ow, osw = synth.f32_to_bf16_bits(W), None
    else:
        wd, sw = ss.quant_lift_act(dev_f32(W), 2, "fp8")
        ow, osw = oracle.quant_lift_act(W, 2, "fp8")
    Y = host(ss.spgemm(ss.SS_SPARSE_X, M, N, K, xv, xm, wd, sx, sw, "f32"))
    ov, om, osx = oracle.prune24_act(X, out)
    exp = oracle.spgemm("X", ov, om, ow, K, out, osx, osw, "f32")
    assert_product(Y, exp, "X", ov, om, ow, K, out, osx, osw, "f32", TOL)
