"""GPU parity at the full workload sizes, in the launch configuration the
benchmark uses. Preparation outputs (values, metadata, scales, lifted codes)
are compared in full; products are compared on sampled token rows that the
oracle computes exactly (INT8 bit-exact, FP8/bf16 within 1e-2 relative
Frobenius error and element by element within 4e-5 sum|terms| plus one output
rounding)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_product, dev_bf16, dev_f32, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ss():
    import structured_sparse_quantized_amd as m
    return m


def _rows(M, k=48, seed=0):
    rng = np.random.default_rng(seed)
    r = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(k, M), replace=False)]))
    return r


def _check_prep(got, exp):
    for g, e in zip(got, exp):
        if e is None:
            assert g is None
            continue
        assert np.array_equal(host(g).view(np.uint8), np.ascontiguousarray(e).view(np.uint8))


def test_small_24_int8_exact(ss):
    """X 64x512 fp32, W 256x512 fp32 2:4, INT8, int32 accumulators and fp32 out."""
    c = synth.CFG_SMALL_24_INT8
    X, W, _ = synth.workload(c["seed"], c["M"], c["N"], c["K"], x_kind="f32")
    w = ss.prune24(dev_f32(W), "i8")
    x = ss.quant_lift_act(dev_f32(X), 2, "i8")
    ow, ox = oracle.prune24(W, "i8"), oracle.quant_lift_act(X, 2, "i8")
    _check_prep(w, ow)
    _check_prep(x, ox)
    tv, tm = ss.pack_sparse(w[0], w[1])
    for y in ("i32", "f32"):
        exp = oracle.spgemm("W", ow[0], ow[1], ox[0], c["K"], "i8", ox[1], ow[2], y)
        Y = host(ss.spgemm(ss.SS_SPARSE_W, c["M"], c["N"], c["K"], w[0], w[1], x[0], x[1], w[2], y))
        assert np.array_equal(Y, exp)
        Yt = host(ss.spgemm_tiled(ss.SS_SPARSE_W, c["M"], c["N"], c["K"], tv, tm, x[0], x[1], w[2], y))
        assert np.array_equal(Yt, exp)


def test_68_int8_full_size(ss):
    """W 4096x4096 6:8 -> K'=6144, X 2048x4096 bf16 with 1% outlier columns."""
    c = synth.CFG_68_INT8
    M, N, K, n = c["M"], c["N"], c["K"], c["n"]
    X, W, _ = synth.workload(0, M, N, K, x_kind="bf16", outlier_frac=0.01)
    w = ss.slide_decompose(dev_f32(W), n, "i8")
    x = ss.quant_lift_act(dev_bf16(X), n, "i8")
    Kc = ss.lifted_k(K, n)
    assert Kc == 6144
    Y = host(ss.spgemm(ss.SS_SPARSE_W, M, N, Kc, w[0], w[1], x[0], x[1], w[2], "bf16"))
    ow = oracle.slide_decompose(W, n, "i8")
    ox = oracle.quant_lift_act(X, n, "i8")
    _check_prep(w, ow)
    _check_prep(x, ox)
    r = _rows(M)
    exp = oracle.spgemm("W", ow[0], ow[1], ox[0][r], Kc, "i8", ox[1][r], ow[2], "bf16")
    assert np.array_equal(Y[r], exp)
    # the tiled product, as the benchmark launches it: same bytes everywhere
    tv, tm = ss.pack_sparse(w[0], w[1])
    Yt = host(ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, x[0], x[1], w[2], "bf16"))
    assert np.array_equal(Yt[r], exp)
    assert np.array_equal(Yt, Y)


@pytest.mark.parametrize("name", ["qkv", "down"])
def test_llama_fp8_24_sampled(ss, name):
    K, N = synth.LLAMA31_8B_LINEARS[name]
    M = 2048
    X, W, _ = synth.workload(3, M, N, K, x_kind="bf16")
    w = ss.prune24(dev_f32(W), "fp8")
    x = ss.quant_lift_act(dev_bf16(X), 2, "fp8")
    Y = host(ss.spgemm(ss.SS_SPARSE_W, M, N, K, w[0], w[1], x[0], x[1], w[2], "bf16"))
    ow = oracle.prune24(W, "fp8")
    _check_prep(w, ow)
    r = _rows(M, 24)
    ox = oracle.quant_lift_act(X[r], 2, "fp8")
    assert np.array_equal(host(x[0])[r].view(np.uint8), ox[0]) and np.array_equal(host(x[1])[r], ox[1])
    exp = oracle.spgemm("W", ow[0], ow[1], ox[0], K, "fp8", ox[1], ow[2], "bf16")
    assert_product(Y[r], exp, "W", ow[0], ow[1], ox[0], K, "fp8", ox[1], ow[2], "bf16")
    tv, tm = ss.pack_sparse(w[0], w[1])
    Yt = host(ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, K, tv, tm, x[0], x[1], w[2], "bf16"))
    assert_product(Yt[r], exp, "W", ow[0], ow[1], ox[0], K, "fp8", ox[1], ow[2], "bf16")


@pytest.mark.parametrize("out", ["bf16", "fp8"])
def test_sparse_activation_full_size(ss, out):
    """X 8192x4096 bf16 pruned 2:4 online, times dense W 4096x4096."""
    M, N, K = 8192, 4096, 4096
    X, W, _ = synth.workload(4, M, N, K, x_kind="bf16")
    xs = ss.prune24_act(dev_bf16(X), out)
    oxs = oracle.prune24_act(X, out)
    _check_prep(xs, oxs)
    if out == "bf16":
        wd, sw = dev_bf16(synth.f32_to_bf16_bits(W)), None
        ow, osw = synth.f32_to_bf16_bits(W), None
    else:
        wd, sw = ss.quant_lift_act(dev_f32(W), 2, "fp8")
        ow, osw = oracle.quant_lift_act(W, 2, "fp8")
        assert np.array_equal(host(wd).view(np.uint8), ow) and np.array_equal(host(sw), osw)
    Y = host(ss.spgemm(ss.SS_SPARSE_X, M, N, K, xs[0], xs[1], wd, xs[2], sw, "bf16"))
    r = _rows(M, 24)
    osx_r = None if oxs[2] is None else oxs[2][r]
    exp = oracle.spgemm("X", oxs[0][r], oxs[1][r], ow, K, out, osx_r, osw, "bf16")
    assert_product(Y[r], exp, "X", oxs[0][r], oxs[1][r], ow, K, out, osx_r, osw, "bf16")
    tv, tm = ss.pack_sparse(xs[0], xs[1])
    Yt = host(ss.spgemm_tiled(ss.SS_SPARSE_X, M, N, K, tv, tm, wd, xs[2], sw, "bf16"))
    assert_product(Yt[r], exp, "X", oxs[0][r], oxs[1][r], ow, K, out, osx_r, osw, "bf16")


@pytest.mark.parametrize("n", [3, 5])
@pytest.mark.parametrize("M", [1, 16, 64, 4096])
def test_qwen_qkv_slide_int8(ss, n, M):
    K, N = synth.QWEN25_7B_LINEARS["qkv"]
    X, W, _ = synth.workload(5, M, N, K, x_kind="bf16")
    w = ss.slide_decompose(dev_f32(W), n, "i8")
    x = ss.quant_lift_act(dev_bf16(X), n, "i8")
    Kc = ss.lifted_k(K, n)
    Y = host(ss.spgemm(ss.SS_SPARSE_W, M, N, Kc, w[0], w[1], x[0], x[1], w[2], "bf16"))
    ow = oracle.slide_decompose(W, n, "i8")
    _check_prep(w, ow)
    r = _rows(M, 32)
    ox = oracle.quant_lift_act(X[r], n, "i8")
    assert np.array_equal(host(x[0])[r], ox[0]) and np.array_equal(host(x[1])[r], ox[1])
    exp = oracle.spgemm("W", ow[0], ow[1], ox[0], Kc, "i8", ox[1], ow[2], "bf16")
    assert np.array_equal(Y[r], exp)
    tv, tm = ss.pack_sparse(w[0], w[1])
    Yt = host(ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, x[0], x[1], w[2], "bf16"))
    assert np.array_equal(Yt[r], exp)


def test_qwen_down_810_int8_decode(ss):
    """K=18944 (not a multiple of 10): padding groups and K' rounded to 30464."""
    K, N = synth.QWEN25_7B_LINEARS["down"]
    M, n = 16, 5
    X, W, _ = synth.workload(6, M, N, K, x_kind="bf16")
    w = ss.slide_decompose(dev_f32(W), n, "i8")
    x = ss.quant_lift_act(dev_bf16(X), n, "i8")
    Kc = ss.lifted_k(K, n)
    assert Kc == 30464
    Y = host(ss.spgemm(ss.SS_SPARSE_W, M, N, Kc, w[0], w[1], x[0], x[1], w[2], "bf16"))
    ow, ox = oracle.slide_decompose(W, n, "i8"), oracle.quant_lift_act(X, n, "i8")
    _check_prep(w, ow)
    _check_prep(x, ox)
    exp = oracle.spgemm("W", ow[0], ow[1], ox[0], Kc, "i8", ox[1], ow[2], "bf16")
    assert np.array_equal(Y, exp)
    tv, tm = ss.pack_sparse(w[0], w[1])
    Yt = host(ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, x[0], x[1], w[2], "bf16"))
    assert np.array_equal(Yt, exp)
