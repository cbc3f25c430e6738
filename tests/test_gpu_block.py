"""GPU parity of the block-scaled FP8 path (LLM Compressor guide, W8A8-FP8_BLOCK:
128 x 128 weight blocks, per-token groups of 128; here on 2:4 weights) against
the CPU oracle on seeded inputs: codes, index words (in the tiled layout) and
scales bit-exact; the product within 1e-2 relative Frobenius error of the
oracle's float64 result (the kernel sums each group's products and the scaled
groups in float32, in its own order)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_elementwise, bf16_to_f64, dev_bf16, dev_f32, have_gpu, host, rel_fro
from tiled_ref import tile_ref

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

TOL = 1e-2


@pytest.fixture(scope="module")
def ss():
    import structured_sparse_quantized_amd as m
    return m


def _dev(x, kind):
    """Device copy; rows padded to a multiple of 16 bytes (the ABI's row-stride rule) and sliced back."""
    per = 8 if kind == "bf16" else 4
    K = x.shape[1]
    wide = np.zeros((x.shape[0], -(-K // per) * per), x.dtype)
    wide[:, :K] = x
    return (dev_bf16(wide) if kind == "bf16" else dev_f32(wide))[:, :K]


def _input(seed, rows, K, kind, outliers=0.0):
    X, _, _ = synth.workload(seed, rows, 1, K, x_kind=kind, outlier_frac=outliers)
    return X


QUANT_SHAPES = [(1, 4096), (5, 100), (3, 129), (16, 128), (33, 1000), (257, 4096), (64, 14336), (2, 8)]


@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("shape", QUANT_SHAPES)
def test_quant_group_act(ss, shape, kind):
    M, K = shape
    X = _input(100 + M + K, M, K, kind, outliers=0.01 if K >= 100 else 0.0)
    xq, sx = ss.quant_group_act(_dev(X, kind))
    eq, es = oracle.quant_group_act(X)
    assert np.array_equal(host(xq), eq)
    assert np.array_equal(host(sx), es)


def test_quant_group_act_zero_groups_and_padded_rows(ss):
    import torch
    M, K = 9, 700
    X = _input(7, M, K, "bf16")
    X[2] = 0                      # an all-zero token
    X[5, 128:256] = 0x8000        # a group of -0
    X[6, 640:700] = 0             # the ragged last group all zero
    wide = np.zeros((M, 712), np.uint16)
    wide[:, :K] = X
    xd = dev_bf16(wide)[:, :K]    # rows 1424 bytes apart
    Kc = ss.lifted_k(K, 2)
    outq = torch.full((M, Kc + 16), 0x55, dtype=torch.uint8, device="cuda")
    xq = outq[:, :Kc].view(torch.float8_e4m3fn)
    sx = torch.full((M, Kc // 128), -1.0, device="cuda")
    ss.quant_group_act(xd, out=(xq, sx))
    eq, es = oracle.quant_group_act(X)
    got = host(outq)
    assert np.array_equal(got[:, :Kc], eq) and np.all(got[:, Kc:] == 0x55)
    assert np.array_equal(host(sx), es)
    assert not eq[2].any() and es[5, 1] == 0 and es[6, 5] == 0


PRUNE_SHAPES = [(1, 128), (16, 256), (130, 256), (300, 520), (64, 1000), (257, 4096), (4100, 512), (3, 8)]


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("shape", PRUNE_SHAPES)
def test_prune24_block(ss, shape, kind):
    rows, K = shape
    _, W, _ = synth.workload(200 + rows + K, 1, rows, K)
    W = synth.f32_to_bf16_bits(W) if kind == "bf16" else W
    tv, tm, sw = ss.prune24_block(_dev(W, kind))
    ev, em, es = oracle.prune24_block(W)
    tev, tem = tile_ref(ev, em, 1)
    assert np.array_equal(host(sw), es)
    assert np.array_equal(host(tm), tem)
    assert np.array_equal(host(tv), tev)


def test_prune24_block_zero_block_and_ties(ss):
    rng = np.random.default_rng(3)
    rows, K = 200, 640
    W = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    W[0:128, 128:256] = 0                                   # an all-zero block
    W[150] = 0                                              # an all-zero row
    W[160, :] = np.float32(0.5)                             # ties everywhere: lower positions kept
    W[170, 0:128] = -W[170, 0:128]
    tv, tm, sw = ss.prune24_block(dev_f32(W))
    ev, em, es = oracle.prune24_block(W)
    tev, tem = tile_ref(ev, em, 1)
    assert es[0, 1] == 0
    assert np.array_equal(host(sw), es) and np.array_equal(host(tm), tem) and np.array_equal(host(tv), tev)


def _block_terms(ov, om, oq, osx, osw, Kc):
    """sum over k of |w| |x| times the two scales of k's group: the magnitude sum that bounds the rounding of
    each block-scaled output element (tokens x channels), in float64 from the oracle's decoded codes."""
    A = np.abs(oracle.decompress24(oracle.e4m3_decode(ov), om, Kc))
    B = np.abs(oracle.e4m3_decode(oq))
    N = A.shape[0]
    absterm = np.zeros((B.shape[0], N))
    for g in range(Kc // 128):
        c = slice(128 * g, 128 * (g + 1))
        absterm += (B[:, c] @ A[:, c].T) * osx[:, g][:, None] * osw[np.arange(N) // 128, g][None, :]
    return absterm


def _rel_to_oracle(ss, X, W, y_dtype):
    M, N, K = X.shape[0], W.shape[0], X.shape[1]
    Kc = ss.lifted_k(K, 2)
    tv, tm, sw = ss.prune24_block(dev_f32(W))
    xq, sx = ss.quant_group_act(dev_bf16(X))
    Y = ss.spgemm_tiled_block(M, N, Kc, tv, tm, xq, sx, sw, y_dtype)
    ov, om, osw = oracle.prune24_block(W)
    oq, osx = oracle.quant_group_act(X)
    # the operands the product reads are the oracle's, byte for byte
    assert np.array_equal(host(xq), oq) and np.array_equal(host(sx), osx) and np.array_equal(host(sw), osw)
    exp = oracle.spgemm_block_f64(ov, om, oq, Kc, osx, osw)
    got = host(Y)
    got = bf16_to_f64(got) if y_dtype == "bf16" else got.astype(np.float64)
    # element by element: each group's 128-position FP8 dot product runs from a zero accumulator, and on
    # inputs with outlier channels its error reached 5.8e-5 sum|terms| (1 of 16384 elements over 4e-5 at
    # 64 x 256 x 512, 3 of 1048576 at 2048 x 512 x 1024, with float32 output), so c = 1e-4 here; a wrong
    # group, block or scale moves whole terms, orders of magnitude more
    assert_elementwise(got, exp, _block_terms(ov, om, oq, osx, osw, Kc), out=y_dtype, c=1e-4)
    return rel_fro(got, exp), got, exp


GEMM_SHAPES = [(1, 128, 256), (64, 256, 512), (100, 300, 520), (300, 520, 1000), (513, 1000, 2048),
               (2048, 512, 1024), (17, 4096, 3584), (256, 128, 14336)]


@pytest.mark.parametrize("y_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_spgemm_tiled_block(ss, shape, y_dtype):
    M, N, K = shape
    X, W, _ = synth.workload(300 + M + N + K, M, N, K, outlier_frac=0.01)
    err, got, exp = _rel_to_oracle(ss, X, W, y_dtype)
    assert err <= TOL, err
    # float32 sums of exact E4M3 products (up to 64 terms a group, then the scaled groups): far inside the
    # bound; a scale applied to the wrong group or block would be off by O(1) (bf16 output adds its rounding)
    assert err <= (5e-3 if y_dtype == "bf16" else 1e-4), err


def test_spgemm_tiled_block_group_scales_are_per_step(ss):
    """Groups of X and blocks of W scaled by independent powers of two (2^-8 .. 2^8): a
    scale applied to the wrong group or block would be off by large factors."""
    rng = np.random.default_rng(11)
    M, N, K = 300, 384, 1536
    Xf = rng.standard_normal((M, K)).astype(np.float32)
    Xf *= (2.0 ** rng.integers(-8, 9, (M, K // 128))).repeat(128, axis=1).astype(np.float32)
    X = synth.f32_to_bf16_bits(Xf)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W *= (2.0 ** rng.integers(-8, 9, (3, K // 128))).repeat(128, axis=0).repeat(128, axis=1).astype(np.float32)
    err, got, exp = _rel_to_oracle(ss, X, W, "f32")
    assert err <= 1e-4, err
    # element by element, against a summation bound |error| <= c * sum of |terms|: the matrix core's FP8
    # dot products keep about 16 bits relative to the sum of magnitudes (one 128-position group through
    # the per-channel product measures up to 1.6e-5), so c = 4e-5; a scale applied to the wrong group or
    # block moves whole terms and fails by orders of magnitude
    Kc = K
    ov, om, osw = oracle.prune24_block(W)
    oq, osx = oracle.quant_group_act(X)
    absterm = _block_terms(ov, om, oq, osx, osw, Kc)
    assert np.all(np.abs(got - exp) <= 4e-5 * absterm + 1e-30)


def test_spgemm_tiled_block_full_size_sampled(ss):
    """The 6:8-bench-sized layer in block-scaled 2:4 FP8 (2048 tokens, 4096 x 4096 weights), launched as
    the benchmark launches it; the oracle recomputes 96 sampled tokens over every channel."""
    M, N, K = 2048, 4096, 4096
    X, W, _ = synth.workload(0, M, N, K, outlier_frac=0.01)
    Kc = ss.lifted_k(K, 2)
    tv, tm, sw = ss.prune24_block(dev_f32(W))
    xq, sx = ss.quant_group_act(dev_bf16(X))
    Y = ss.spgemm_tiled_block(M, N, Kc, tv, tm, xq, sx, sw, "bf16")
    ov, om, osw = oracle.prune24_block(W)
    tev, tem = tile_ref(ov, om, 1)
    assert np.array_equal(host(sw), osw) and np.array_equal(host(tm), tem) and np.array_equal(host(tv), tev)
    pick = np.sort(np.random.default_rng(5).choice(M, 96, replace=False))
    oq, osx = oracle.quant_group_act(X[pick])
    assert np.array_equal(host(xq)[pick], oq) and np.array_equal(host(sx)[pick], osx)
    exp = oracle.spgemm_block_f64(ov, om, oq, Kc, osx, osw)
    got = bf16_to_f64(host(Y)[pick])
    assert rel_fro(got, exp) <= 5e-3
    assert_elementwise(got, exp, _block_terms(ov, om, oq, osx, osw, Kc), out="bf16")
