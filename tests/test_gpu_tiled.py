"""GPU parity of the tiled sparse operand (ss_pack_sparse) and of the product
that reads it (ss_spgemm_tiled), against the CPU oracle on seeded inputs.

The expected tiled bytes are a plain re-indexing of the row-major compressed
operand, written here from the layout description in include/ss.h. Products
are compared with the oracle like ss_spgemm: INT8 bit-exact, FP8 within 1e-2
relative Frobenius error."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_product, dev_bf16, dev_codes, dev_f32, dev_u8, have_gpu, host
from tiled_ref import tile_ref

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

TOL = 1e-2


@pytest.fixture(scope="module")
def ss():
    import structured_sparse_quantized_amd as m
    return m


PACK_SHAPES = [(1, 256), (15, 256), (16, 512), (17, 768), (130, 1024), (300, 6144), (33, 1280)]


@pytest.mark.parametrize("q", ["i8", "fp8", "bf16"])
@pytest.mark.parametrize("shape", PACK_SHAPES)
def test_pack_sparse(ss, q, shape):
    rows, Kc = shape
    es = 2 if q == "bf16" else 1
    rng = np.random.default_rng(rows + Kc)
    vals = rng.integers(0, 256, (rows, Kc // 2 * es), dtype=np.uint8)
    meta = rng.integers(0, 256, (rows, Kc // 8), dtype=np.uint8)
    vd = dev_u8(vals).view(torch_dtype(q))
    tv, tm = ss.pack_sparse(vd, dev_u8(meta))
    ev, em = tile_ref(vals, meta, es)
    assert np.array_equal(host(tv), ev)
    assert np.array_equal(host(tm), em)


def torch_dtype(q):
    import torch
    return {"i8": torch.int8, "fp8": torch.float8_e4m3fn, "bf16": torch.bfloat16}[q]


def test_pack_sparse_padded_leading_dims(ss):
    import torch
    rows, Kc = 40, 512
    rng = np.random.default_rng(3)
    vals = rng.integers(0, 256, (rows, Kc // 2 + 32), dtype=np.uint8)
    meta = rng.integers(0, 256, (rows, Kc // 8 + 16), dtype=np.uint8)
    vd = dev_u8(vals).view(torch.int8)[:, : Kc // 2]
    md = dev_u8(meta)[:, : Kc // 8]
    tv, tm = ss.pack_sparse(vd, md)
    ev, em = tile_ref(vals[:, : Kc // 2], meta[:, : Kc // 8])
    assert np.array_equal(host(tv), ev) and np.array_equal(host(tm), em)


GEMM_SHAPES = [(1, 1, 8), (64, 256, 512), (200, 130, 768), (129, 257, 1024), (17, 300, 40), (300, 520, 2000)]


def _gemm_case(seed, M, N, K, n, ab, side):
    """Operands built by the oracle (no HIP step). bf16: unscaled bf16 operands (scales None)."""
    X, W, _ = synth.workload(seed, M, N, K, x_kind="bf16")
    if side == "W":
        vals, meta, sw = oracle.prune24(W, ab) if n == 2 else oracle.slide_decompose(W, n, ab)
        if ab == "bf16":
            Kc = oracle.lifted_k_alloc(K, n)
            lifted = oracle.lift(X, n)
            dense = np.zeros((M, Kc), np.uint16)
            dense[:, : lifted.shape[1]] = lifted
            sx, sw = None, None
        else:
            dense, sx = oracle.quant_lift_act(X, n, ab)
    else:
        vals, meta, sx = oracle.prune24_act(X, ab)
        if ab == "bf16":
            Kc = oracle.lifted_k_alloc(K, 2)
            dense = np.zeros((N, Kc), np.uint16)
            dense[:, :K] = synth.f32_to_bf16_bits(W)
            sw = None
        else:
            dense, sw = oracle.quant_lift_act(W, 2, ab)
    Kc = meta.shape[1] * 8
    return vals, meta, dense, sx, sw, Kc


def _scales(sx, sw):
    return (None if sx is None else dev_f32(sx)), (None if sw is None else dev_f32(sw))


@pytest.mark.parametrize("side", ["W", "X"])
@pytest.mark.parametrize("ab", ["i8", "fp8", "bf16"])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_spgemm_tiled_against_oracle_operands(ss, side, ab, shape):
    M, N, K = shape
    n = 4 if (side == "W" and K % 8 == 0 and K > 8) else 2
    vals, meta, dense, sx, sw, Kc = _gemm_case(77 + M + N, M, N, K, n, ab, side)
    s = ss.SS_SPARSE_W if side == "W" else ss.SS_SPARSE_X
    tv, tm = ss.pack_sparse(dev_codes(vals, ab), dev_u8(meta))
    d = dev_codes(dense, ab)
    dsx, dsw = _scales(sx, sw)
    for y in (["i32", "f32", "bf16"] if ab == "i8" else ["f32", "bf16"]):
        Y = host(ss.spgemm_tiled(s, M, N, Kc, tv, tm, d, dsx, dsw, y_dtype=y))
        exp = oracle.spgemm(side, vals, meta, dense, Kc, ab, sx, sw, y)
        assert_product(Y, exp, side, vals, meta, dense, Kc, ab, sx, sw, y, TOL)


def test_spgemm_tiled_output_leading_dim(ss):
    """Y rows with a leading dimension not a multiple of 4 take the scalar stores."""
    import torch
    M, N, K = 70, 150, 512
    vals, meta, dense, sx, sw, Kc = _gemm_case(5, M, N, K, 2, "i8", "W")
    tv, tm = ss.pack_sparse(dev_codes(vals, "i8"), dev_u8(meta))
    big = torch.zeros((M, N + 3), dtype=torch.int32, device="cuda")
    out = big[:, :N]
    ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, dev_codes(dense, "i8"), dev_f32(sx), dev_f32(sw), "i32",
                    out=out)
    got = host(big)
    assert np.array_equal(got[:, :N], oracle.spgemm("W", vals, meta, dense, Kc, "i8", sx, sw, "i32"))
    assert not got[:, N:].any()


@pytest.mark.parametrize("n", [2, 3, 4, 5])
@pytest.mark.parametrize("q", ["i8", "fp8"])
def test_weight_sparse_path_tiled(ss, n, q):
    """GPU prune/decompose + pack + GPU quant-lift + tiled product vs the oracle path."""
    M, N, K = 150, 260, 1000
    X, W, _ = synth.workload(61 + n, M, N, K, x_kind="bf16", outlier_frac=0.01)
    wv, wm, sw = (ss.prune24(dev_f32(W), q) if n == 2 else ss.slide_decompose(dev_f32(W), n, q))
    tv, tm = ss.pack_sparse(wv, wm)
    xq, sx = ss.quant_lift_act(dev_bf16(X), n, q)
    Kc = ss.lifted_k(K, n)
    Y = host(ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, xq, sx, sw, "bf16"))
    ov, om, osw = oracle.slide_decompose(W, n, q) if n > 2 else oracle.prune24(W, q)
    oxq, osx = oracle.quant_lift_act(X, n, q)
    exp = oracle.spgemm("W", ov, om, oxq, Kc, q, osx, osw, "bf16")
    assert_product(Y, exp, "W", ov, om, oxq, Kc, q, osx, osw, "bf16", TOL)


@pytest.mark.parametrize("out", ["i8", "fp8"])
def test_activation_sparse_path_tiled(ss, out):
    M, N, K = 300, 200, 512
    X, W, _ = synth.workload(71, M, N, K, x_kind="bf16")
    xv, xm, sx = ss.prune24_act(dev_bf16(X), out)
    tv, tm = ss.pack_sparse(xv, xm)
    wd, sw = ss.quant_lift_act(dev_f32(W), 2, out)
    Y = host(ss.spgemm_tiled(ss.SS_SPARSE_X, M, N, K, tv, tm, wd, sx, sw, "f32"))
    ov, om, osx = oracle.prune24_act(X, out)
    ow, osw = oracle.quant_lift_act(W, 2, out)
    exp = oracle.spgemm("X", ov, om, ow, K, out, osx, osw, "f32")
    assert_product(Y, exp, "X", ov, om, ow, K, out, osx, osw, "f32", TOL)


def test_repeated_calls_and_streams(ss):
    """Back-to-back calls on a side stream give identical results."""
    import torch
    M, N, K = 256, 512, 2048
    vals, meta, dense, sx, sw, Kc = _gemm_case(9, M, N, K, 2, "i8", "W")
    tv, tm = ss.pack_sparse(dev_codes(vals, "i8"), dev_u8(meta))
    d, dsx, dsw = dev_codes(dense, "i8"), dev_f32(sx), dev_f32(sw)
    exp = oracle.spgemm("W", vals, meta, dense, Kc, "i8", sx, sw, "i32")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        outs = [ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, d, dsx, dsw, "i32") for _ in range(4)]
    st.synchronize()
    for o in outs:
        assert np.array_equal(host(o), exp)


# Few tokens (side W): the product runs the row-block decode kernel (16 rows per workgroup, K split across
# waves, partial sums reduced in LDS); these cases cover its column-tile counts (<= 16, 32, 64 tokens), ragged
# row counts, K short enough that some waves get no work, and long K.
DECODE_SHAPES = [(1, 1000, 512), (5, 1000, 600), (8, 260, 2048), (9, 300, 1000), (16, 512, 4096), (17, 130, 512),
                 (32, 700, 3000), (33, 520, 768), (64, 1000, 6000), (64, 4608, 3584), (40, 300, 18944),
                 (64, 3584, 18944)]


@pytest.mark.parametrize("path", ["auto", "no_workspace"])
@pytest.mark.parametrize("ab", ["i8", "fp8", "bf16"])
@pytest.mark.parametrize("shape", DECODE_SHAPES)
def test_spgemm_tiled_decode_tokens(ss, ab, shape, path):
    """Few-token weight-sparse products: the split-K path (17..64 tokens, workspace from torch) and the
    row-block kernel (no workspace), against the oracle."""
    M, N, K = shape
    n = 3 if K % 6 == 0 else 2
    vals, meta, dense, sx, sw, Kc = _gemm_case(101 + M + N, M, N, K, n, ab, "W")
    tv, tm = ss.pack_sparse(dev_codes(vals, ab), dev_u8(meta))
    d = dev_codes(dense, ab)
    dsx, dsw = _scales(sx, sw)
    for y in (["i32", "bf16"] if ab == "i8" else ["f32", "bf16"]):
        Y = host(ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, d, dsx, dsw, y_dtype=y,
                                 workspace=None if path == "auto" else False))
        exp = oracle.spgemm("W", vals, meta, dense, Kc, ab, sx, sw, y)
        assert_product(Y, exp, "W", vals, meta, dense, Kc, ab, sx, sw, y, TOL)


def test_activation_sparse_path_tiled_bf16(ss):
    """bf16 activations pruned 2:4 online, times bf16 weights, on the tiled product."""
    M, N, K = 300, 200, 512
    X, W, _ = synth.workload(73, M, N, K, x_kind="bf16")
    xv, xm, _ = ss.prune24_act(dev_bf16(X), "bf16")
    tv, tm = ss.pack_sparse(xv, xm)
    wb = synth.f32_to_bf16_bits(W)
    Y = host(ss.spgemm_tiled(ss.SS_SPARSE_X, M, N, K, tv, tm, dev_bf16(wb), None, None, "f32"))
    ov, om, _ = oracle.prune24_act(X, "bf16")
    exp = oracle.spgemm("X", ov, om, wb, K, "bf16", None, None, "f32")
    assert_product(Y, exp, "X", ov, om, wb, K, "bf16", None, None, "f32", TOL)


# K = 4096 / 6000 / 18944 hold one / two / no groups per wave in registers (8-bit codes); K = 100 and 1004
# end inside a 16-byte chunk of the row, K = 520 and 1000 inside a 16-element unit
PRUNE_TILED_SHAPES = [(1, 8), (7, 24), (5, 100), (16, 512), (33, 4096), (130, 520), (2, 18944), (300, 1000),
                      (9, 1004), (20, 6000)]


@pytest.mark.parametrize("out", ["i8", "fp8", "bf16"])
@pytest.mark.parametrize("shape", PRUNE_TILED_SHAPES)
def test_prune24_act_tiled(ss, out, shape):
    """One-pass prune into the tiled layout: the oracle's compressed operand re-indexed, and the same bytes as
    ss_prune24_act followed by ss_pack_sparse."""
    M, K = shape
    rng = np.random.default_rng(M * 7 + K)
    X = synth.f32_to_bf16_bits(synth.normal_f32(rng, (M, K)))
    if M > 3:
        X[3] = 0  # an all-zero token
    # rows start 16-byte aligned: ragged K lives in a wider buffer, whose columns past K hold 1024.0 (read
    # into the last chunk's registers, they must not reach the absmax or the selection)
    ldk = -(-K // 8) * 8
    xp = np.full((M, ldk), 0x4480, np.uint16)
    xp[:, :K] = X
    xd = dev_bf16(xp)[:, :K]
    tv, tm, sx = ss.prune24_act_tiled(xd, out)
    ov, om, osx = oracle.prune24_act(X, out)
    es = 2 if out == "bf16" else 1
    ev, em = tile_ref(np.ascontiguousarray(ov).view(np.uint8).reshape(M, -1), om, es)
    assert np.array_equal(host(tv), ev)
    assert np.array_equal(host(tm), em)
    if out == "bf16":
        assert sx is None
    else:
        assert np.array_equal(host(sx), osx)
    pv, pm, psx = ss.prune24_act(xd, out)
    rv, rm = ss.pack_sparse(pv, pm)
    assert np.array_equal(host(rv), host(tv)) and np.array_equal(host(rm), host(tm))


@pytest.mark.parametrize("out", ["fp8", "bf16"])
def test_activation_sparse_layer_one_pass(ss, out):
    """Online prune into the tiled layout + tiled product, against the oracle layer."""
    M, N, K = 260, 300, 1024
    X, W, _ = synth.workload(81, M, N, K, x_kind="bf16")
    tv, tm, sx = ss.prune24_act_tiled(dev_bf16(X), out)
    ov, om, osx = oracle.prune24_act(X, out)
    if out == "bf16":
        wb = synth.f32_to_bf16_bits(W)
        wd, sw, ow, osw = dev_bf16(wb), None, wb, None
    else:
        wd, sw = ss.quant_lift_act(dev_f32(W), 2, out)
        ow, osw = oracle.quant_lift_act(W, 2, out)
    Y = host(ss.spgemm_tiled(ss.SS_SPARSE_X, M, N, K, tv, tm, wd, sx, sw, "f32"))
    exp = oracle.spgemm("X", ov, om, ow, K, out, osx, osw, "f32")
    assert_product(Y, exp, "X", ov, om, ow, K, out, osx, osw, "f32", TOL)


SLIDE_TILED_SHAPES = [(1, 8), (5, 40), (3, 1001), (16, 512), (130, 520), (257, 1000), (3, 18944), (2, 60000)]


def _w_ties(seed, rows, K, kind):
    """Weights N(0, 0.02^2) with many equal magnitudes (ties), an all-zero row and a half-zero row."""
    rng = np.random.default_rng(seed)
    w = synth.normal_f32(rng, (rows, K), 0.02)
    w[:, ::2] = np.round(w[:, ::2] * 100) / 100
    K4 = K // 4 * 4
    w[:, 1:K4:4] = -w[:, 0:K4:4]
    if rows > 2:
        w[2] = 0
        w[1, : K // 2] = 0
    return synth.f32_to_bf16_bits(w) if kind == "bf16" else w


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("out", ["i8", "fp8", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("shape", SLIDE_TILED_SHAPES)
def test_slide_decompose_tiled(ss, kind, out, n, shape):
    """One-pass weight preparation into the tiled layout: the oracle's decomposed operand re-indexed, and the
    same bytes as ss_slide_decompose followed by ss_pack_sparse. Rows past 128 exercise the XCD row order."""
    rows, K = shape
    w = _w_ties(rows * 13 + K + n, rows, K, kind)
    # rows start 16-byte aligned: ragged K lives in a wider buffer
    ldk = -(-K // 8) * 8
    wp = np.zeros((rows, ldk), w.dtype)
    wp[:, :K] = w
    wd = (dev_bf16(wp) if kind == "bf16" else dev_f32(wp))[:, :K]
    tv, tm, sc = ss.slide_decompose_tiled(wd, n, out)
    ov, om, osc = oracle.slide_decompose(w, n, out)
    es = 2 if out == "bf16" else 1
    ev, em = tile_ref(np.ascontiguousarray(ov).view(np.uint8).reshape(rows, -1), om, es)
    assert np.array_equal(host(tm), em)
    assert np.array_equal(host(tv), ev)
    if out == "bf16":
        assert sc is None
    else:
        assert np.array_equal(host(sc), osc)
    pv, pm, psc = ss.slide_decompose(wd, n, out)
    rv, rm = ss.pack_sparse(pv, pm)
    assert np.array_equal(host(rv), host(tv)) and np.array_equal(host(rm), host(tm))


@pytest.mark.parametrize("n", [2, 4])
def test_weight_sparse_path_one_pass(ss, n):
    """One-pass weight preparation + fused quant/lift + tiled product, INT8 bit-exact against the oracle."""
    M, N, K = 150, 260, 1000
    X, W, _ = synth.workload(91 + n, M, N, K, x_kind="bf16", outlier_frac=0.01)
    tv, tm, sw = ss.slide_decompose_tiled(dev_f32(W), n, "i8")
    xq, sx = ss.quant_lift_act(dev_bf16(X), n, "i8")
    Kc = ss.lifted_k(K, n)
    Y = host(ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, xq, sx, sw, "bf16"))
    ov, om, osw = oracle.slide_decompose(W, n, "i8")
    oxq, osx = oracle.quant_lift_act(X, n, "i8")
    assert np.array_equal(Y, oracle.spgemm("W", ov, om, oxq, Kc, "i8", osx, osw, "bf16"))


def test_spgemm_tiled_shared_workspace(ss):
    """One caller-owned workspace reused by two split-K products in a row, the second smaller; INT8 exact."""
    Kc_max = 0
    cases = []
    for seed, (M, N, K) in ((211, (64, 2000, 4096)), (212, (24, 700, 1024))):
        vals, meta, dense, sx, sw, Kc = _gemm_case(seed, M, N, K, 2, "i8", "W")
        cases.append((M, N, K, vals, meta, dense, sx, sw, Kc))
    need = max(ss.spgemm_tiled_workspace_bytes(ss.SS_SPARSE_W, M, N, Kc, "i8") for M, N, _, _, _, _, _, _, Kc in cases)
    assert need > 0
    import torch
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for M, N, K, vals, meta, dense, sx, sw, Kc in cases:
        tv, tm = ss.pack_sparse(dev_codes(vals, "i8"), dev_u8(meta))
        dsx, dsw = _scales(sx, sw)
        Y = host(ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, dev_codes(dense, "i8"), dsx, dsw, "bf16",
                                 workspace=ws))
        assert np.array_equal(Y, oracle.spgemm("W", vals, meta, dense, Kc, "i8", sx, sw, "bf16"))
