"""GPU parity of the few-token fused entry (ss_quant_lift_spgemm_decode: quant+lift done by every workgroup
of the row-block product into LDS): equal bit for bit to ss_quant_lift_act followed by ss_spgemm_tiled
(INT8 and FP8, every output type), and to the CPU oracle (INT8 bit-exact, FP8 within 1e-2 relative
Frobenius error and element by element within 4e-5 sum|terms| plus one output rounding); the per-token
scales it can return equal the oracle's."""
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


def _dev_rows(x, kind):
    per = 8 if kind == "bf16" else 4
    K = x.shape[1]
    wide = np.zeros((x.shape[0], -(-K // per) * per + per), x.dtype)
    wide[:, :K] = x
    return (dev_bf16(wide) if kind == "bf16" else dev_f32(wide))[:, :K]


# (M, N, K, n): Qwen2.5-7B-shaped rows, ragged N and K (K not a multiple of 8 or of 2n), every pattern
CASES = [(1, 4608, 3584, 3), (4, 4608, 3584, 5), (2, 3584, 18944, 3), (1, 3584, 18944, 5), (3, 1000, 1002, 4),
         (4, 130, 203, 2), (1, 17, 64, 4), (2, 300, 4096, 4), (3, 520, 777, 8), (4, 256, 4096, 6)]


@pytest.mark.parametrize("q", ["i8", "fp8"])
@pytest.mark.parametrize("case", CASES)
def test_fused_matches_two_calls_and_oracle(ss, case, q):
    import torch
    M, N, K, n = case
    X, W, _ = synth.workload(M * 7 + N + K + n, M, N, K, outlier_frac=0.01 if K >= 100 else 0.0)
    if M >= 3:
        X[1] = 0  # an all-zero token
    xd = _dev_rows(X, "bf16")
    tv, tm, sw = ss.slide_decompose_tiled(_dev_rows(W, "f32"), n, q)
    Kc = ss.lifted_k(K, n)
    sxo = torch.full((M,), -1.0, device="cuda")
    Yf = ss.quant_lift_spgemm_decode(xd, n, tv, tm, sw, N, q, "bf16", sx_out=sxo)
    xq, sx = ss.quant_lift_act(xd, n, q)
    Y2 = ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, xq, sx, sw, "bf16")
    assert torch.equal(Yf.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(sxo, sx)
    ov, om, osw = oracle.slide_decompose(W, n, q)
    oq, osx = oracle.quant_lift_act(X, n, q)
    assert np.array_equal(host(sxo), osx)
    exp = oracle.spgemm("W", ov, om, oq, Kc, q, osx, osw, "bf16")
    assert_product(host(Yf), exp, "W", ov, om, oq, Kc, q, osx, osw, "bf16")


# (M, N, K, n, q): more row blocks than twice the CUs, so the persistent kernel hands every workgroup two or
# more of them whatever its per-CU count: Qwen2.5-7B gate_up with a ragged last block (small LDS, two
# workgroups a CU, 2368 blocks), four tokens at K = 12000 (about 80 KB of LDS, one workgroup a CU, 563 blocks),
# 6:8 from bf16 (no staging row, 1250 blocks)
MANY_BLOCKS = [(1, 37885, 3584, 3, "i8"), (4, 9000, 12000, 3, "fp8"), (3, 20000, 4096, 4, "i8")]


@pytest.mark.parametrize("case", MANY_BLOCKS)
def test_fused_row_blocks_past_the_grid(ss, case):
    """Workgroups that run a second and later row block reuse their LDS codes, reduction slots and scale
    registers: the whole output equals the two calls bit for bit (the row-block kernel there runs one block a
    workgroup), and sampled channels, including row blocks past the first pass of the grid and the ragged
    last block, equal the oracle (INT8 bit-exact, FP8 within 1e-2)."""
    import torch
    M, N, K, n, q = case
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nrb = -(-N // 16)
    assert nrb > 2 * cus, "the case must give every workgroup more than one row block"
    X, W, _ = synth.workload(M * 7 + N + K + n, M, N, K)
    xd = _dev_rows(X, "bf16")
    tv, tm, sw = ss.slide_decompose_tiled(_dev_rows(W, "f32"), n, q)
    Kc = ss.lifted_k(K, n)
    Yf = ss.quant_lift_spgemm_decode(xd, n, tv, tm, sw, N, q, "bf16")
    xq, sx = ss.quant_lift_act(xd, n, q)
    Y2 = ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, xq, sx, sw, "bf16")
    assert torch.equal(Yf.view(torch.int16), Y2.view(torch.int16))
    rng = np.random.default_rng(N)
    later = [g * 16 + r for g in (cus, 2 * cus, 2 * cus + 1, nrb - 2) for r in (0, 7, 15)]
    chans = np.unique(np.concatenate([np.arange(16), np.arange(N - 48, N), np.asarray(later),
                                      rng.choice(N, 160, replace=False)]))
    chans = chans[chans < N]
    ov, om, osw = oracle.slide_decompose(np.ascontiguousarray(W[chans]), n, q)
    oq, osx = oracle.quant_lift_act(X, n, q)
    exp = oracle.spgemm("W", ov, om, oq, Kc, q, osx, osw, "bf16")
    got = host(Yf)[:, chans]
    assert_product(got, exp, "W", ov, om, oq, Kc, q, osx, osw, "bf16")


@pytest.mark.parametrize("y", ["f32", "i32"])
@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_fused_output_types_and_f32_input(ss, kind, y):
    import torch
    M, N, K, n = 3, 700, 2050, 4
    X, W, _ = synth.workload(91, M, N, K, x_kind=kind)
    xd = _dev_rows(X, kind)
    tv, tm, sw = ss.slide_decompose_tiled(_dev_rows(W, "f32"), n, "i8")
    Kc = ss.lifted_k(K, n)
    Yf = ss.quant_lift_spgemm_decode(xd, n, tv, tm, sw, N, "i8", y)
    xq, sx = ss.quant_lift_act(xd, n, "i8")
    Y2 = ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, xq, sx, sw, y)
    assert np.array_equal(host(Yf), host(Y2))
    ov, om, osw = oracle.slide_decompose(W, n, "i8")
    oq, osx = oracle.quant_lift_act(X, n, "i8")
    assert np.array_equal(host(Yf), oracle.spgemm("W", ov, om, oq, Kc, "i8", osx, osw, y))


def test_fused_limits_fall_back_cleanly(ss):
    import torch
    M, N, K = 5, 64, 512
    xd = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    tv, tm, sw = ss.slide_decompose_tiled(torch.zeros((N, K), device="cuda"), 4, "i8")
    with pytest.raises(ss.SSError) as e:
        ss.quant_lift_spgemm_decode(xd, 4, tv, tm, sw, N)
    assert e.value.status == ss.SS_ERR_UNSUPPORTED
