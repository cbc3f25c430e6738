"""GPU parity of ss_quant_spgemm_prefill, the prefill layer with the per-token quantisation inside the sparse
product (the coded activations are written into the product's LDS stages, never to HBM): its output and
per-token scales equal ss_quant_lift_act (n = 2) followed by ss_spgemm_tiled bit for bit, INT8 and FP8,
bf16 and f32 outputs, on ragged tiles, a reduction with a padding step (K = 1152: 9 steps of 128 in a
10-step K'), all-zero tokens and the Llama-shaped layers; INT8 also equals the oracle."""
import numpy as np
import pytest

import oracle
from helpers import have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ss():
    import structured_sparse_quantized_amd as m
    return m


@pytest.mark.parametrize("y", ["bf16", "f32"])
@pytest.mark.parametrize("q", ["i8", "fp8"])
@pytest.mark.parametrize("shape", [(300, 520, 1152), (129, 257, 128), (2048, 4096, 4096), (4096, 6144, 4096),
                                   (1000, 4096, 14336)])
def test_quant_prefill_equals_two_calls(ss, shape, q, y):
    import torch
    M, N, K = shape
    gen = torch.Generator(device="cuda")
    gen.manual_seed(M + N + K)
    W = torch.randn((N, K), generator=gen, device="cuda") * 0.02
    X = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    X[min(3, M - 1)] = 0  # an all-zero token
    tv, tm, sw = ss.slide_decompose_tiled(W, 2, q)
    Yf, sxf = ss.quant_spgemm_prefill(X, tv, tm, sw, N, q, y)
    xq, sx = ss.quant_lift_act(X, 2, q)
    Y2 = ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, ss.lifted_k(K, 2), tv, tm, xq, sx, sw, y)
    assert torch.equal(sxf, sx)
    assert torch.equal(Yf.view(torch.int16 if y == "bf16" else torch.int32),
                       Y2.view(torch.int16 if y == "bf16" else torch.int32))
    if q == "i8" and M * N <= 4096 * 4096:
        rng = np.random.default_rng(1)
        toks = np.unique(np.concatenate([[0, min(3, M - 1), M - 1], rng.choice(M, min(M, 40), replace=False)]))
        td = torch.from_numpy(toks).cuda()
        ow = oracle.prune24(W.cpu().numpy(), "i8")
        ox = oracle.quant_lift_act(X.index_select(0, td).view(torch.int16).cpu().numpy().view(np.uint16), 2, "i8")
        exp = oracle.spgemm("W", ow[0], ow[1], ox[0], ss.lifted_k(K, 2), "i8", ox[1], ow[2], y)
        assert np.array_equal(host(Yf)[toks], exp)


def test_quant_prefill_rejects_ragged_k(ss):
    import torch
    X = torch.zeros((16, 1000), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((32, 1000), device="cuda")
    tv, tm, sw = ss.slide_decompose_tiled(W, 2, "i8")
    with pytest.raises(ss.SSError) as e:
        ss.quant_spgemm_prefill(X, tv, tm, sw, 32, "i8")
    assert e.value.status == ss.SS_ERR_SHAPE
