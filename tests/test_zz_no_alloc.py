"""GPU test of ss_spgemm_tiled_noalloc, the split-K entry point for callers that cannot allocate (its
partial tiles live in the library's static per-GPU scratch): called through the C ABI, its output equals
ss_spgemm_tiled_ws with a caller workspace bit for bit, on two calls in a row whose second is smaller (the
scratch keeps the first call's contents), in INT8 and FP8; the INT8 result also equals the oracle's."""
import ctypes

import numpy as np
import pytest

import oracle
from helpers import have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ss():
    import structured_sparse_quantized_amd as m
    return m


def _call_noalloc(ss, M, N, Kc, tv, tm, xq, sx, sw, Y):
    import torch
    st = ss.lib.ss_spgemm_tiled_noalloc(ss.SS_SPARSE_W, M, N, Kc, ss.dtype_code(xq.dtype), ctypes.c_void_p(tv.data_ptr()),
                                        ctypes.c_void_p(tm.data_ptr()), ctypes.c_void_p(xq.data_ptr()), xq.stride(0),
                                        ctypes.c_void_p(sx.data_ptr()), ctypes.c_void_p(sw.data_ptr()), ss.SS_BF16,
                                        ctypes.c_void_p(Y.data_ptr()), Y.stride(0),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == ss.SS_OK, ss.lib.ss_last_error().decode()


def _case(ss, q, M, N, K, n, seed):
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    W = torch.randn((N, K), generator=gen, device="cuda") * 0.02
    X = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    tv, tm, sw = ss.slide_decompose_tiled(W, n, q)
    xq, sx = ss.quant_lift_act(X, n, q)
    Kc = ss.lifted_k(K, n)
    need = ss.spgemm_tiled_workspace_bytes(ss.SS_SPARSE_W, M, N, Kc, q)
    assert 0 < need <= 8 << 20, need  # takes the split-K path, within the static scratch
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    Yws = ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, xq, sx, sw, "bf16", workspace=ws)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    _call_noalloc(ss, M, N, Kc, tv, tm, xq, sx, sw, Y)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yws.view(torch.int16))
    return W, X, Y, Kc


@pytest.mark.parametrize("q", ["i8", "fp8"])
def test_noalloc_equals_workspace_entry_two_calls(ss, q):
    import torch
    # first: Qwen2.5-7B-shaped 4:6 down at 64 tokens (8.3 MB of partial tiles, near the scratch's size);
    # second: a smaller ragged problem that reuses the scratch the first left behind
    _case(ss, q, 64, 3584, 18944, 3, seed=1)
    W, X, Y, Kc = _case(ss, q, 20, 1000, 1000, 3, seed=2)
    if q == "i8":
        Wh = W.cpu().numpy()
        Xh = X.view(torch.int16).cpu().numpy().view(np.uint16)
        ow, ox = oracle.slide_decompose(Wh, 3, "i8"), oracle.quant_lift_act(Xh, 3, "i8")
        exp = oracle.spgemm("W", ow[0], ow[1], ox[0], Kc, "i8", ox[1], ow[2], "bf16")
        assert np.array_equal(host(Y), exp)
