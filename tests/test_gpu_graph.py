"""The online half of the path (quant+lift, then the sparse product) captured in a HIP graph: the calls
are stateless, allocate nothing and record no memset, so a graph replays them. Each replay runs on new
input contents written between replays, with eager work and synchronisations in between, and must equal
eager calls on the same inputs bit for bit. Covers the prefill kernels, the few-token row-block kernel,
the split-K kernel with a caller-owned workspace, the block-scaled FP8 pair and the one-launch few-token
entry."""
import numpy as np
import pytest

from helpers import have_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ss():
    import structured_sparse_quantized_amd as m
    return m


# (tokens, channels, K, n): prefill 6:8 (8-wave kernel); 2:4 prefill on the wide-wave kernel's 256 x 128
# (4096 x 6144) and 256 x 256 (16384 x 4096) forms; decode 4:6 at 1 token (row-block kernel) and 48 tokens
# (split-K)
CASES = [(2048, 4096, 4096, 4), (4096, 6144, 4096, 2), (16384, 4096, 4096, 2), (1, 3584, 18944, 3),
         (48, 3584, 18944, 3), (40, 4608, 3584, 5)]


@pytest.mark.parametrize("case", CASES)
def test_graph_replays_match_eager(ss, case):
    import torch
    M, N, K, n = case
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(M + N + K + n)
    W = torch.randn((N, K), generator=gen, device=dev) * 0.02
    tv, tm, sw = ss.slide_decompose_tiled(W, n, "i8")
    Kc = ss.lifted_k(K, n)
    X = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    xq = torch.empty((M, Kc), dtype=torch.int8, device=dev)
    sx = torch.empty(M, dtype=torch.float32, device=dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    need = ss.spgemm_tiled_workspace_bytes(ss.SS_SPARSE_W, M, N, Kc, "i8")
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else False
    if M == 48:
        assert need > 0, "this case is meant to take the split-K path"

    def path():
        ss.quant_lift_act(X, n, "i8", out=(xq, sx))
        ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, xq, sx, sw, "bf16", out=Y, workspace=ws)

    X.copy_(torch.randn((M, K), generator=gen, device=dev))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    torch.cuda.synchronize()
    for rep in range(3):
        X.copy_(torch.randn((M, K), generator=gen, device=dev) * (1.0 + rep))
        graph.replay()
        torch.cuda.synchronize()
        got = Y.clone()
        got_q, got_s = xq.clone(), sx.clone()
        # eager on the same input, into fresh buffers
        eq, es = ss.quant_lift_act(X, n, "i8")
        ey = ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, eq, es, sw, "bf16")
        torch.cuda.synchronize()
        assert torch.equal(got_q, eq) and torch.equal(got_s, es), rep
        assert torch.equal(got.view(torch.int16), ey.view(torch.int16)), rep
    assert np.isfinite(Y.float().cpu().numpy()).all()


def _replay_check(ss, path, inputs, outputs, eager, reps=3, seed=0):
    """Capture path() once, then for each replay write new inputs, replay, and compare every output with
    eager() on the same inputs (bit for bit)."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    torch.cuda.synchronize()
    for rep in range(reps):
        for t in inputs:
            t.copy_(torch.randn(t.shape, generator=gen, device="cuda") * (1.0 + rep))
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outputs]
        exp = eager()
        torch.cuda.synchronize()
        for g, e in zip(got, exp):
            assert torch.equal(g.view(torch.uint8), e.view(torch.uint8)), rep


def test_graph_block_scaled_pair(ss):
    import torch
    M, N, K = 512, 1024, 2048
    W = torch.randn((N, K), device="cuda") * 0.02
    tv, tm, sw = ss.prune24_block(W)
    Kc = ss.lifted_k(K, 2)
    X = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    xq = torch.empty((M, Kc), dtype=torch.float8_e4m3fn, device="cuda")
    sx = torch.empty((M, Kc // 128), device="cuda")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def path():
        ss.quant_group_act(X, out=(xq, sx))
        ss.spgemm_tiled_block(M, N, Kc, tv, tm, xq, sx, sw, "bf16", out=Y)

    def eager():
        q, s = ss.quant_group_act(X)
        return [q, s, ss.spgemm_tiled_block(M, N, Kc, tv, tm, q, s, sw, "bf16")]

    _replay_check(ss, path, [X], [xq, sx, Y], eager, seed=1)


@pytest.mark.parametrize("M", [1, 3])
def test_graph_one_launch_decode(ss, M):
    import torch
    N, K, n = 3584, 18944, 3
    W = torch.randn((N, K), device="cuda") * 0.02
    tv, tm, sw = ss.slide_decompose_tiled(W, n, "i8")
    X = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    sxo = torch.empty(M, device="cuda")

    def path():
        ss.quant_lift_spgemm_decode(X, n, tv, tm, sw, N, "i8", "bf16", out=Y, sx_out=sxo)

    def eager():
        s = torch.empty(M, device="cuda")
        y = ss.quant_lift_spgemm_decode(X, n, tv, tm, sw, N, "i8", "bf16", sx_out=s)
        return [y, s]

    _replay_check(ss, path, [X], [Y, sxo], eager, seed=2)
