"""GPU parity of the sparse products at the layer sizes the benchmark times: the Llama-3.1-8B-shaped
projection layers (qkv 4096->6144, o 4096->4096, gate_up 4096->28672, down 14336->4096) in 2:4 FP8 and in
6:8 INT8 / FP8, and the Qwen2.5-7B-shaped 4:6 and 8:10 INT8 layers (gate_up 3584->37888, down
18944->3584) at decode and prefill token counts, each launched exactly as the benchmark launches it
(weights prepared in the tiled layout, per-token quant(+lift), then ss_spgemm_tiled, which picks the
row-block, split-K, 256 x 128 or 256 x 256 kernel by shape).

Inputs are seeded on the GPU (W ~ N(0, 0.02^2) float32, X ~ N(0, 1) bf16). The oracle recomputes a sample
of tokens (the first and last 16 and 32 random ones) against a sample of output channels (the first and
last 128 -- tile edges and the ragged end -- and 128 random ones): the weight prep of a channel and the
quantisation of a token depend on that row alone, so the sample needs no full-size oracle run. Codes and
scales of the sampled rows are compared bit for bit; products INT8 bit for bit, FP8 within 1e-2 relative
Frobenius error and element by element within 4e-5 sum|terms| plus one bf16 rounding step."""
import numpy as np
import pytest

import oracle
from helpers import assert_elementwise, bf16_to_f64, have_gpu, host, rel_fro, sum_abs_terms

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ss():
    import structured_sparse_quantized_amd as m
    return m


def _sample(n, k, rng, edge=16):
    if n <= 2 * edge + k:
        return np.arange(n)
    mid = rng.choice(np.arange(edge, n - edge), k, replace=False)
    return np.unique(np.concatenate([np.arange(edge), np.arange(n - edge, n), mid]))


def _layer(ss, n, q, M, K, N, seed, fused=False):
    """One layer as the benchmark runs it, checked on a sample against the oracle."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    W = torch.randn((N, K), generator=gen, device="cuda") * 0.02
    X = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    tv, tm, sw = ss.slide_decompose_tiled(W, n, q)
    Kc = ss.lifted_k(K, n)
    if fused:
        Y = ss.quant_lift_spgemm_decode(X, n, tv, tm, sw, N, q, "bf16")
        xq, sx = ss.quant_lift_act(X, n, q)
        Y2 = ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, xq, sx, sw, "bf16")
        assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), "one launch != two launches"
    else:
        xq, sx = ss.quant_lift_act(X, n, q)
        Y = ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, xq, sx, sw, "bf16")
    rng = np.random.default_rng(seed)
    toks = _sample(M, 32, rng)
    chans = _sample(N, 128, rng, edge=128)
    td = torch.from_numpy(toks).cuda()
    cd = torch.from_numpy(chans).cuda()
    Wh = W.index_select(0, cd).cpu().numpy()
    Xh = X.index_select(0, td).view(torch.int16).cpu().numpy().view(np.uint16)
    ow = oracle.prune24(Wh, q) if n == 2 else oracle.slide_decompose(Wh, n, q)
    ox = oracle.quant_lift_act(Xh, n, q)
    assert np.array_equal(host(sw)[chans], ow[2])
    assert np.array_equal(host(sx)[toks], ox[1])
    assert np.array_equal(host(xq)[toks].view(np.uint8), np.asarray(ox[0]).view(np.uint8))
    got = host(Y)[np.ix_(toks, chans)]
    exp = oracle.spgemm("W", ow[0], ow[1], ox[0], Kc, q, ox[1], ow[2], "bf16")
    if q == "i8":
        assert np.array_equal(got, exp)
    else:
        g, e = bf16_to_f64(got), bf16_to_f64(exp)
        assert rel_fro(g, e) <= 1e-2
        assert_elementwise(g, e, sum_abs_terms(ow[0], ow[1], ox[0], Kc, q, ox[1], ow[2]))


LLAMA = {"qkv": (4096, 6144), "o": (4096, 4096), "gate_up": (4096, 28672), "down": (14336, 4096)}


@pytest.mark.parametrize("case", [
    ("gate_up", 2, "fp8", 4096), ("o", 2, "fp8", 4096), ("qkv", 2, "fp8", 4096), ("down", 2, "fp8", 4096),
    ("gate_up", 2, "fp8", 16384), ("down", 2, "fp8", 16384), ("qkv", 2, "fp8", 16384), ("o", 2, "fp8", 16384),
    ("qkv", 4, "i8", 4096), ("o", 4, "i8", 4096), ("gate_up", 4, "i8", 4096), ("down", 4, "i8", 4096),
    ("gate_up", 4, "fp8", 4096), ("down", 4, "fp8", 4096), ("gate_up", 4, "i8", 16384), ("down", 4, "i8", 16384),
])
def test_llama_layers(ss, case):
    """2:4 FP8 at 4096 and 16384 tokens (the benchmark's headline layer), and 6:8 (K' = 1.5 K, down at
    K' = 21504) in INT8 and FP8."""
    name, n, q, M = case
    K, N = LLAMA[name]
    _layer(ss, n, q, M, K, N, seed=sum(map(ord, name)) + 10 * n + M)


QWEN = {"qkv": (3584, 4608), "gate_up": (3584, 37888), "down": (18944, 3584)}


@pytest.mark.parametrize("n", [3, 5])
@pytest.mark.parametrize("case", [("gate_up", 1), ("gate_up", 64), ("gate_up", 4096), ("down", 4096),
                                  ("down", 64), ("qkv", 4096)])
def test_qwen_layers(ss, n, case):
    """4:6 and 8:10 INT8 (K' = 4/3 K and 1.6 K, K not a multiple of 2n) at decode and prefill token counts:
    row-block (1 token), split-K (64 tokens) and the prefill kernels; down at 4096 tokens runs K' = 25344
    (4:6) and 30464 (8:10) through the prefill kernel."""
    name, M = case
    K, N = QWEN[name]
    _layer(ss, n, "i8", M, K, N, seed=31 * n + M)


@pytest.mark.parametrize("n", [2, 3, 4, 5])
@pytest.mark.parametrize("M", [1, 4])
def test_one_launch_decode_many_row_blocks(ss, n, M):
    """The one-launch few-token layer with N = 37888 (2368 row blocks): every persistent workgroup runs
    several row blocks, so the reuse of the partial-sum buffer, the reload of the channel scales and the
    wait states between the last matrix instruction and the store are exercised; lifts that stage plain
    codes and gather windows (4:6, 8:10) and those written from registers (2:4, 6:8 from bf16)."""
    K, N = QWEN["gate_up"]
    _layer(ss, n, "i8", M, K, N, seed=7 * n + M, fused=True)


@pytest.mark.parametrize("q,y", [("i8", "i32"), ("i8", "bf16"), ("fp8", "f32"), ("fp8", "bf16"), ("bf16", "f32")])
def test_wide_kernel_sparse_activations_ragged(ss, q, y):
    """The sparse-activation side on the wide-wave kernel's 256 x 128 form (6000 tokens pruned 2:4 online into
    the tiled layout x 1500 dense channels: 288 tiles), ragged on both sides, K = 1280 ending inside a 4-step
    index group; outputs Y[token][channel] staged as whole 16-byte row pieces."""
    import torch
    M, K, N = 6000, 1280, 1500
    gen = torch.Generator(device="cuda")
    gen.manual_seed(123)
    X = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    W = torch.randn((N, K), generator=gen, device="cuda") * 0.02
    tv, tm, sx = ss.prune24_act_tiled(X, q)
    if q == "bf16":
        wd, sw = W.to(torch.bfloat16), None
    else:
        wd, sw = ss.quant_lift_act(W, 2, q)
    Y = ss.spgemm_tiled(ss.SS_SPARSE_X, M, N, K, tv, tm, wd, sx, sw, y)
    rng = np.random.default_rng(9)
    toks = _sample(M, 48, rng, edge=128)
    chans = _sample(N, 96, rng, edge=128)
    Xh = X.index_select(0, torch.from_numpy(toks).cuda()).view(torch.int16).cpu().numpy().view(np.uint16)
    Wc = W.index_select(0, torch.from_numpy(chans).cuda())
    got = host(Y)[np.ix_(toks, chans)]
    ov, om, osx = oracle.prune24_act(Xh, q)
    if q == "bf16":
        ow, osw = Wc.to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16), None
    else:
        ow, osw = oracle.quant_lift_act(Wc.cpu().numpy(), 2, q)
    exp = oracle.spgemm("X", ov, om, ow, K, q, osx, osw, y)
    if q == "i8":
        assert np.array_equal(got, exp)
        return
    g, e = (bf16_to_f64(got), bf16_to_f64(exp)) if y == "bf16" else (got, exp)
    assert rel_fro(g, e) <= 1e-2
    assert_elementwise(g, e, sum_abs_terms(ov, om, ow, K, q, osw, osx).T, out=y)


@pytest.mark.parametrize("shape", [(4000, 1280, 16484), (4000, 8960, 16484), (1500, 1280, 6000), (3000, 8960, 4000),
                                   (2300, 8960, 4000)],
                         ids=["256x256-8waves", "256x256-4waves", "256x128", "256x256-4waves-long-k", "256x128-long-k"])
@pytest.mark.parametrize("q", ["i8", "fp8", "bf16"])
def test_wide_kernel_ragged(ss, q, shape):
    """Products routed to the wide-wave kernel, with ragged tiles on both sides and a reduction that ends inside
    a 4-step index group: N = 16484 channels and 4000 tokens take its 256 x 256 tiles (four or more per CU), with
    eight waves at K = 1280 (INT8 / FP8 10 steps of 128, bf16 20 steps of 64) and four at K = 8960 (70 and 140
    steps); N = 6000 and 1500 tokens at K = 1280 its 256 x 128 tiles with two workgroups per CU (288 such
    tiles, 144 of 256 x 256). With a reduction over 64 steps (K = 8960) 256 x 256 tiles are taken from 0.6 of
    one per CU: N = 4000 and 3000 tokens (192 of them, four waves); N = 4000 and 2300 tokens (144, below that)
    take the 256 x 128 form (288 tiles)."""
    import torch
    M, K, N = shape
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    W = torch.randn((N, K), generator=gen, device="cuda") * 0.02
    X = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    Kc = ss.lifted_k(K, 2)
    if q == "bf16":
        tv, tm, _ = ss.slide_decompose_tiled(W.to(torch.bfloat16), 2, "bf16")
        Y = ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, X, None, None, "f32")
    else:
        tv, tm, sw = ss.slide_decompose_tiled(W, 2, q)
        xq, sx = ss.quant_lift_act(X, 2, q)
        Y = ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, tv, tm, xq, sx, sw, "i32" if q == "i8" else "f32")
    rng = np.random.default_rng(5)
    toks = _sample(M, 32, rng)
    chans = _sample(N, 128, rng, edge=128)
    td = torch.from_numpy(toks).cuda()
    cd = torch.from_numpy(chans).cuda()
    Xh = X.index_select(0, td).view(torch.int16).cpu().numpy().view(np.uint16)
    got = host(Y)[np.ix_(toks, chans)]
    if q == "bf16":
        Wh = W.index_select(0, cd).to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
        ow = oracle.prune24(Wh, "bf16")
        exp = oracle.spgemm("W", ow[0], ow[1], Xh, Kc, "bf16", None, None, "f32")
        assert rel_fro(got, exp) <= 1e-2
        assert_elementwise(got, exp, sum_abs_terms(ow[0], ow[1], Xh, Kc, "bf16"), out="f32")
        return
    Wh = W.index_select(0, cd).cpu().numpy()
    ow = oracle.prune24(Wh, q)
    ox = oracle.quant_lift_act(Xh, 2, q)
    if q == "i8":
        exp = oracle.spgemm("W", ow[0], ow[1], ox[0], Kc, q, None, None, "i32")
        assert np.array_equal(got, exp)
    else:
        exp = oracle.spgemm("W", ow[0], ow[1], ox[0], Kc, q, ox[1], ow[2], "f32")
        assert rel_fro(got, exp) <= 1e-2
        assert_elementwise(got, exp, sum_abs_terms(ow[0], ow[1], ox[0], Kc, q, ox[1], ow[2]), out="f32")
