"""Host-side logic of bench.py (no GPU): the one-GPU contract, the byte and operation accounting behind the
roofline figures, the buffer rotation and the size of the last stdout line."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "structured_sparse_quantized_amd", "libss.so")


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus_requested"] == int(n)


@pytest.mark.skipif(not os.path.exists(LIB), reason="libss.so not built")
@pytest.mark.parametrize("rows,Kc", [(4096, 4096), (2048, 6144), (1, 256), (17, 512), (4096, 18944 * 3 // 2 // 256 * 256),
                                     (100, 1280), (28672, 4096)])
def test_bench_tiled_bytes_match_the_abi(rows, Kc):
    """The bench prices the tiled operand with its own formula; it must equal the library's size queries
    (8-bit and bf16 codes), or the GB/s and roofline fractions it prints are off."""
    import structured_sparse_quantized_amd as ss
    b = _bench()
    assert b.tiled_bytes(rows, Kc) == ss.tiled_bytes(rows, Kc, "i8")
    assert b.tiled_bytes(rows, Kc, 2) == ss.tiled_bytes(rows, Kc, "bf16")


def test_bench_work_counts():
    """Products count 2 M N K'/2 operations (kept values only); quantisation reads bf16 once and writes one code
    per lifted position plus a scale per token; weight prep reads float32 W once and writes the tiled operand."""
    b = _bench()
    assert b.product_ops(16384, 28672, 4096) == 16384 * 28672 * 4096
    assert b.product_ops(4096, 4096, 6144) == 4096 * 4096 * 6144
    assert b.quant_bytes(2048, 4096, 6144) == 2 * 2048 * 4096 + 2048 * 6144 + 4 * 2048
    # 2:4 at K = 4096: K/2 code bytes and K/8 index bytes per row
    assert b.prep_bytes(4096, 4096, 4096) == 4 * 4096 * 4096 + 4096 * 2048 + 4096 * 512 + 4 * 4096


def test_rotation_covers_twice_the_infinity_cache():
    b = _bench()
    for nbytes in (1, 29_000_000, 100 << 20, 300 << 20, 1 << 30):
        k = b.rotation(nbytes)
        assert k >= 1 and (k * nbytes >= 2 * b.MALL_BYTES or k == 64)
        assert k == 1 or (k - 1) * nbytes < 2 * b.MALL_BYTES


def test_last_line_is_compact():
    """The driver keeps a bounded tail of stdout: the final JSON line must stay well under 2,000 characters with
    every field filled (a synthetic line of the same shape and precision as main() prints, rounded the same
    way to 6 significant digits)."""
    b = _bench()
    out = {
        "metric": b.METRIC, "value": 8024332.757171267, "unit": "tokens/s", "n_gpus": 1, "steps": 20, "warmup": 5,
        "ms_per_step": 2.041789703369141, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped layer linears qkv+o+gate_up+down, 2:4 FP8-e4m3 W per-channel, "
                               "dynamic per-token FP8 X, bf16 out, 16384 tokens (online quant + sparse GEMM)",
                   "tokens": 16384, "global_batch": 16384, "parallelism": "none (1 GPU)"},
        "model_tokens_per_s": 250760.39866160208,
        "roofline": {"bound": "mfma", "achieved": 1924.1565513970645, "peak": 5000.0, "unit": "TFLOP/s",
                     "frac": 0.3848313102794129, "traffic": 3101175136.8254504,
                     "kernel": "gate_up product 16384x28672x4096, 2:4 FP8 (256x256 wide kernel)"},
        "vs_dense": 1.4618011575005978, "gemm_frac": {"qkv": 0.383, "o": 0.377, "gate_up": 0.392, "down": 0.434},
        "quant_GBs": 5232.1, "sclk_MHz_gate_up": 1832.5, "weight_prep_us": 214.0,
        "l24_fp8_4096": {"tps": 12345678, "vs_dense": 1.234, "gemm_frac_max": 0.345},
        "l68_i8_4096": {"tps": 12345678, "vs_dense": 1.234, "gemm_frac_max": 0.345},
        "l68_fp8_4096": {"tps": 12345678, "vs_dense": 1.234, "gemm_frac_max": 0.345},
        "l68_i8_16384": {"tps": 12345678, "vs_dense": 1.234, "gemm_frac_max": 0.345},
        "l68_fp8_16384": {"tps": 12345678, "vs_dense": 1.234, "gemm_frac_max": 0.345},
        "cpu_baseline": {"value": 147.89924188351085, "unit": "tokens/s", "cores": 16, "kind": "oracle",
                         "cpu": "AMD EPYC 9575F 64-Core Processor", "host_cpus": 16,
                         "sample": "256 tokens, four linears: FP8 quant of all K, product over >= 768 channels of each "
                                   "(scaled to all); float64 BLAS on 16 threads; weight prep (12.3 s) not counted"},
        "parity_vs_oracle": {"ok": True, "codes_bit_exact": True, "max_rel_fro": 0.00016947884109797242,
                             "max_elem_over_bound": 0.8965563788201644,
                             "sample": "256 tokens x >= 768 channels per linear, set 0 of the timed steps"},
        "detail": "gpurun_out/bench_detail.json",
    }
    line = json.dumps(b._sig6(out), default=b._round, separators=(",", ":"))
    assert len(line) < 1900, len(line)
    assert json.loads(line)["value"] == 8024330.0 and json.loads(line)["roofline"]["frac"] == 0.384831


def _fake_layer(plant):
    """A layer of small Llama-named linears whose 'GPU' outputs are the oracle's own (CPU tensors), optionally
    with one output element of gate_up off by a few bf16 ulps at a position every sample holds."""
    import numpy as np
    import torch
    import oracle

    class Lay:
        lin = {}

    lay = Lay()
    g = torch.Generator().manual_seed(0)
    for name, (K, N) in {"qkv": (512, 640), "o": (512, 384), "gate_up": (512, 1024), "down": (1024, 512)}.items():
        W = torch.randn((N, K), generator=g) * 0.02
        X = torch.randn((300, K), generator=g).to(torch.bfloat16)
        ow = oracle.prune24(W.numpy(), "fp8")
        ox = oracle.quant_lift_act(X.view(torch.int16).numpy().view(np.uint16), 2, "fp8")
        y = oracle.spgemm("W", ow[0], ow[1], ox[0], K, "fp8", ox[1], ow[2], "bf16")
        if plant and name == "gate_up":
            y = y.copy()
            y[0, 7] ^= 0x0040
        lay.lin[name] = dict(N=N, K=K, Kc=K, W=W, sw=torch.from_numpy(ow[2]),
                             sets=[dict(X=X, Y=torch.from_numpy(y.view(np.int16)).view(torch.bfloat16),
                                        xq=torch.from_numpy(ox[0]).view(torch.float8_e4m3fn),
                                        sx=torch.from_numpy(ox[1]))])
    return lay


@pytest.mark.parametrize("plant", [False, True])
def test_cpu_leg_parity_flags_one_wrong_element(plant):
    """The bench's sampled parity check passes the oracle's own outputs and fails when one element is off by a
    few ulps -- which the 1e-2 relative Frobenius gate alone lets through."""
    import torch
    b = _bench()
    parity, cpu = b.cpu_leg(torch, _fake_layer(plant), 300, 64, 300)
    assert parity["codes_bit_exact"]
    assert parity["ok"] is (not plant)
    if plant:
        assert parity["max_rel_fro"] < 1e-2 and parity["max_elem_over_bound"] > 1.0
    assert cpu["value"] > 0 and cpu["kind"] == "oracle"
