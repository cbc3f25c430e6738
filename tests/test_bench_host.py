"""Host-side logic of bench.py (no GPU): the one-GPU contract and the byte accounting behind the roofline
figures of the streaming kernels."""
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
                                     (100, 1280)])
def test_bench_tiled_bytes_match_the_abi(rows, Kc):
    """The bench prices the tiled operand with its own formula; it must equal the library's size queries
    (8-bit codes), or the GB/s and roofline fractions it prints are off."""
    import structured_sparse_quantized_amd as ss
    assert _bench().tiled_bytes(rows, Kc) == ss.tiled_bytes(rows, Kc, "i8")


def test_bench_kernel_work_counts():
    """Products count 2 M N K'/2 operations (kept values only); the prep kernels read their input once and
    write the operand they produce once."""
    b = _bench()
    M, N, K = b.M, b.N, b.K
    Kc68, Kc24 = 6144, 4096
    kind, ops = b.kernel_work("spgemm_68", Kc68, Kc24)
    assert kind == "mfma" and ops == M * N * Kc68
    kind, byts = b.kernel_work("quant_lift_68", Kc68, Kc24)
    assert kind == "hbm" and byts == 2 * M * K + M * Kc68 + 4 * M
    # 2:4 activation prune into the tiled layout: K/2 code bytes and K/8 index bytes per row at this shape
    kind, byts = b.kernel_work("prune24_act_tiled", Kc68, Kc24)
    assert byts == 2 * M * K + M * K // 2 + M * K // 8 + 4 * M
