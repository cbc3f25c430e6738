"""Benchmark of the structured-sparse quantised linear path on one MI355X.

A step is one pass of every kernel on the path over one batch of the
6:8 sliding-window INT8 workload (W 4096x4096 N(0, 0.02^2) float32, X
2048x4096 bf16 N(0,1) with 1% outlier columns x20), all INT8:

  slide_decompose_tiled(W, n=4) -> quant_lift_act(X, n=4) -> spgemm_tiled(sparse W')   6:8
  slide_decompose_tiled(W, n=2) -> quant_lift_act(X, n=2) -> spgemm_tiled(sparse W)    2:4
  prune24_act_tiled(X), quant_lift_act(W, n=2) -> spgemm_tiled(sparse X)              2:4 on X

The weight-side preparation (decompose or prune, written straight into the
product's tiled layout) runs offline in a deployment; it is timed here per
step all the same.

``value`` is tokens per second of the whole step (M tokens per step), from K
steps launched back to back between one pair of events. Per-kernel times come
from a second timed region in which each call runs K times back to back
between its own pair of events (an event between every two launches would
drain the queue and add ~3.5 us per event). The JSON line carries these
per-kernel times with their throughput against the roofline, the online 6:8 prefill rate (quant_lift + spgemm only), the dense
INT8 comparator, the roofline of the dominant kernel and the CPU oracle
baseline. Inputs are seeded and synthetic; NBUF rotating buffer sets keep the
working set above the 256 MB Infinity Cache so kernels stream from HBM.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse GEMM TOPS & prefill tokens/s (2:4, 6:8) vs dense; quant+lift GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_DENSE_PEAK_TOPS = 5000.0  # MI355X dense INT8 MFMA (ops counted on kept values only)

M, N, K, PAT = 2048, 4096, 4096, 4
NBUF = 3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--kernels-only", action="store_true", help="skip the dense comparator and CPU baseline")
    p.add_argument("--no-clock", action="store_true", help="skip the engine-clock sampling loop")
    p.add_argument("--no-suite", action="store_true", help="skip the Llama/Qwen-shaped layer suite")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 256 MiB device copy (the reference for HBM byte counters)")
    return p.parse_args()


def traffic_record(kernel):
    """HBM traffic per launch measured with rocprofv3 counters, if it was taken
    on the current source of the kernel (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, "structured_sparse_quantized_amd", "csrc", f), "rb").read())
    return rec["bytes_per_launch"] if h.hexdigest()[:16] == rec["source_sha256_16"] else None


def tiled_bytes(rows, Kc):
    """Bytes of the tiled operand (values, metadata), as include/ss.h defines them."""
    g = -(-(Kc // 128) // 4)
    rb = -(-rows // 16)
    return rb * g * 4 * 1024, rb * g * 1024


def kernel_work(name, Kc68, Kc24):
    """Algorithmic bytes (HBM-bound kernels) or ops (products) per launch."""
    b = {
        # weight preparation written in the tiled layout: W read once, tiled operand + scales written
        "slide_decompose_tiled_68": 4 * N * K + sum(tiled_bytes(N, Kc68)) + 4 * N,
        "quant_lift_68": 2 * M * K + M * Kc68 + 4 * M,
        "prune24_w_tiled": 4 * N * K + sum(tiled_bytes(N, Kc24)) + 4 * N,
        "quant_lift_24": 2 * M * K + M * Kc24 + 4 * M,
        # online prune of X written in the tiled layout: X read once, tiled operand + scales written
        "prune24_act_tiled": 2 * M * K + sum(tiled_bytes(M, Kc24)) + 4 * M,
        "quant_w": 4 * N * K + N * Kc24 + 4 * N,
    }
    # products: multiply-adds on the kept values only (K'/2 per row), x2 ops
    ops = {
        "spgemm_68": 2 * M * N * (Kc68 // 2),
        "spgemm_24": 2 * M * N * (Kc24 // 2),
        "spgemm_x": 2 * M * N * (Kc24 // 2),
    }
    if name in b:
        return "hbm", b[name]
    return "mfma", ops[name]


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; run with --gpus 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    import structured_sparse_quantized_amd as ss
    import synth

    dev = torch.device("cuda:0")
    Kc68, Kc24 = ss.lifted_k(K, PAT), ss.lifted_k(K, 2)
    print(f"[bench] generating inputs M={M} N={N} K={K}", file=sys.stderr, flush=True)
    X_np, W_np, _ = synth.workload(0, M, N, K, x_kind="bf16", outlier_frac=0.01)
    X0 = torch.from_numpy(X_np.view(np.int16)).view(torch.bfloat16).to(dev)
    W0 = torch.from_numpy(W_np).to(dev)

    def mk(shape, dt):
        return torch.empty(shape, dtype=dt, device=dev)

    bufs = []
    for i in range(NBUF):
        bufs.append(dict(
            X=X0.clone(), W=W0.clone(),
            t68=tuple(mk(nb, torch.uint8) for nb in tiled_bytes(N, Kc68)) + (mk(N, torch.float32),),
            t24=tuple(mk(nb, torch.uint8) for nb in tiled_bytes(N, Kc24)) + (mk(N, torch.float32),),
            tx=tuple(mk(nb, torch.uint8) for nb in tiled_bytes(M, Kc24)),
            x68=(mk((M, Kc68), torch.int8), mk(M, torch.float32)),
            y68=mk((M, N), torch.bfloat16),
            x24=(mk((M, Kc24), torch.int8), mk(M, torch.float32)),
            y24=mk((M, N), torch.bfloat16),
            xs=(mk(M, torch.float32),),
            wq=(mk((N, Kc24), torch.int8), mk(N, torch.float32)),
            yx=mk((M, N), torch.bfloat16),
        ))
    names = ["slide_decompose_tiled_68", "quant_lift_68", "spgemm_68", "prune24_w_tiled", "quant_lift_24",
             "spgemm_24", "prune24_act_tiled", "quant_w", "spgemm_x"]

    def calls(b):
        return [
            lambda: ss.slide_decompose_tiled(b["W"], PAT, "i8", out=b["t68"]),
            lambda: ss.quant_lift_act(b["X"], PAT, "i8", out=b["x68"]),
            lambda: ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc68, b["t68"][0], b["t68"][1], b["x68"][0], b["x68"][1],
                                    b["t68"][2], "bf16", out=b["y68"]),
            lambda: ss.slide_decompose_tiled(b["W"], 2, "i8", out=b["t24"]),
            lambda: ss.quant_lift_act(b["X"], 2, "i8", out=b["x24"]),
            lambda: ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc24, b["t24"][0], b["t24"][1], b["x24"][0], b["x24"][1],
                                    b["t24"][2], "bf16", out=b["y24"]),
            lambda: ss.prune24_act_tiled(b["X"], "i8", out=(b["tx"][0], b["tx"][1], b["xs"][0])),
            lambda: ss.quant_lift_act(b["W"], 2, "i8", out=b["wq"]),
            lambda: ss.spgemm_tiled(ss.SS_SPARSE_X, M, N, Kc24, b["tx"][0], b["tx"][1], b["wq"][0], b["xs"][0],
                                    b["wq"][1], "bf16", out=b["yx"]),
        ]

    steps_calls = [calls(b) for b in bufs]

    def step(s):
        for c in steps_calls[s % NBUF]:
            c()

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    # Timed region 1: K whole steps back to back, no per-call events (a timing
    # event between two launches costs the GPU ~3.5 us: it drains the queue).
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        step(s)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step (wall {wall:.3f} s)", file=sys.stderr, flush=True)

    # Timed region 2: per-call durations. Each call of the step runs K times
    # back to back (rotating buffer sets) between one pair of events on the
    # stream the kernels are launched on; duration = elapsed / K.
    per_kernel_ms = {}
    for i, n in enumerate(names):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for s in range(args.steps):
            steps_calls[s % NBUF][i]()
        e1.record()
        torch.cuda.synchronize()
        per_kernel_ms[n] = e0.elapsed_time(e1) / args.steps
    print("[bench] per-call us: " + ", ".join(f"{n} {v * 1e3:.1f}" for n, v in per_kernel_ms.items()),
          file=sys.stderr, flush=True)

    kernels = {}
    for n in names:
        kind, work = kernel_work(n, Kc68, Kc24)
        t = per_kernel_ms[n] * 1e-3
        if kind == "hbm":
            a = work / t / 1e9
            kernels[n] = {"us": per_kernel_ms[n] * 1e3, "bound": "hbm", "GB/s": a, "frac": a / HBM_PEAK_GBS,
                          "bytes": work}
        else:
            a = work / t / 1e12
            kernels[n] = {"us": per_kernel_ms[n] * 1e3, "bound": "mfma", "TOPS": a,
                          "frac": a / INT8_DENSE_PEAK_TOPS, "ops": work,
                          "dense_equiv_TOPS": 2 * a}
    dom = max(names, key=lambda n: per_kernel_ms[n])
    dk = kernels[dom]
    roofline = {
        "kernel": dom, "bound": dk["bound"],
        "achieved": dk["GB/s"] if dk["bound"] == "hbm" else dk["TOPS"],
        "peak": HBM_PEAK_GBS if dk["bound"] == "hbm" else INT8_DENSE_PEAK_TOPS,
        "unit": "GB/s" if dk["bound"] == "hbm" else "TFLOP/s",
        "frac": dk["frac"], "traffic": traffic_record(dom),
    }
    # the three outputs of one step, kept on the host for the parity check against the oracle below (not in
    # the counter runs, whose last dispatches must be the calibration copies)
    check_parity = not (args.no_cpu or args.kernels_only)
    y_gpu = ({k: bufs[0][k].view(torch.int16).cpu().numpy().view(np.uint16) for k in ("y68", "y24", "yx")}
             if check_parity else None)
    online68_s = (per_kernel_ms["quant_lift_68"] + per_kernel_ms["spgemm_68"]) * 1e-3
    online24_s = (per_kernel_ms["quant_lift_24"] + per_kernel_ms["spgemm_24"]) * 1e-3
    # sparse-activation layer: online prune + pack of X, then the product (W quantised offline)
    onlinex_s = (per_kernel_ms["prune24_act_tiled"] + per_kernel_ms["spgemm_x"]) * 1e-3

    # dense INT8 comparator: our per-token quantiser + hipBLASLt int8 GEMM (torch._int_mm)
    dense = None
    if not args.kernels_only:
        try:
            b = bufs[0]
            wq = b["wq"][0][:, :K].contiguous()
            xq = b["x24"][0][:, :K].contiguous()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for _ in range(3):
                torch._int_mm(xq, wq.t())
            torch.cuda.synchronize()
            reps = 20
            e0.record()
            for _ in range(reps):
                torch._int_mm(xq, wq.t())
            e1.record()
            torch.cuda.synchronize()
            t_mm = e0.elapsed_time(e1) / reps * 1e-3
            t_q = per_kernel_ms["quant_lift_24"] * 1e-3
            dense = {"gemm_us": t_mm * 1e6, "quant_us": t_q * 1e6, "gemm_TOPS": 2 * M * N * K / t_mm / 1e12,
                     "library": "hipBLASLt via torch._int_mm (int32 out, no rescale)",
                     "speedup_68": (t_mm + t_q) / online68_s, "speedup_24": (t_mm + t_q) / online24_s}
        except Exception as e:  # comparator unavailable on this stack
            dense = {"error": repr(e)[:200]}

    # engine clock while the product runs back to back (sysfs; None where it is not readable)
    sclk = None
    if not (args.kernels_only or args.no_clock):
        sclk = sample_sclk(lambda: steps_calls[0][names.index("spgemm_68")](), torch, seconds=0.3)

    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    suite_res = None
    if not (args.no_suite or args.kernels_only):
        del bufs
        torch.cuda.empty_cache()
        suite_res = suite(ss, torch, dev)

    cpu, parity = None, None
    if check_parity:
        y_ref, cpu = cpu_baseline(X_np, W_np, Kc68, Kc24)
        # INT8 path: every output of the benchmarked step must equal the oracle's bf16 bits
        parity = {k: {"bit_exact": bool(np.array_equal(y_gpu[k], y_ref[k])),
                      "mismatches": int(np.count_nonzero(y_gpu[k] != y_ref[k]))} for k in y_gpu}
        parity["checked"] = f"all {M}x{N} outputs of each product, bf16 bits against the oracle on the same inputs"

    out = {
        "metric": METRIC, "value": M / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": "6:8 sliding-window INT8 linear, W 4096x4096 -> K'=6144, X 2048x4096 bf16 "
                               "with 1% outlier channels; plus 2:4 on W and 2:4 on X of the same batch",
                   "M": M, "N": N, "K": K, "K_prime": Kc68, "global_batch": M, "parallelism": "none (1 GPU)"},
        "online_68_tokens_per_s": M / online68_s,
        "online_24_tokens_per_s": M / online24_s,
        "online_x_tokens_per_s": M / onlinex_s,
        "gemm_68_dense_equiv_TOPS": kernels["spgemm_68"]["dense_equiv_TOPS"],
        "gemm_24_dense_equiv_TOPS": kernels["spgemm_24"]["dense_equiv_TOPS"],
        "quant_lift_68_GBs": kernels["quant_lift_68"]["GB/s"],
        "dense_int8": dense,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "rotating_buffer_sets": NBUF,
        "sclk_MHz_during_spgemm_68": sclk,
        "per_call_sum_ms": sum(per_kernel_ms.values()),
        "suite": suite_res,
    }
    print(json.dumps(out))


def suite(ss, torch, dev, reps=10):
    """Layer-shaped products on synthetic data (seeded on the GPU): Llama-3.1-8B-shaped 2:4 FP8 weight
    GEMMs at M = 2048..16384 against dense FP8 (hipBLASLt through torch._scaled_mm, same per-token /
    per-channel scales) and in block-scaled FP8; Qwen2.5-7B-shaped 4:6 and 8:10 INT8 GEMMs at decode and prefill M; the
    sparse-activation FP8 layer; quant+lift bandwidth on a large batch and a plain device copy."""
    import synth
    print("[bench] layer suite", file=sys.stderr, flush=True)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261203)

    def randn(shape, std=1.0, dtype=torch.float32):
        return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std).to(dtype)

    def timed(fn, n=reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    res = {"data": "synthetic: W ~ N(0, 0.02^2) float32, X ~ N(0, 1) bf16, generated on the GPU (seeded)"}
    # Llama-3.1-8B-shaped 2:4 FP8 weight GEMMs
    llama = {}
    for M in (2048, 4096, 8192, 16384):
        rows, tot_sp, tot_dn = [], 0.0, 0.0
        for name, (K, Nout) in synth.LLAMA31_8B_LINEARS.items():
            W = randn((Nout, K), 0.02)
            wv, wm, sw = ss.prune24(W, "fp8")
            tv, tm = ss.pack_sparse(wv, wm)
            wq, swd = ss.quant_lift_act(W, 2, "fp8")
            del W, wv, wm
            X = randn((M, K), 1.0, torch.bfloat16)
            xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
            sx = torch.empty(M, dtype=torch.float32, device=dev)
            Y = torch.empty((M, Nout), dtype=torch.bfloat16, device=dev)
            t_q = timed(lambda: ss.quant_lift_act(X, 2, "fp8", out=(xq, sx)))
            t_sp = timed(lambda: ss.spgemm_tiled(ss.SS_SPARSE_W, M, Nout, K, tv, tm, xq, sx, sw, "bf16", out=Y))
            try:
                t_dn = timed(lambda: torch._scaled_mm(xq, wq.t(), scale_a=sx[:, None], scale_b=swd[None, :],
                                                      out_dtype=torch.bfloat16))
            except Exception:
                t_dn = None
            dense_eq = 2.0 * M * Nout * K
            rows.append({"layer": name, "K": K, "N": Nout, "quant_us": t_q, "sparse_gemm_us": t_sp,
                         "sparse_TOPS_dense_equiv": dense_eq / t_sp / 1e6,
                         "sparse_frac_of_10070": dense_eq / t_sp / 1e6 / 10070.0,
                         "dense_fp8_gemm_us": t_dn,
                         "dense_TFLOPS": None if t_dn is None else dense_eq / t_dn / 1e6})
            tot_sp += t_q + t_sp
            tot_dn += t_q + (t_dn if t_dn is not None else float("nan"))
            del tv, tm, wq, swd, X, xq, sx, Y
        llama[str(M)] = {"layers": rows, "sparse_tokens_per_s": M / (tot_sp * 1e-6),
                         "dense_tokens_per_s": M / (tot_dn * 1e-6), "speedup": tot_dn / tot_sp}
        torch.cuda.empty_cache()
    res["llama31_8b_24_fp8"] = llama
    # the same Llama-shaped 2:4 layers with block-scaled FP8 (LLM Compressor W8A8-FP8_BLOCK: 128 x 128 weight
    # blocks, per-token groups of 128): weight prep, group quant and the product with per-step promotion
    blk = {}
    for M in (4096, 8192):
        rows, tot = [], 0.0
        for name, (K, Nout) in synth.LLAMA31_8B_LINEARS.items():
            W = randn((Nout, K), 0.02)
            tv, tm, sw = ss.prune24_block(W)
            t_w = timed(lambda: ss.prune24_block(W, out=(tv, tm, sw)), n=3) if M == 4096 else None
            del W
            Kc = ss.lifted_k(K, 2)
            X = randn((M, K), 1.0, torch.bfloat16)
            xq = torch.empty((M, Kc), dtype=torch.float8_e4m3fn, device=dev)
            sx = torch.empty((M, Kc // 128), dtype=torch.float32, device=dev)
            Y = torch.empty((M, Nout), dtype=torch.bfloat16, device=dev)
            t_q = timed(lambda: ss.quant_group_act(X, out=(xq, sx)))
            t_sp = timed(lambda: ss.spgemm_tiled_block(M, Nout, Kc, tv, tm, xq, sx, sw, "bf16", out=Y))
            hw = 2.0 * M * Nout * Kc
            qbytes = 2 * M * K + M * Kc + 4 * M * (Kc // 128)
            row = {"layer": name, "K": K, "N": Nout, "quant_group_us": t_q, "quant_group_GBs": qbytes / t_q / 1e3,
                   "sparse_gemm_us": t_sp, "sparse_TOPS_dense_equiv": hw / t_sp / 1e6,
                   "sparse_frac_of_10070": hw / t_sp / 1e6 / 10070.0}
            if t_w is not None:
                wbytes = 4 * Nout * K + Nout * Kc // 2 + Nout * Kc // 8 + 4 * ((Nout + 127) // 128) * (Kc // 128)
                row.update({"prune24_block_us": t_w, "prune24_block_GBs": wbytes / t_w / 1e3})
            rows.append(row)
            tot += t_q + t_sp
            del tv, tm, sw, X, xq, sx, Y
        blk[str(M)] = {"layers": rows, "sparse_tokens_per_s": M / (tot * 1e-6),
                       "time_vs_per_channel_24_fp8": llama[str(M)]["sparse_tokens_per_s"] / (M / (tot * 1e-6))}
        torch.cuda.empty_cache()
    res["llama31_8b_24_fp8_block"] = blk
    # the same Llama-shaped layers with 6:8 (K' = 1.5 K) at M >= 4096, INT8 and FP8, against dense
    llama68 = {}
    for q in ("i8", "fp8"):
        for M in (4096, 8192):
            rows, tot_sp, tot_dn = [], 0.0, 0.0
            for name, (K, Nout) in synth.LLAMA31_8B_LINEARS.items():
                W = randn((Nout, K), 0.02)
                tv, tm, sw = ss.slide_decompose_tiled(W, 4, q)
                wq, swd = ss.quant_lift_act(W, 2, q)
                del W
                Kc = ss.lifted_k(K, 4)
                X = randn((M, K), 1.0, torch.bfloat16)
                qdt = torch.int8 if q == "i8" else torch.float8_e4m3fn
                xl = torch.empty((M, Kc), dtype=qdt, device=dev)
                xq = torch.empty((M, K), dtype=qdt, device=dev)
                sx = torch.empty(M, dtype=torch.float32, device=dev)
                sx2 = torch.empty(M, dtype=torch.float32, device=dev)
                Y = torch.empty((M, Nout), dtype=torch.bfloat16, device=dev)
                t_q = timed(lambda: ss.quant_lift_act(X, 4, q, out=(xl, sx)))
                t_sp = timed(lambda: ss.spgemm_tiled(ss.SS_SPARSE_W, M, Nout, Kc, tv, tm, xl, sx, sw, "bf16", out=Y))
                t_dq = timed(lambda: ss.quant_lift_act(X, 2, q, out=(xq, sx2)))
                try:
                    if q == "i8":
                        t_dn = timed(lambda: torch._int_mm(xq, wq.t()))
                    else:
                        t_dn = timed(lambda: torch._scaled_mm(xq, wq.t(), scale_a=sx2[:, None], scale_b=swd[None, :],
                                                              out_dtype=torch.bfloat16))
                except Exception:
                    t_dn = None
                hw = 2.0 * M * Nout * Kc
                rows.append({"layer": name, "K": K, "K_prime": Kc, "N": Nout, "quant_lift_us": t_q,
                             "sparse_gemm_us": t_sp, "sparse_TOPS_dense_equiv": hw / t_sp / 1e6,
                             "sparse_frac_of_10070": hw / t_sp / 1e6 / 10070.0,
                             "effective_TOPS": 2.0 * M * Nout * K / t_sp / 1e6,
                             "dense_quant_us": t_dq, "dense_gemm_us": t_dn})
                tot_sp += t_q + t_sp
                tot_dn += t_dq + (t_dn if t_dn is not None else float("nan"))
                del tv, tm, sw, wq, swd, X, xl, xq, sx, sx2, Y
            llama68[f"{q}_{M}"] = {"layers": rows, "sparse_tokens_per_s": M / (tot_sp * 1e-6),
                                   "dense_tokens_per_s": M / (tot_dn * 1e-6), "speedup": tot_dn / tot_sp,
                                   "dense_library": "hipBLASLt (torch._int_mm int32 out / torch._scaled_mm bf16 out)"}
            torch.cuda.empty_cache()
    res["llama31_8b_68"] = llama68
    # Qwen2.5-7B-shaped sliding-window INT8 GEMMs, decode and prefill token counts
    qwen = []
    for n in (3, 5):
        for name, (K, Nout) in synth.QWEN25_7B_LINEARS.items():
            W = randn((Nout, K), 0.02)
            wv, wm, sw = ss.slide_decompose(W, n, "i8")
            tv, tm = ss.pack_sparse(wv, wm)
            Kc = ss.lifted_k(K, n)
            del W, wv, wm
            for M in (1, 16, 64, 4096):
                X = randn((M, K), 1.0, torch.bfloat16)
                xq = torch.empty((M, Kc), dtype=torch.int8, device=dev)
                sx = torch.empty(M, dtype=torch.float32, device=dev)
                Y = torch.empty((M, Nout), dtype=torch.bfloat16, device=dev)
                need = ss.spgemm_tiled_workspace_bytes(ss.SS_SPARSE_W, M, Nout, Kc, "i8")
                ws = torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else False
                t_q = timed(lambda: ss.quant_lift_act(X, n, "i8", out=(xq, sx)))
                t_sp = timed(lambda: ss.spgemm_tiled(ss.SS_SPARSE_W, M, Nout, Kc, tv, tm, xq, sx, sw, "bf16", out=Y,
                                                     workspace=ws))
                wbytes = tv.numel() + tm.numel()
                row = {"pattern": f"{2 * n - 2}:{2 * n}", "layer": name, "M": M, "K": K, "K_prime": Kc,
                       "N": Nout, "quant_lift_us": t_q, "sparse_gemm_us": t_sp, "split_k_workspace_bytes": need,
                       "sparse_TOPS_dense_equiv": 2.0 * M * Nout * Kc / t_sp / 1e6,
                       "weight_stream_GBs": wbytes / t_sp / 1e3,
                       "tokens_per_s": M / ((t_q + t_sp) * 1e-6)}
                if M <= 64:  # decode: the quant+lift / product pair replayed from a HIP graph (no launch gaps)
                    graph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(graph):
                        ss.quant_lift_act(X, n, "i8", out=(xq, sx))
                        ss.spgemm_tiled(ss.SS_SPARSE_W, M, Nout, Kc, tv, tm, xq, sx, sw, "bf16", out=Y, workspace=ws)
                    t_g = timed(graph.replay)
                    row.update({"graph_pair_us": t_g, "graph_tokens_per_s": M / (t_g * 1e-6)})
                    del graph
                if M <= 4:  # the same layer in one launch: quant+lift inside the few-token product
                    t_f = timed(lambda: ss.quant_lift_spgemm_decode(X, n, tv, tm, sw, Nout, "i8", "bf16", out=Y))
                    row.update({"fused_us": t_f, "fused_tokens_per_s": M / (t_f * 1e-6),
                                "fused_weight_stream_GBs": wbytes / t_f / 1e3})
                qwen.append(row)
                del X, xq, sx, Y, ws
            del tv, tm
            torch.cuda.empty_cache()
    res["qwen25_7b_slide_int8"] = qwen
    # sparse-activation layer: X 8192x4096 pruned 2:4 online (FP8), dense W 4096x4096 FP8
    M, K, Nout = 8192, 4096, 4096
    X = randn((M, K), 1.0, torch.bfloat16)
    wq, swd = ss.quant_lift_act(randn((Nout, K), 0.02), 2, "fp8")
    sx = torch.empty(M, dtype=torch.float32, device=dev)
    nv, nm = ss.tiled_bytes(M, K)
    tv = torch.empty(nv, dtype=torch.uint8, device=dev)
    tm = torch.empty(nm, dtype=torch.uint8, device=dev)
    Y = torch.empty((M, Nout), dtype=torch.bfloat16, device=dev)
    xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    t_pr = timed(lambda: ss.prune24_act_tiled(X, "fp8", out=(tv, tm, sx)))
    t_sp = timed(lambda: ss.spgemm_tiled(ss.SS_SPARSE_X, M, Nout, K, tv, tm, wq, sx, swd, "bf16", out=Y))
    t_q = timed(lambda: ss.quant_lift_act(X, 2, "fp8", out=(xq, sx)))
    try:
        t_dn = timed(lambda: torch._scaled_mm(xq, wq.t(), scale_a=sx[:, None], scale_b=swd[None, :],
                                              out_dtype=torch.bfloat16))
    except Exception:
        t_dn = None
    res["sparse_activation_fp8"] = {
        "M": M, "K": K, "N": Nout, "prune24_act_tiled_us": t_pr, "sparse_gemm_us": t_sp,
        "sparse_TOPS_dense_equiv": 2.0 * M * Nout * K / t_sp / 1e6, "dense_quant_us": t_q,
        "dense_fp8_gemm_us": t_dn,
        "speedup_vs_dense": None if t_dn is None else (t_q + t_dn) / (t_pr + t_sp)}
    del X, wq, swd, sx, tv, tm, Y, xq
    torch.cuda.empty_cache()
    # the same layer in bf16 (no quantisation): online prune + pack + product against dense bf16 (hipBLASLt)
    X = randn((M, K), 1.0, torch.bfloat16)
    Wb = randn((Nout, K), 0.02, torch.bfloat16)
    nv, nm = ss.tiled_bytes(M, K, "bf16")
    tv = torch.empty(nv, dtype=torch.uint8, device=dev)
    tm = torch.empty(nm, dtype=torch.uint8, device=dev)
    Y = torch.empty((M, Nout), dtype=torch.bfloat16, device=dev)
    t_pr = timed(lambda: ss.prune24_act_tiled(X, "bf16", out=(tv, tm, None)))
    t_sp = timed(lambda: ss.spgemm_tiled(ss.SS_SPARSE_X, M, Nout, K, tv, tm, Wb, None, None, "bf16", out=Y))
    t_dn = timed(lambda: torch.matmul(X, Wb.t()))
    res["sparse_activation_bf16"] = {
        "M": M, "K": K, "N": Nout, "prune24_act_tiled_us": t_pr, "sparse_gemm_us": t_sp,
        "sparse_TFLOPS_dense_equiv": 2.0 * M * Nout * K / t_sp / 1e6,
        "sparse_frac_of_5030": 2.0 * M * Nout * K / t_sp / 1e6 / 5030.0, "dense_bf16_gemm_us": t_dn,
        "speedup_vs_dense": t_dn / (t_pr + t_sp)}
    del X, Wb, tv, tm, Y
    torch.cuda.empty_cache()
    # online 2:4 on the attention operand roles, bf16, one batched launch over 32 heads (Llama-3.1-8B: 32 heads
    # of 128) at 4096 tokens: S = Q K^T with Q pruned along the head dimension (K' = 128 padded to 256, the
    # product's step alignment), O = P V with the probabilities pruned along the keys; dense torch.bmm beside
    H, L, d = 32, 4096, 128
    Kq = ss.lifted_k(d, 2)
    Q = randn((H * L, d), 1.0, torch.bfloat16)
    Kp = torch.zeros((H, L, Kq), dtype=torch.bfloat16, device=dev)
    Kp[:, :, :d] = randn((H, L, d), 1.0, torch.bfloat16)
    nv, nm = ss.tiled_bytes(H * L, Kq, "bf16")
    tvq = torch.empty(nv, dtype=torch.uint8, device=dev)
    tmq = torch.empty(nm, dtype=torch.uint8, device=dev)
    S = torch.empty((H, L, L), dtype=torch.bfloat16, device=dev)
    t_pq = timed(lambda: ss.prune24_act_tiled(Q, "bf16", out=(tvq, tmq, None)))
    t_qk = timed(lambda: ss.spgemm_tiled_batched(ss.SS_SPARSE_X, H, L, L, Kq, tvq, tmq, Kp, None, None, "bf16", out=S))
    Qh, Kt = Q.view(H, L, d), Kp[:, :, :d].transpose(1, 2).contiguous()
    t_qk_dn = timed(lambda: torch.bmm(Qh, Kt))
    del Q, Kp, tvq, tmq, Qh, Kt
    P = torch.softmax(randn((H * L, L), 2.0), dim=1).to(torch.bfloat16)
    Vt = randn((H, d, L), 1.0, torch.bfloat16)
    nv, nm = ss.tiled_bytes(H * L, L, "bf16")
    tvp = torch.empty(nv, dtype=torch.uint8, device=dev)
    tmp = torch.empty(nm, dtype=torch.uint8, device=dev)
    O = torch.empty((H, L, d), dtype=torch.bfloat16, device=dev)
    t_pp = timed(lambda: ss.prune24_act_tiled(P, "bf16", out=(tvp, tmp, None)))
    t_pv = timed(lambda: ss.spgemm_tiled_batched(ss.SS_SPARSE_X, H, L, d, L, tvp, tmp, Vt, None, None, "bf16", out=O))
    Ph, V = P.view(H, L, L), Vt.transpose(1, 2).contiguous()
    t_pv_dn = timed(lambda: torch.bmm(Ph, V))
    fl = 2.0 * H * L * L * d
    res["attention_roles_bf16"] = {
        "heads": H, "tokens": L, "head_dim": d,
        "qk": {"prune_q_us": t_pq, "sparse_batched_us": t_qk, "dense_bmm_us": t_qk_dn,
               "sparse_TFLOPS_dense_equiv": 2.0 * H * L * L * Kq / t_qk / 1e6,
               "speedup_vs_dense": t_qk_dn / (t_pq + t_qk)},
        "pv": {"prune_p_us": t_pp, "sparse_batched_us": t_pv, "dense_bmm_us": t_pv_dn,
               "sparse_TFLOPS_dense_equiv": fl / t_pv / 1e6, "sparse_frac_of_5030": fl / t_pv / 1e6 / 5030.0,
               "speedup_vs_dense": t_pv_dn / (t_pp + t_pv), "product_speedup_vs_dense": t_pv_dn / t_pv}}
    del P, Vt, tvp, tmp, O, Ph, V, S
    torch.cuda.empty_cache()
    # quant+lift on a large batch (launch latency amortised) and a plain device copy
    ql = {}
    for n in (2, 4):
        M, K = 16384, 4096
        X = randn((M, K), 1.0, torch.bfloat16)
        Kc = ss.lifted_k(K, n)
        xq = torch.empty((M, Kc), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        t = timed(lambda: ss.quant_lift_act(X, n, "i8", out=(xq, sx)))
        byts = 2 * M * K + M * Kc + 4 * M
        ql[f"n{n}"] = {"M": M, "K": K, "K_prime": Kc, "us": t, "GB/s": byts / t / 1e3,
                       "frac_of_8000": byts / t / 1e3 / 8000.0}
        del X, xq, sx
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), n=5)
    ql["device_copy_1GiB_GBs"] = 2 * (1 << 30) / t / 1e3
    del src, dst
    torch.cuda.empty_cache()
    res["quant_lift_large_int8"] = ql
    return res


def read_sclk_mhz():
    """Current engine clock from the amdgpu sysfs DPM table (the level marked '*'), or None."""
    import glob
    import re
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path).read().splitlines():
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                    if m:
                        return int(m.group(1))
        except OSError:
            continue
    return None


def sample_sclk(launch, torch, seconds=0.3, period=0.002):
    """Launch `launch` back to back for `seconds` while a thread samples the engine clock."""
    import statistics
    import threading
    if read_sclk_mhz() is None:
        return {"error": "no readable pp_dpm_sclk"}
    samples, stop = [], threading.Event()

    def run():
        while not stop.is_set():
            v = read_sclk_mhz()
            if v is not None:
                samples.append(v)
            time.sleep(period)

    th = threading.Thread(target=run)
    launch()
    torch.cuda.synchronize()
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            launch()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return {"error": "no samples"}
    return {"samples": len(samples), "median": statistics.median(samples), "min": min(samples),
            "max": max(samples), "idle_after": read_sclk_mhz()}


def cpu_baseline(X_np, W_np, Kc68, Kc24):
    """The oracle, as it stands, on one whole step of the same batch."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        threads = 1
    print("[bench] CPU oracle: three full steps", file=sys.stderr, flush=True)

    outs = {}

    def one_step():
        t0 = time.perf_counter()
        w68 = oracle.slide_decompose(W_np, PAT, "i8")
        x68 = oracle.quant_lift_act(X_np, PAT, "i8")
        y68 = oracle.spgemm("W", w68[0], w68[1], x68[0], Kc68, "i8", x68[1], w68[2], "bf16")
        w24 = oracle.prune24(W_np, "i8")
        x24 = oracle.quant_lift_act(X_np, 2, "i8")
        y24 = oracle.spgemm("W", w24[0], w24[1], x24[0], Kc24, "i8", x24[1], w24[2], "bf16")
        xs = oracle.prune24_act(X_np, "i8")
        wq = oracle.quant_lift_act(W_np, 2, "i8")
        yx = oracle.spgemm("X", xs[0], xs[1], wq[0], Kc24, "i8", xs[2], wq[1], "bf16")
        dt = time.perf_counter() - t0
        outs.update(y68=y68, y24=y24, yx=yx)
        return dt

    times = sorted(one_step() for _ in range(3))
    t = times[1]
    return outs, {"value": M / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole step (the same 9 calls; the tiled layout is a GPU storage detail with no oracle "
                      f"counterpart, M={M} tokens), median of 3 runs: {t:.2f} s (runs {times[0]:.2f}-{times[2]:.2f} s); "
                      f"products in float64 BLAS ({threads} threads), element-wise steps single-threaded NumPy; "
                      f"host CPUs visible: {len(os.sched_getaffinity(0))}"}


if __name__ == "__main__":
    main()
