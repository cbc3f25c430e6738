"""Benchmark of the structured-sparse quantised linear path on one MI355X.

Headline workload: the four projection layers of one Llama-3.1-8B-shaped
decoder layer (qkv 4096->6144, o 4096->4096, gate_up 4096->28672, down
14336->4096) in 2:4 FP8-E4M3 with per-channel weight scales and dynamic
per-token activation scales, bf16 output, 16384 tokens (prefill). Weights are
W ~ N(0, 0.02^2), activations X ~ N(0, 1) in bf16, seeded on the GPU; no model
weight or dataset is involved.

A step is the online path of that layer: for each of the four linears the
per-token FP8 quantisation of its input (``ss_quant_lift_act``, n = 2) and the
sparse product with the rescale epilogue (``ss_spgemm_tiled``). The offline
weight preparation (2:4 prune or 6:8 decomposition straight into the
product's tiled layout) runs once per model, not per token; it is timed apart
and reported beside the headline. ``value`` = tokens per second of the step
(16384 tokens per step) from K steps launched back to back between one pair of
events; per-call times come from medians of 5 samples of at least 20 ms each,
over rotating buffer sets whose working set is at least twice the 256 MB
Infinity Cache.

The last stdout line is one compact JSON object (the headline, the roofline of
the dominant kernel, the CPU oracle baseline, parity on sampled outputs, and a
few summary figures of other rows). Every other row -- per-call times, the
6:8 layers, the M = 4096 layer, the Qwen2.5-7B-shaped 4:6 / 8:10 rows at
decode and prefill token counts against dense INT8, the online activation
prune, block-scaled FP8, the attention operand roles, quant+lift bandwidth --
goes to stderr (one JSON object per line) and to ``--detail`` (a JSON file).

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-suite] [--kernels-only]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse GEMM TOPS & prefill tokens/s (2:4, 6:8) vs dense; quant+lift GB/s"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
DENSE_PEAK_T = {"fp8": 5000.0, "i8": 5000.0, "bf16": 2500.0}  # dense MFMA, TFLOP/s (TOPS for INT8)
PEAK_UNIT = {"fp8": "TFLOP/s", "i8": "TOPS", "bf16": "TFLOP/s"}
MALL_BYTES = 256 << 20          # Infinity Cache
HEAD_M = 16384
LLAMA_LAYERS = 32               # decoder layers of Llama-3.1-8B (public model config)
QWEN_LAYERS = 28                # decoder layers of Qwen2.5-7B
NBUF = 3                        # rotating buffer sets of the headline layer


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--tokens", type=int, default=HEAD_M, help="tokens per step of the headline layer")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline and the parity check")
    p.add_argument("--no-suite", action="store_true", help="skip the rows beyond the headline")
    p.add_argument("--kernels-only", action="store_true",
                   help="only the timed headline steps (for counter runs); no comparators, suite or CPU leg")
    p.add_argument("--calib-copy", action="store_true",
                   help="end with three plain 256 MiB device copies (the reference for HBM byte counters)")
    p.add_argument("--cpu-tokens", type=int, default=256, help="tokens of the CPU oracle sample")
    p.add_argument("--cpu-channels", type=int, default=768, help="output channels per linear of the CPU sample")
    p.add_argument("--detail", default=os.path.join(ROOT, "gpurun_out", "bench_detail.json"),
                   help="where the full results go (JSON); empty to skip")
    return p.parse_args(argv)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def row(name, **kw):
    """One result row on stderr (one JSON object per line)."""
    d = {"row": name, **kw}
    log(json.dumps(d, default=_round))
    return d


def _round(x):
    return float(x)


def _sig6(o):
    """The final line's numbers to 6 significant digits (it stays one short line)."""
    if isinstance(o, float):
        return float(f"{o:.6g}")
    if isinstance(o, dict):
        return {k: _sig6(v) for k, v in o.items()}
    if isinstance(o, (list, tuple)):
        return [_sig6(v) for v in o]
    return o


def traffic_record(kernel):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
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


def tiled_bytes(rows, Kc, es=1):
    """Bytes of the tiled operand (values, metadata) as include/ss.h defines them (es = value bytes)."""
    g = -(-(Kc * es // 128) // 4)
    rb = -(-rows // 16)
    return rb * g * 4 * 1024, rb * g * 256 * (4 // es)


def product_ops(M, N, Kc):
    """Operations of one sparse product: multiply-adds on the kept values only (K'/2 per row), x2. Priced
    against the dense matrix-core peak this is the same fraction as the dense-equivalent count 2 M N K'
    against the sparse peak."""
    return 2 * M * N * (Kc // 2)


def quant_bytes(M, K, Kc, code_bytes=1):
    """Algorithmic bytes of quant(+lift): bf16 rows read once, codes and one scale per token written."""
    return 2 * M * K + code_bytes * M * Kc + 4 * M


def prep_bytes(N, K, Kc, es=1):
    """Algorithmic bytes of weight prep into the tiled layout: float32 W read once, operand + scales written."""
    return 4 * N * K + sum(tiled_bytes(N, Kc, es)) + 4 * N


def median_us(torch, fns, min_ms=20.0, samples=5):
    """Per-call time (us): the median of ``samples`` samples, each running the callables of ``fns`` round robin
    (one per rotating buffer set) enough times to last at least ``min_ms``, between one pair of events on the
    launch stream (torch's current stream)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for f in fns:
        f()
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    for f in fns:
        f()
    e1.record()
    torch.cuda.synchronize()
    est = max(e0.elapsed_time(e1) / len(fns), 1e-3)
    reps = len(fns) * max(1, math.ceil(min_ms / est / len(fns)))
    out = []
    for _ in range(samples):
        e0.record()
        for i in range(reps):
            fns[i % len(fns)]()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / reps * 1e3)
    return statistics.median(out)


def median_us_graph(torch, fns, calls=256, min_ms=20.0, samples=5):
    """Per-call time (us) with the host out of the loop: ``calls`` calls (round robin over ``fns``) captured
    once in a HIP graph, replayed back to back; the median of ``samples`` samples of at least ``min_ms``. For
    calls of a few microseconds, where launching through Python takes longer than the kernel. The graph's
    first replay is compared with the eager result by the caller (see graph_check)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fns[i % len(fns)]()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(min_ms / max(e0.elapsed_time(e1), 1e-3)))
    out = []
    for _ in range(samples):
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / (reps * calls) * 1e3)
    del g
    return statistics.median(out)


def rotation(nbytes, floor=2 * MALL_BYTES, cap=64):
    """Buffer copies so that ``nbytes`` per copy add up to at least ``floor`` bytes (twice the Infinity Cache:
    a row whose working set fits the cache would time the cache, not HBM)."""
    return max(1, min(cap, math.ceil(floor / max(nbytes, 1))))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ------------------------------------------------------------------------------------------------------------
# the Llama-shaped layer


class Layer:
    """The four Llama-3.1-8B-shaped linears on the GPU: float32 W, the prepared sparse operand (tiled layout),
    dense per-channel codes for the comparator, and ``nbuf`` sets of activations, codes and outputs."""

    def __init__(self, ss, torch, dev, gen, M, n, q, nbuf, dense=True, keep_w=False):
        import synth
        self.ss, self.torch, self.M, self.n, self.q = ss, torch, M, n, q
        qdt = torch.int8 if q == "i8" else torch.float8_e4m3fn
        self.lin = {}
        for name, (K, N) in synth.LLAMA31_8B_LINEARS.items():
            W = torch.randn((N, K), generator=gen, device=dev) * 0.02
            Kc = ss.lifted_k(K, n)
            tv, tm, sw = ss.slide_decompose_tiled(W, n, q)
            L = dict(K=K, N=N, Kc=Kc, tv=tv, tm=tm, sw=sw, W=W if keep_w else None)
            if dense:
                L["wq"], L["swd"] = ss.quant_lift_act(W, 2, q)
            del W
            X = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
            sets = []
            for i in range(nbuf):
                s = dict(X=X if i == 0 else X.clone(), xq=torch.empty((M, Kc), dtype=qdt, device=dev),
                         sx=torch.empty(M, dtype=torch.float32, device=dev),
                         Y=torch.empty((M, N), dtype=torch.bfloat16, device=dev))
                if dense and n != 2:  # the dense comparator quantises without the lift
                    s["xd"] = torch.empty((M, K), dtype=qdt, device=dev)
                    s["sxd"] = torch.empty(M, dtype=torch.float32, device=dev)
                sets.append(s)
            L["sets"] = sets
            self.lin[name] = L
        self.nbuf = nbuf

    def quant(self, name, b):
        L, s = self.lin[name], self.lin[name]["sets"][b]
        return lambda: self.ss.quant_lift_act(s["X"], self.n, self.q, out=(s["xq"], s["sx"]))

    def gemm(self, name, b):
        L, s = self.lin[name], self.lin[name]["sets"][b]
        ss = self.ss
        return lambda: ss.spgemm_tiled(ss.SS_SPARSE_W, self.M, L["N"], L["Kc"], L["tv"], L["tm"], s["xq"], s["sx"],
                                       L["sw"], "bf16", out=s["Y"], workspace=False)

    def calls(self, b):
        """The step on buffer set b: (name, callable) in launch order."""
        out = []
        for name in self.lin:
            out.append((f"quant_{name}", self.quant(name, b)))
            out.append((f"gemm_{name}", self.gemm(name, b)))
        return out

    def dense_calls(self, b):
        """The same layer dense: per-token quantisation (no lift) + hipBLASLt (torch._scaled_mm with the same
        per-token x per-channel scales, bf16 out; INT8: torch._int_mm, int32 out and no rescale)."""
        torch, ss = self.torch, self.ss
        out = []
        for name, L in self.lin.items():
            s = L["sets"][b]
            if self.n == 2:
                xq, sx = s["xq"], s["sx"]
                out.append((f"quant_{name}", self.quant(name, b)))
            else:
                xq, sx = s["xd"], s["sxd"]
                out.append((f"quant_{name}", lambda s=s: ss.quant_lift_act(s["X"], 2, self.q, out=(s["xd"], s["sxd"]))))
            wq, swd = L["wq"], L["swd"]
            if self.q == "i8":
                out.append((f"gemm_{name}", lambda xq=xq, wq=wq: torch._int_mm(xq, wq.t())))
            else:
                out.append((f"gemm_{name}", lambda xq=xq, wq=wq, sx=sx, swd=swd: torch._scaled_mm(
                    xq, wq.t(), scale_a=sx[:, None], scale_b=swd[None, :], out_dtype=torch.bfloat16)))
        return out


def time_steps(torch, layer_calls, steps, warmup, mark=None):
    """K steps launched back to back (rotating buffer sets) between one pair of events, after W warm-up
    steps; ``mark`` names one call whose launches are also bracketed by events inside the timed region.
    Returns (ms per step, average ms of the marked call or None)."""
    nb = len(layer_calls)
    for s in range(warmup):
        for _, c in layer_calls[s % nb]:
            c()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    marks = [(ev(), ev()) for _ in range(steps)] if mark else None
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()
    e0.record()
    for s in range(steps):
        for name, c in layer_calls[s % nb]:
            if marks and name == mark:
                marks[s][0].record()
                c()
                marks[s][1].record()
            else:
                c()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    mk = statistics.fmean(a.elapsed_time(b) for a, b in marks) if marks else None
    return ms, mk


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


def sample_sclk(fns, torch, seconds=0.3, period=0.002):
    """Run the callables ``fns`` round robin, back to back, for ``seconds`` while a thread samples the engine
    clock; the median, range and sample count of the DPM level (None where the table is not readable)."""
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

    for f in fns:
        f()
    torch.cuda.synchronize()
    th = threading.Thread(target=run)
    th.start()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fns[i % len(fns)]()
            i += 1
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return {"error": "no samples"}
    return {"samples": len(samples), "median": statistics.median(samples), "min": min(samples),
            "max": max(samples), "idle_after": read_sclk_mhz()}


def per_call(torch, layer_calls):
    """Median per-call us of every call of the step, each over the rotating buffer sets."""
    names = [n for n, _ in layer_calls[0]]
    return {n: median_us(torch, [dict(c)[n] for c in layer_calls]) for n in names}


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU (this build runs on one); run with --gpus 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    import structured_sparse_quantized_amd as ss

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261203)
    M = args.tokens
    detail = {"data": "synthetic: W ~ N(0, 0.02^2) float32, X ~ N(0, 1) bf16, generated on the GPU (seeded)"}

    # ---- headline: the Llama-shaped layer, 2:4 FP8, M tokens ----
    log(f"[bench] headline layer: 2:4 FP8, {M} tokens, {NBUF} buffer sets")
    lay = Layer(ss, torch, dev, gen, M, 2, "fp8", NBUF, dense=not args.kernels_only, keep_w=not args.kernels_only)
    steps_calls = [lay.calls(b) for b in range(NBUF)]
    ms_step, ms_gate = time_steps(torch, steps_calls, args.steps, args.warmup, mark="gemm_gate_up")
    log(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step; gate_up product {ms_gate * 1e3:.1f} us (live)")
    gu = lay.lin["gate_up"]
    gu_ops = product_ops(M, gu["N"], gu["Kc"])
    roof = {"bound": "mfma", "achieved": gu_ops / (ms_gate * 1e-3) / 1e12, "peak": DENSE_PEAK_T["fp8"],
            "unit": PEAK_UNIT["fp8"]}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_record(f"gemm_gate_up_{M}")
    roof["kernel"] = f"gate_up product {M}x28672x4096, 2:4 FP8 ({'256x256 wide' if M >= 2304 else '256x128 or decode'} kernel)"
    out = {
        "metric": METRIC, "value": M / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
        "config": {"workload": f"Llama-3.1-8B-shaped layer linears qkv+o+gate_up+down, 2:4 FP8-e4m3 W per-channel, "
                               f"dynamic per-token FP8 X, bf16 out, {M} tokens (online quant + sparse GEMM)",
                   "tokens": M, "global_batch": M, "parallelism": "none (1 GPU)"},
        "model_tokens_per_s": M / (ms_step * 1e-3) / LLAMA_LAYERS,
        "roofline": roof,
    }
    if args.kernels_only:
        if args.calib_copy:
            calib_copy(torch, dev)
        print(json.dumps(out, default=_round))
        return

    pc = per_call(torch, steps_calls)
    calls = {}
    for name, L in lay.lin.items():
        tq, tg = pc[f"quant_{name}"], pc[f"gemm_{name}"]
        ops = product_ops(M, L["N"], L["Kc"])
        qb = quant_bytes(M, L["K"], L["Kc"])
        calls[name] = {"quant_us": tq, "quant_GBs": qb / tq / 1e3, "quant_frac": qb / tq / 1e3 / HBM_PEAK_GBS,
                       "gemm_us": tg, "gemm_TFLOPs": ops / tg / 1e6, "gemm_frac": ops / tg / 1e6 / DENSE_PEAK_T["fp8"]}
    detail["headline_per_call"] = row("headline_per_call", tokens=M, rotating_sets=NBUF, calls=calls)
    # engine clock while the dominant product runs back to back
    sclk = sample_sclk([dict(c)["gemm_gate_up"] for c in steps_calls], torch)
    detail["sclk_gate_up"] = row("sclk_gate_up", **sclk)
    # dense FP8 comparator on the same buffers
    dense_calls = [lay.dense_calls(b) for b in range(NBUF)]
    try:
        ms_dense, _ = time_steps(torch, dense_calls, args.steps, args.warmup)
        pcd = per_call(torch, dense_calls)
    except Exception as e:  # noqa: BLE001 -- the comparator library may be missing on a stack
        ms_dense, pcd = None, {"error": repr(e)[:200]}
    detail["headline_dense"] = row("headline_dense_fp8", ms_per_step=ms_dense, per_call_us=pcd,
                                   library="hipBLASLt via torch._scaled_mm (bf16 out, same scales)")
    # offline weight preparation of the layer (2:4 prune + FP8 codes into the tiled layout), per call
    prep = {}
    for name, L in lay.lin.items():
        W = L["W"]
        bufs = [(torch.empty_like(L["tv"]), torch.empty_like(L["tm"]), torch.empty_like(L["sw"]))
                for _ in range(rotation(W.numel() * 4))]
        t = median_us(torch, [lambda o=o: ss.slide_decompose_tiled(W, 2, "fp8", out=o) for o in bufs])
        b = prep_bytes(L["N"], L["K"], L["Kc"])
        prep[name] = {"us": t, "GBs": b / t / 1e3, "frac": b / t / 1e3 / HBM_PEAK_GBS}
        del bufs
    detail["weight_prep_24_fp8"] = row("weight_prep_24_fp8", per_linear=prep)

    parity, cpu = None, None
    if not args.no_cpu:
        parity, cpu = cpu_leg(torch, lay, M, args.cpu_tokens, args.cpu_channels)
        detail["parity_vs_oracle"] = row("parity_vs_oracle", **parity)
    out.update({
        "vs_dense": None if ms_dense is None else ms_dense / ms_step,
        "gemm_frac": {k: round(v["gemm_frac"], 3) for k, v in calls.items()},
        "quant_GBs": round(calls["qkv"]["quant_GBs"], 1),
        "sclk_MHz_gate_up": sclk.get("median"),
        "weight_prep_us": round(sum(v["us"] for v in prep.values()), 1),
    })
    del lay, steps_calls, dense_calls
    torch.cuda.empty_cache()

    # ---- the same layer at 4096 tokens, and with 6:8 (INT8 and FP8) ----
    if not args.no_suite:
        extra = layer_rows(ss, torch, dev, gen, args, detail)
        out.update(extra)
        suite(ss, torch, dev, gen, detail, check=not args.no_cpu)
    out["cpu_baseline"] = cpu
    out["parity_vs_oracle"] = None if parity is None else {
        k: parity[k] for k in ("ok", "codes_bit_exact", "max_rel_fro", "max_elem_over_bound", "sample")}
    if parity is not None:
        checked = _parity_checks({k: v for k, v in detail.items() if k != "parity_vs_oracle"})
        out["parity_vs_oracle"]["other_rows"] = f"{sum(checked)} of {len(checked)} sampled checks ok"
    if args.detail:
        try:
            os.makedirs(os.path.dirname(args.detail), exist_ok=True)
            detail["line"] = out
            with open(args.detail, "w") as f:
                json.dump(detail, f, indent=1, default=_round)
            out["detail"] = os.path.relpath(args.detail, ROOT)
        except OSError:
            pass
    if args.calib_copy:
        calib_copy(torch, dev)
    print(json.dumps(_sig6(out), default=_round, separators=(",", ":")))


def calib_copy(torch, dev):
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def layer_rows(ss, torch, dev, gen, args, detail):
    """The 2:4 FP8 layer at 4096 tokens and the 6:8 layers (INT8, FP8) at 4096 tokens, each against dense;
    returns the summary fields of the last line."""
    res = {}
    for (n, q, M) in ((2, "fp8", 4096), (4, "i8", 4096), (4, "fp8", 4096), (4, "i8", 16384), (4, "fp8", 16384)):
        log(f"[bench] layer n={n} {q} M={M}")
        lay = Layer(ss, torch, dev, gen, M, n, q, NBUF, keep_w=not args.no_cpu)
        sc = [lay.calls(b) for b in range(NBUF)]
        dc = [lay.dense_calls(b) for b in range(NBUF)]
        ms, _ = time_steps(torch, sc, args.steps, 2)
        try:
            msd, _ = time_steps(torch, dc, args.steps, 2)
        except Exception:  # noqa: BLE001
            msd = None
        pc = per_call(torch, sc)
        fr = {name: product_ops(M, L["N"], L["Kc"]) / pc[f"gemm_{name}"] / 1e6 / DENSE_PEAK_T[q]
              for name, L in lay.lin.items()}
        speed = None if msd is None else msd / ms
        theo = n / (n - 1)
        key = f"{'24' if n == 2 else '68'}_{q}_{M}"
        par = None if args.no_cpu else layer_parity(torch, lay, n, q)
        detail[f"layer_{key}"] = row(f"layer_{key}", pattern="2:4" if n == 2 else "6:8", q=q, tokens=M,
                                     ms_per_step=ms, dense_ms_per_step=msd, tokens_per_s=M / (ms * 1e-3),
                                     vs_dense=speed, efficiency=None if speed is None else speed / theo,
                                     per_call_us=pc, gemm_frac=fr, parity_vs_oracle=par,
                                     dense_library="torch._int_mm (int32 out, no rescale)" if q == "i8" else
                                     "torch._scaled_mm (bf16 out)")
        res[f"l{key}"] = {"tps": round(M / (ms * 1e-3)), "vs_dense": None if speed is None else round(speed, 3),
                          "gemm_frac_max": round(max(fr.values()), 3),
                          "parity": None if par is None else all(v["ok"] for v in par.values())}
        del lay, sc, dc
        torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------------------------------------
# CPU oracle baseline and parity on sampled outputs


def cpu_leg(torch, lay, M, n_tok, n_ch, seed=7):
    """The oracle, as it stands, on a sample of the headline layer: ``n_tok`` tokens through all four linears'
    quantisation and ``n_ch`` output channels of each product (first and last 128 channels plus random ones,
    so tile edges are covered). The same sample checks the GPU's codes, scales and outputs of the timed steps:
    codes and scales bit for bit, products against the oracle's exact float64 sums within 1e-2 relative
    Frobenius error and element by element within 4e-5 sum|terms| + 2^-7 |y| (the matrix core's FP8 sum
    precision, then one bf16 rounding step)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = 1
    log(f"[bench] CPU oracle on {n_tok} tokens x {n_ch} channels per linear")
    rng = np.random.default_rng(seed)
    toks = np.unique(np.concatenate([[0, M - 1], rng.choice(M, n_tok - 2, replace=False)]))
    per_token_s, prep_s = 0.0, 0.0
    ok, codes_ok, worst_fro, worst_elem = True, True, 0.0, 0.0
    tok_d = torch.from_numpy(toks).to(lay.lin["qkv"]["sw"].device)
    for name, L in lay.lin.items():
        N, K, Kc = L["N"], L["K"], L["Kc"]
        chans = np.unique(np.concatenate([np.arange(128), np.arange(N - 128, N),
                                          rng.choice(N, max(n_ch - 256, 0), replace=False)]))
        ch_d = torch.from_numpy(chans).to(tok_d.device)
        s = L["sets"][0]
        Wh = L["W"].index_select(0, ch_d).cpu().numpy()
        Xh = s["X"].index_select(0, tok_d).view(torch.int16).cpu().numpy().view(np.uint16)
        yg = s["Y"].index_select(0, tok_d).index_select(1, ch_d).view(torch.int16).cpu().numpy().view(np.uint16)
        xq_g = s["xq"].index_select(0, tok_d).view(torch.uint8).cpu().numpy()
        sx_g = s["sx"].index_select(0, tok_d).cpu().numpy()
        sw_g = L["sw"].index_select(0, ch_d).cpu().numpy()
        t0 = time.perf_counter()
        ow = oracle.prune24(Wh, "fp8")  # offline weight prep of the sampled channels (not in the rate)
        prep_s += time.perf_counter() - t0
        t0 = time.perf_counter()
        ox = oracle.quant_lift_act(Xh, 2, "fp8")
        t_q = time.perf_counter() - t0
        t0 = time.perf_counter()
        y = oracle.spgemm("W", ow[0], ow[1], ox[0], Kc, "fp8", ox[1], ow[2], "bf16")
        t_p = time.perf_counter() - t0
        per_token_s += t_q / len(toks) + t_p / len(toks) * N / len(chans)
        codes_ok &= bool(np.array_equal(xq_g, ox[0]) and np.array_equal(sx_g, ox[1]) and np.array_equal(sw_g, ow[2]))
        # products: sum of |terms| for the element-wise bound
        a = np.abs(oracle.decompress24(oracle.e4m3_decode(ow[0])[:, : Kc // 2], ow[1], Kc))
        b = np.abs(oracle.e4m3_decode(ox[0]))[:, :Kc]
        terms = (b @ a.T) * ox[1].astype(np.float64)[:, None] * ow[2].astype(np.float64)[None, :]
        yr, yv = _bf16(y), _bf16(yg)
        den = np.linalg.norm(yr)
        fro = float(np.linalg.norm(yv - yr) / (den if den > 0 else 1.0))
        bound = 4e-5 * terms + 2.0 ** -7 * np.abs(yr)
        elem = float(np.max(np.abs(yv - yr) / np.maximum(bound, 1e-30)))
        worst_fro, worst_elem = max(worst_fro, fro), max(worst_elem, elem)
        ok &= fro <= 1e-2 and elem <= 1.0
    ok &= codes_ok
    parity = {"ok": bool(ok), "codes_bit_exact": bool(codes_ok), "max_rel_fro": worst_fro,
              "max_elem_over_bound": worst_elem,
              "sample": f"{len(toks)} tokens x >= {n_ch} channels per linear, set 0 of the timed steps"}
    cpu = {"value": 1.0 / per_token_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "cpu": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
           "sample": f"{len(toks)} tokens, four linears: FP8 quant of all K, product over >= {n_ch} channels "
                     f"of each (scaled to all); float64 BLAS on {threads} threads; weight prep ({prep_s:.1f} s) "
                     f"not counted"}
    log(f"[bench] CPU oracle: {cpu['value']:.1f} tokens/s; parity {parity}")
    return parity, cpu


def sampled_parity(side, n, q, Kc, w_rows, x_rows, y_gpu, sx_gpu=None, sw_gpu=None, xq_gpu=None):
    """The oracle on one benchmark row's own inputs, on a sample: ``w_rows`` the sampled output channels' float32
    weights, ``x_rows`` the sampled tokens' bf16 bits, ``y_gpu`` the GPU's bf16 outputs at [tokens, channels],
    and (when given) the GPU's scales and codes of the same rows. Side "W": weights pruned (2:4, or the
    (2n-2):2n decomposition) and tokens quantised (+ lifted); side "X": tokens pruned 2:4 online, weights
    quantised per channel. Scales and codes bit for bit; the product INT8 bit for bit, FP8 within 1e-2 relative
    Frobenius error and element by element within 4e-5 sum|terms| + 2^-7 |y|."""
    import numpy as np
    import oracle
    if side == "W":
        ow = oracle.prune24(w_rows, q) if n == 2 else oracle.slide_decompose(w_rows, n, q)
        ox = oracle.quant_lift_act(x_rows, n, q)
        sp_v, sp_m, dense, s_sp, s_dn = ow[0], ow[1], ox[0], ow[2], ox[1]
        y = oracle.spgemm("W", ow[0], ow[1], ox[0], Kc, q, ox[1], ow[2], "bf16")
        codes = [(sx_gpu, ox[1]), (sw_gpu, ow[2]), (xq_gpu, None if xq_gpu is None else ox[0])]
    else:
        ox = oracle.prune24_act(x_rows, q)
        ow = oracle.quant_lift_act(w_rows, 2, q)
        sp_v, sp_m, dense, s_sp, s_dn = ox[0], ox[1], ow[0], ox[2], ow[1]
        y = oracle.spgemm("X", ox[0], ox[1], ow[0], Kc, q, ox[2], ow[1], "bf16")
        codes = [(sx_gpu, ox[2]), (sw_gpu, ow[1])]
    codes_ok = True
    for g, e in codes:
        if g is None:
            continue
        g, e = np.asarray(g), np.asarray(e)
        codes_ok &= bool(np.array_equal(g, e) if g.dtype == np.float32 else np.array_equal(g.view(np.uint8),
                                                                                             e.view(np.uint8)))
    yr, yv = _bf16(y), _bf16(y_gpu)
    if q == "i8":
        exact = bool(np.array_equal(np.asarray(y_gpu, np.uint16), np.asarray(y, np.uint16)))
        return {"ok": bool(codes_ok and exact), "codes_bit_exact": bool(codes_ok), "product_bit_exact": exact,
                "sample": f"{yr.shape[0]} tokens x {yr.shape[1]} channels"}
    dec = oracle.e4m3_decode
    a = np.abs(oracle.decompress24(dec(sp_v)[:, : Kc // 2], sp_m, Kc))
    b = np.abs(dec(dense))[:, :Kc]
    terms = (b @ a.T) * np.asarray(s_dn, np.float64)[:, None] * np.asarray(s_sp, np.float64)[None, :]
    if side == "X":
        terms = terms.T
    den = np.linalg.norm(yr)
    fro = float(np.linalg.norm(yv - yr) / (den if den > 0 else 1.0))
    elem = float(np.max(np.abs(yv - yr) / np.maximum(4e-5 * terms + 2.0 ** -7 * np.abs(yr), 1e-30)))
    return {"ok": bool(codes_ok and fro <= 1e-2 and elem <= 1.0), "codes_bit_exact": bool(codes_ok),
            "max_rel_fro": fro, "max_elem_over_bound": elem, "sample": f"{yr.shape[0]} tokens x {yr.shape[1]} channels"}


def _parity_checks(o):
    """The ``ok`` of every sampled_parity result in the detail record (the headline's own is in cpu_leg)."""
    found = []
    if isinstance(o, dict):
        for k, v in o.items():
            if k == "parity_vs_oracle" and isinstance(v, dict):
                found += [v["ok"]] if "ok" in v else [x["ok"] for x in v.values()]
            elif k != "parity_vs_oracle":
                found += _parity_checks(v)
    elif isinstance(o, list):
        for v in o:
            found += _parity_checks(v)
    return found


def _pick(N, k, rng, edge=64):
    """Sampled indices: the first and last ``edge`` (tile edges, the ragged end) and ``k`` random ones."""
    import numpy as np
    if N <= 2 * edge + k:
        return np.arange(N)
    mid = rng.choice(np.arange(edge, N - edge), k, replace=False)
    return np.unique(np.concatenate([np.arange(edge), np.arange(N - edge, N), mid]))


def layer_parity(torch, lay, n, q, seed=11):
    """sampled_parity on each linear of a Layer (set 0 of its timed steps)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = {}
    for name, L in lay.lin.items():
        s = L["sets"][0]
        toks = _pick(lay.M, 16, rng, edge=8)
        chans = _pick(L["N"], 64, rng)
        td = torch.from_numpy(toks).to(s["X"].device)
        cd = torch.from_numpy(chans).to(s["X"].device)
        out[name] = sampled_parity(
            "W", n, q, L["Kc"], L["W"].index_select(0, cd).cpu().numpy(),
            s["X"].index_select(0, td).view(torch.int16).cpu().numpy().view(np.uint16),
            s["Y"].index_select(0, td).index_select(1, cd).view(torch.int16).cpu().numpy().view(np.uint16),
            s["sx"].index_select(0, td).cpu().numpy(), L["sw"].index_select(0, cd).cpu().numpy(),
            s["xq"].index_select(0, td).view(torch.uint8).cpu().numpy())
    return out


def _bf16(bits):
    import numpy as np
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------------------------------------------------
# the other rows


def suite(ss, torch, dev, gen, detail, check=True):
    """Rows beyond the Llama layers (stderr + detail file); with ``check``, the Qwen-shaped and sparse-activation
    rows also carry sampled_parity on their own inputs."""
    import numpy as np
    import synth
    rng = np.random.default_rng(13)

    def randn(shape, std=1.0, dtype=torch.float32):
        return (torch.randn(shape, generator=gen, device=dev) * std).to(dtype)

    # Qwen2.5-7B-shaped 4:6 and 8:10 INT8 linears at decode and prefill token counts, against dense INT8
    qwen = []
    for n in (3, 5):
        tot = {}
        for name, (K, Nout) in synth.QWEN25_7B_LINEARS.items():
            W = randn((Nout, K), 0.02)
            tv, tm, sw = ss.slide_decompose_tiled(W, n, "i8")
            wq, swd = ss.quant_lift_act(W, 2, "i8")
            chans = _pick(Nout, 64, rng)
            cd = torch.from_numpy(chans).to(dev)
            Wh = W.index_select(0, cd).cpu().numpy() if check else None
            del W
            Kc = ss.lifted_k(K, n)
            wbytes = tv.numel() + tm.numel() + 4 * Nout
            nrot = rotation(wbytes)  # weight copies so decode streams them from HBM, not the Infinity Cache
            ops = [(tv, tm, sw)] + [(tv.clone(), tm.clone(), sw.clone()) for _ in range(nrot - 1)]
            dops = [wq] + [wq.clone() for _ in range(rotation(wq.numel()) - 1)]
            for M in (1, 16, 64, 4096):
                X = randn((M, K), 1.0, torch.bfloat16)
                xq = torch.empty((M, Kc), dtype=torch.int8, device=dev)
                xd = torch.empty((M, K), dtype=torch.int8, device=dev)
                sx = torch.empty(M, dtype=torch.float32, device=dev)
                sxd = torch.empty(M, dtype=torch.float32, device=dev)
                Y = torch.empty((M, Nout), dtype=torch.bfloat16, device=dev)
                need = ss.spgemm_tiled_workspace_bytes(ss.SS_SPARSE_W, M, Nout, Kc, "i8")
                ws = torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else False
                t_q = median_us(torch, [lambda: ss.quant_lift_act(X, n, "i8", out=(xq, sx))])
                spf = [lambda o=o: ss.spgemm_tiled(ss.SS_SPARSE_W, M, Nout, Kc, o[0], o[1], xq, sx, o[2], "bf16", out=Y,
                                                   workspace=ws) for o in ops]
                t_sp = median_us(torch, spf)
                gr = {}
                if M <= 64:  # few tokens: the kernels run for microseconds, so time them without the host too
                    yref = Y.clone()
                    gr["quant_lift_graph_us"] = median_us_graph(torch, [lambda: ss.quant_lift_act(X, n, "i8", out=(xq, sx))])
                    gr["sparse_gemm_graph_us"] = median_us_graph(torch, spf)
                    gr["graph_equals_eager"] = bool(torch.equal(Y.view(torch.int16), yref.view(torch.int16)))
                    gr["weight_stream_graph_GBs"] = wbytes / gr["sparse_gemm_graph_us"] / 1e3
                t_dq = median_us(torch, [lambda: ss.quant_lift_act(X, 2, "i8", out=(xd, sxd))])
                r = {"pattern": f"{2 * n - 2}:{2 * n}", "layer": name, "M": M, "K": K, "K_prime": Kc, "N": Nout,
                     "quant_lift_us": t_q, "sparse_gemm_us": t_sp, "weight_copies": nrot,
                     "sparse_TOPS_dense_equiv": 2.0 * M * Nout * Kc / t_sp / 1e6,
                     "weight_stream_GBs": wbytes / t_sp / 1e3, "dense_quant_us": t_dq, **gr}
                if M > 16:  # hipBLASLt int8 needs M > 16 through torch._int_mm
                    try:
                        t_dn = median_us(torch, [lambda d=d: torch._int_mm(xd, d.t()) for d in dops])
                    except Exception as e:  # noqa: BLE001
                        t_dn, r["dense_error"] = None, repr(e)[:120]
                else:
                    t_dn = None
                    r["dense"] = "not measured: torch._int_mm (hipBLASLt int8) requires more than 16 rows"
                if t_dn is not None:
                    sp = (t_dq + t_dn) / (t_q + t_sp)
                    r.update({"dense_gemm_us": t_dn, "vs_dense": sp, "efficiency": sp / (n / (n - 1)),
                              "gemm_vs_dense": t_dn / t_sp})
                if check:
                    td = torch.from_numpy(_pick(M, 16, rng, edge=8)).to(dev)
                    r["parity_vs_oracle"] = sampled_parity(
                        "W", n, "i8", Kc, Wh, X.index_select(0, td).view(torch.int16).cpu().numpy().view(np.uint16),
                        Y.index_select(0, td).index_select(1, cd).view(torch.int16).cpu().numpy().view(np.uint16),
                        sx.index_select(0, td).cpu().numpy(), sw.index_select(0, cd).cpu().numpy(),
                        xq.index_select(0, td).view(torch.uint8).cpu().numpy())
                if M <= 4:  # the same layer in one launch: quant+lift inside the few-token product
                    ff = [lambda o=o: ss.quant_lift_spgemm_decode(X, n, o[0], o[1], o[2], Nout, "i8", "bf16", out=Y)
                          for o in ops]
                    t_f = median_us(torch, ff)
                    t_fg = median_us_graph(torch, ff)
                    r.update({"fused_us": t_f, "fused_weight_stream_GBs": wbytes / t_f / 1e3, "fused_graph_us": t_fg,
                              "fused_weight_stream_graph_GBs": wbytes / t_fg / 1e3})
                tot.setdefault(M, [0.0, 0.0])
                tot[M][0] += t_q + t_sp
                tot[M][1] += (t_dq + t_dn) if t_dn is not None else float("nan")
                qwen.append(row("qwen25_7b", **r))
                del X, xq, xd, sx, sxd, Y, ws
            del ops, dops, tv, tm, sw, wq, swd
            torch.cuda.empty_cache()
        for M, (ts, td) in tot.items():
            sp = td / ts
            qwen.append(row("qwen25_7b_layer", pattern=f"{2 * n - 2}:{2 * n}", M=M,
                            tokens_per_s_layer=M / (ts * 1e-6), tokens_per_s_model=M / (ts * 1e-6) / QWEN_LAYERS,
                            vs_dense=None if math.isnan(sp) else sp,
                            efficiency=None if math.isnan(sp) else sp / (n / (n - 1))))
    detail["qwen25_7b_slide_int8"] = qwen

    # online 2:4 prune of activations (X 8192x4096) with FP8 codes, dense FP8 W, against dense FP8
    M, K, Nout = 8192, 4096, 4096
    Xs = [randn((M, K), 1.0, torch.bfloat16)]
    Xs += [Xs[0].clone() for _ in range(rotation(2 * M * K) - 1)]
    Wf = randn((Nout, K), 0.02)
    wq, swd = ss.quant_lift_act(Wf, 2, "fp8")
    sx = torch.empty(M, dtype=torch.float32, device=dev)
    nv, nm = ss.tiled_bytes(M, K, "fp8")
    tv = torch.empty(nv, dtype=torch.uint8, device=dev)
    tm = torch.empty(nm, dtype=torch.uint8, device=dev)
    Y = torch.empty((M, Nout), dtype=torch.bfloat16, device=dev)
    xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    t_pr = median_us(torch, [lambda X=X: ss.prune24_act_tiled(X, "fp8", out=(tv, tm, sx)) for X in Xs])
    t_sp = median_us(torch, [lambda: ss.spgemm_tiled(ss.SS_SPARSE_X, M, Nout, K, tv, tm, wq, sx, swd, "bf16", out=Y)])
    par = None
    if check:  # before the dense comparator's quantiser rewrites sx
        td = torch.from_numpy(_pick(M, 16, rng, edge=8)).to(dev)
        cd = torch.from_numpy(_pick(Nout, 64, rng)).to(dev)
        par = sampled_parity("X", 2, "fp8", K, Wf.index_select(0, cd).cpu().numpy(),
                             Xs[0].index_select(0, td).view(torch.int16).cpu().numpy().view(np.uint16),
                             Y.index_select(0, td).index_select(1, cd).view(torch.int16).cpu().numpy().view(np.uint16),
                             sx.index_select(0, td).cpu().numpy(), swd.index_select(0, cd).cpu().numpy())
    t_q = median_us(torch, [lambda X=X: ss.quant_lift_act(X, 2, "fp8", out=(xq, sx)) for X in Xs])
    try:
        t_dn = median_us(torch, [lambda: torch._scaled_mm(xq, wq.t(), scale_a=sx[:, None], scale_b=swd[None, :],
                                                          out_dtype=torch.bfloat16)])
    except Exception:  # noqa: BLE001
        t_dn = None
    pb = 2 * M * K + nv + nm + 4 * M
    detail["sparse_activation_fp8"] = row(
        "sparse_activation_fp8", M=M, K=K, N=Nout, prune24_act_tiled_us=t_pr, prune_GBs=pb / t_pr / 1e3,
        prune_frac=pb / t_pr / 1e3 / HBM_PEAK_GBS, sparse_gemm_us=t_sp,
        gemm_frac=product_ops(M, Nout, K) / t_sp / 1e6 / DENSE_PEAK_T["fp8"], dense_quant_us=t_q,
        dense_fp8_gemm_us=t_dn, vs_dense=None if t_dn is None else (t_q + t_dn) / (t_pr + t_sp),
        input_copies=len(Xs), parity_vs_oracle=par)
    del Xs, Wf, wq, swd, sx, tv, tm, Y, xq
    torch.cuda.empty_cache()

    # quant+lift bandwidth on 2048 and 16384 tokens (K = 4096), inputs rotated out of the Infinity Cache
    ql = []
    for M in (2048, 16384):
        for n in (2, 4):
            K = 4096
            Kc = ss.lifted_k(K, n)
            byts = quant_bytes(M, K, Kc)
            nr = rotation(byts)
            bufs = [(randn((M, K), 1.0, torch.bfloat16), torch.empty((M, Kc), dtype=torch.int8, device=dev),
                     torch.empty(M, dtype=torch.float32, device=dev)) for _ in range(nr)]
            qf = [lambda b=b: ss.quant_lift_act(b[0], n, "i8", out=(b[1], b[2])) for b in bufs]
            t = median_us(torch, qf)
            gr = {}
            if M <= 4096:  # a few microseconds per call: also timed without the host in the loop
                tg = median_us_graph(torch, qf)
                gr = {"graph_us": tg, "graph_GBs": byts / tg / 1e3, "graph_frac": byts / tg / 1e3 / HBM_PEAK_GBS}
            ql.append(row("quant_lift_int8", M=M, K=K, n=n, K_prime=Kc, us=t, GBs=byts / t / 1e3,
                          frac=byts / t / 1e3 / HBM_PEAK_GBS, buffer_sets=nr, working_set_MB=nr * byts / 1e6, **gr))
            del bufs
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t = median_us(torch, [lambda: dst.copy_(src)])
    ql.append(row("device_copy_1GiB", GBs=2 * (1 << 30) / t / 1e3))
    del src, dst
    torch.cuda.empty_cache()
    detail["quant_lift"] = ql

    # block-scaled FP8 (128 x 128 weight blocks, per-token groups of 128) on the Llama-shaped 2:4 layers
    blk = []
    for M in (4096,):
        tot = 0.0
        for name, (K, Nout) in synth.LLAMA31_8B_LINEARS.items():
            W = randn((Nout, K), 0.02)
            tv, tm, sw = ss.prune24_block(W)
            del W
            Kc = ss.lifted_k(K, 2)
            X = randn((M, K), 1.0, torch.bfloat16)
            xq = torch.empty((M, Kc), dtype=torch.float8_e4m3fn, device=dev)
            sx = torch.empty((M, Kc // 128), dtype=torch.float32, device=dev)
            Y = torch.empty((M, Nout), dtype=torch.bfloat16, device=dev)
            t_q = median_us(torch, [lambda: ss.quant_group_act(X, out=(xq, sx))])
            t_sp = median_us(torch, [lambda: ss.spgemm_tiled_block(M, Nout, Kc, tv, tm, xq, sx, sw, "bf16", out=Y)])
            tot += t_q + t_sp
            blk.append(row("block_fp8", layer=name, M=M, K=K, N=Nout, quant_group_us=t_q, sparse_gemm_us=t_sp,
                           gemm_frac=product_ops(M, Nout, Kc) / t_sp / 1e6 / DENSE_PEAK_T["fp8"]))
            del tv, tm, sw, X, xq, sx, Y
        blk.append(row("block_fp8_layer", M=M, tokens_per_s=M / (tot * 1e-6)))
        torch.cuda.empty_cache()
    detail["block_fp8"] = blk

    # quant+product A/B: the per-token quantisation inside the product's prologue (ss_quant_spgemm_prefill, one
    # absmax pass + the product coding bf16 rows into its LDS stages + scales) against ss_quant_lift_act +
    # ss_spgemm_tiled, Llama-shaped 2:4 FP8 layers
    fused = []
    for M in (4096, 16384):
        tot_f, tot_2 = 0.0, 0.0
        for name, (K, Nout) in synth.LLAMA31_8B_LINEARS.items():
            W = randn((Nout, K), 0.02)
            tv, tm, sw = ss.slide_decompose_tiled(W, 2, "fp8")
            del W
            X = randn((M, K), 1.0, torch.bfloat16)
            xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
            sx = torch.empty(M, dtype=torch.float32, device=dev)
            sxf = torch.empty(M, dtype=torch.float32, device=dev)
            Y = torch.empty((M, Nout), dtype=torch.bfloat16, device=dev)
            t_f = median_us(torch, [lambda: ss.quant_spgemm_prefill(X, tv, tm, sw, Nout, "fp8", "bf16", out=Y, sx_out=sxf)])

            def two():
                ss.quant_lift_act(X, 2, "fp8", out=(xq, sx))
                ss.spgemm_tiled(ss.SS_SPARSE_W, M, Nout, K, tv, tm, xq, sx, sw, "bf16", out=Y, workspace=False)
            t_2 = median_us(torch, [two])
            tot_f += t_f
            tot_2 += t_2
            fused.append(row("quant_in_product", layer=name, M=M, K=K, N=Nout, fused_us=t_f, two_calls_us=t_2,
                             fused_vs_two_calls=t_2 / t_f))
            del tv, tm, sw, X, xq, sx, sxf, Y
        fused.append(row("quant_in_product_layer", M=M, fused_us=tot_f, two_calls_us=tot_2,
                         fused_vs_two_calls=tot_2 / tot_f))
        torch.cuda.empty_cache()
    detail["quant_in_product"] = fused

    # online 2:4 on the attention operand roles (bf16), 32 heads x 4096 tokens x 128, one batched launch
    H, L, d = 32, 4096, 128
    Kq = ss.lifted_k(d, 2)
    Q = randn((H * L, d), 1.0, torch.bfloat16)
    Kp = torch.zeros((H, L, Kq), dtype=torch.bfloat16, device=dev)
    Kp[:, :, :d] = randn((H, L, d), 1.0, torch.bfloat16)
    nv, nm = ss.tiled_bytes(H * L, Kq, "bf16")
    tvq = torch.empty(nv, dtype=torch.uint8, device=dev)
    tmq = torch.empty(nm, dtype=torch.uint8, device=dev)
    S = torch.empty((H, L, L), dtype=torch.bfloat16, device=dev)
    t_pq = median_us(torch, [lambda: ss.prune24_act_tiled(Q, "bf16", out=(tvq, tmq, None))])
    t_qk = median_us(torch, [lambda: ss.spgemm_tiled_batched(ss.SS_SPARSE_X, H, L, L, Kq, tvq, tmq, Kp, None, None,
                                                             "bf16", out=S)])
    Qh, Kt = Q.view(H, L, d), Kp[:, :, :d].transpose(1, 2).contiguous()
    t_qk_dn = median_us(torch, [lambda: torch.bmm(Qh, Kt)])
    # K pruned along the head dimension: the keys are the sparse operand (side W), Q the dense one
    Qp = torch.zeros((H, L, Kq), dtype=torch.bfloat16, device=dev)
    Qp[:, :, :d] = Q.view(H, L, d)
    Kr = Kp[:, :, :d].reshape(H * L, d).contiguous()
    t_pk = median_us(torch, [lambda: ss.prune24_act_tiled(Kr, "bf16", out=(tvq, tmq, None))])
    t_qk2 = median_us(torch, [lambda: ss.spgemm_tiled_batched(ss.SS_SPARSE_W, H, L, L, Kq, tvq, tmq, Qp, None, None,
                                                              "bf16", out=S)])
    del Q, Kp, tvq, tmq, Qh, Kt, S, Qp, Kr
    P = torch.softmax(randn((H * L, L), 2.0), dim=1).to(torch.bfloat16)
    Vt = randn((H, d, L), 1.0, torch.bfloat16)
    nv, nm = ss.tiled_bytes(H * L, L, "bf16")
    tvp = torch.empty(nv, dtype=torch.uint8, device=dev)
    tmp = torch.empty(nm, dtype=torch.uint8, device=dev)
    O = torch.empty((H, L, d), dtype=torch.bfloat16, device=dev)
    t_pp = median_us(torch, [lambda: ss.prune24_act_tiled(P, "bf16", out=(tvp, tmp, None))])
    t_pv = median_us(torch, [lambda: ss.spgemm_tiled_batched(ss.SS_SPARSE_X, H, L, d, L, tvp, tmp, Vt, None, None,
                                                             "bf16", out=O)])
    Ph, V = P.view(H, L, L), Vt.transpose(1, 2).contiguous()
    t_pv_dn = median_us(torch, [lambda: torch.bmm(Ph, V)])
    # V pruned along the keys: V^T [d, L] per head is the sparse operand (side W), P the dense one
    nv, nm = ss.tiled_bytes(H * d, L, "bf16")
    tvv = torch.empty(nv, dtype=torch.uint8, device=dev)
    tmv = torch.empty(nm, dtype=torch.uint8, device=dev)
    Vt2 = Vt.reshape(H * d, L)
    t_pvv = median_us(torch, [lambda: ss.prune24_act_tiled(Vt2, "bf16", out=(tvv, tmv, None))])
    P3 = P.view(H, L, L)
    t_pv2 = median_us(torch, [lambda: ss.spgemm_tiled_batched(ss.SS_SPARSE_W, H, L, d, L, tvv, tmv, P3, None, None,
                                                              "bf16", out=O)])
    del tvv, tmv
    detail["attention_roles_bf16"] = row(
        "attention_roles_bf16", heads=H, tokens=L, head_dim=d,
        qk={"prune_q_us": t_pq, "sparse_batched_us": t_qk, "dense_bmm_us": t_qk_dn,
            "vs_dense": t_qk_dn / (t_pq + t_qk)},
        qk_k_pruned={"prune_k_us": t_pk, "sparse_batched_us": t_qk2, "vs_dense": t_qk_dn / (t_pk + t_qk2)},
        pv_v_pruned={"prune_v_us": t_pvv, "sparse_batched_us": t_pv2, "vs_dense": t_pv_dn / (t_pvv + t_pv2),
                     "product_vs_dense": t_pv_dn / t_pv2},
        pv={"prune_p_us": t_pp, "sparse_batched_us": t_pv, "dense_bmm_us": t_pv_dn,
            "gemm_frac": 2.0 * H * L * L * d / 2 / t_pv / 1e6 / DENSE_PEAK_T["bf16"],
            "vs_dense": t_pv_dn / (t_pp + t_pv), "product_vs_dense": t_pv_dn / t_pv})
    del P, Vt, tvp, tmp, O, Ph, V
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
