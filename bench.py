#!/usr/bin/env python3
"""Benchmark of the W4A16 group-32 path on one MI355X.

Headline workload: the dense SwiGLU MLP at decode size (M = 4 tokens, hidden
7168, intermediate 18432, float32 activations), one w4a16_swiglu_mlp call per
step.  Weights are drawn on the GPU (seeded), quantized and prepacked by the
library, and several copies are rotated across steps so the 256 MB Infinity
Cache cannot serve them.  Inputs are resident in HBM before timing starts.

The default run prints one JSON line: the headline step throughput
(algorithmic HBM bytes per second over a timed region of exactly --steps
plain calls, synchronised on both sides), its per-step p10/p50/p90, the
roofline of the dominant kernel (its duration measured live with HIP events
that the library takes from the kernel's own dispatch) and the CPU oracle
timed on a bounded sample of the same workload.  Under "workloads" the same
record follows for every other configuration: the single GEMM (cold and
warm), the tree-verify MLP at 64 tokens (float32 and bf16), the MoE decode
and prefill layers, the hot-expert GEMM, and one GPU's share of the dense MLP
under 8-way tensor parallelism (intermediate 2304) at 4 and 64 tokens.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
    python bench.py --workload NAME        # one workload's line only
    python bench.py --traffic-summary DIR --workload NAME
        # writes profiles/traffic_<kernel>_<workload>.txt from two rocprofv3
        # --pmc runs (FETCH_SIZE, then WRITE_SIZE) under DIR/fetch, DIR/write
        # and a copy calibration under DIR/fetch_copy, DIR/write_copy
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))

METRIC = "W4A16 GEMM/MoE µs + achieved HBM GB/s (% of 8 TB/s) at decode M; TFLOP/s at M≥512"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 / f16 matrix cores, published
OTHER_WORKLOADS = ("gemm_m1", "mlp_verify_m64_f32", "mlp_verify_m64_bf16", "moe_decode_m64",
                   "moe_prefill_m2048", "gemm_m2048_hot_expert", "mlp_decode_m4_tp8", "mlp_verify_m64_bf16_tp8")
CSRC = "int4_w4a16_group_g32_amd/csrc/"
# Sources of each dominant kernel: a stored counter summary is used only
# while they hash to the value it was taken on.
KERNEL_SOURCES = {
    "gemv": (CSRC + "gemv.hip", CSRC + "gemv.h", CSRC + "mfma_ops.h", CSRC + "common.h"),
    "mfma": (CSRC + "mfma.hip", CSRC + "mfma.h", CSRC + "mfma_ops.h", CSRC + "common.h"),
    "wide": (CSRC + "wide.hip", CSRC + "mfma.h", CSRC + "mfma_ops.h", CSRC + "common.h"),
}


# ---------------------------------------------------------------- timing

def _events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:  # torch creates the HIP event on first record
        e.record()
    return evs


def _handles(evs):
    arr = (ctypes.c_void_p * len(evs))()
    for i, e in enumerate(evs):
        arr[i] = e.cuda_event
    return arr


def timed_steps_ms(steps, step):
    """The timed region: exactly `steps` plain steps between two events, with a
    device synchronization on both sides.  Returns the mean ms per step."""
    import torch
    t0, t1 = _events(2)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def step_percentiles(steps, step):
    """A second pass of `steps` steps with an event between consecutive steps:
    the p10, p50 and p90 of the per-step times (ms)."""
    import torch
    evs = _events(steps + 1)
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(steps):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    d = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    q = lambda f: d[min(len(d) - 1, int(round(f * (len(d) - 1))))]
    return {"p10": round(q(0.1), 5), "p50": round(q(0.5), 5), "p90": round(q(0.9), 5)}


def kernel_ms(steps, names, timed_step, cap):
    """A pass of `steps` steps through a *_timed entry point, which brackets
    kernel j with events 2j and 2j + 1 taken from the kernel's own dispatch:
    the mean execution time (ms) of each kernel."""
    import torch
    evs = [_events(cap) for _ in range(steps)]
    handles = [_handles(e) for e in evs]
    torch.cuda.synchronize()
    rec = [timed_step(i, handles[i]) for i in range(steps)]
    torch.cuda.synchronize()
    n = min(rec) // 2
    return {nm: statistics.mean(e[2 * j].elapsed_time(e[2 * j + 1]) for e in evs)
            for j, nm in enumerate(names[:n])}


# ---------------------------------------------------------------- counters

def sources_sha(kernel):
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(kernel_key, workload):
    return os.path.join(ROOT, "profiles", f"traffic_{kernel_key}_{workload}.txt")


def stored_traffic(workload, kernel_key, kernel):
    """HBM bytes per launch from profiles/traffic_<kernel_key>_<workload>.txt:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the factor
    the same counter shows on a plain copy of known size.  None if the file
    is missing or was taken on other kernel sources."""
    path = traffic_path(kernel_key, workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha") != sources_sha(kernel):
        return None
    fetch = float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"]) * 1024
    write = float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"]) * 1024
    return int(round(fetch + write))


def copy_calibration():
    """A plain device copy of 256 MiB, three times: the reference for scaling
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = 64 * 1024 * 1024
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "repeats": 3}), flush=True)


def _counter_mean(run_dir, counter, match, nth=None):
    import csv
    vals = []
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
                    vals.append((int(r.get("Dispatch_Id", 0) or 0), float(r["Counter_Value"])))
    vals.sort()
    if nth is not None:  # one kernel of a pair with the same name: every nth dispatch
        vals = vals[nth[0]::nth[1]]
    if not vals:
        raise SystemExit(f"no {counter} rows for the kernel under {run_dir}")
    return statistics.mean(v for _, v in vals), len(vals)


def traffic_summary(src_dir, workload):
    """Write profiles/traffic_<kernel>_<workload>.txt for the workload's
    dominant kernel from rocprofv3 counter runs (see the module docstring)."""
    key, kernel, match, nth = DOMINANT[workload]
    cp = lambda n: "copyBuffer" in n
    copy_kib = 256 * 1024  # the calibration copy reads and writes 256 MiB per dispatch
    fetch, nf = _counter_mean(os.path.join(src_dir, "fetch"), "FETCH_SIZE", match, nth)
    write, nw = _counter_mean(os.path.join(src_dir, "write"), "WRITE_SIZE", match, nth)
    cf, _ = _counter_mean(os.path.join(src_dir, "fetch_copy"), "FETCH_SIZE", cp)
    cw, _ = _counter_mean(os.path.join(src_dir, "write_copy"), "WRITE_SIZE", cp)
    fs, ws = copy_kib / cf, copy_kib / cw
    path = traffic_path(key, workload)
    with open(path, "w") as f:
        f.write(f"# HBM traffic of {kernel} in the {workload} workload, per dispatch.\n")
        f.write(f"# commands: rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --workload {workload} --steps 3 "
                f"--warmup 1 --no-cpu-baseline; the same with WRITE_SIZE; the same two on "
                f"python3 bench.py --copy-calibration; then python3 bench.py --traffic-summary DIR "
                f"--workload {workload}\n")
        f.write(f"# scale = 256 MiB / the counter's KiB on a 256 MiB device copy\n")
        f.write(f"kernel = {kernel}\nworkload = {workload}\nsource_sha = {sources_sha(KERNEL_OF[key])}\n")
        f.write(f"fetch_kib_per_dispatch = {fetch:.1f}\nfetch_dispatches = {nf}\nfetch_scale = {fs:.5f}\n")
        f.write(f"write_kib_per_dispatch = {write:.1f}\nwrite_dispatches = {nw}\nwrite_scale = {ws:.5f}\n")
        f.write(f"traffic_bytes_per_dispatch = {int(round((fetch * fs + write * ws) * 1024))}\n")
    print(path)


# dominant kernel per workload: (file key, kernel description, name match, every-nth selector)
KERNEL_OF = {"gate_up": "gemv", "gemv": "gemv", "mfma_gate_up": "mfma", "wide": "wide"}
DOMINANT = {
    "gemm_m1": ("gemv", "gemv_kernel", lambda n: "gemv_kernel" in n, None),
    "mlp_decode_m4": ("gate_up", "gemv_kernel<4, 2>", lambda n: "gemv_kernel<4, 2>" in n, None),
    "mlp_verify_m64_f32": ("mfma_gate_up", "mfma_kernel<2, 8, 2, true> (gate/up)",
                           lambda n: "mfma_kernel<2, 8, 2, true>" in n, (0, 2)),
    "mlp_verify_m64_bf16": ("mfma_gate_up", "mfma_kernel<1, 8, 2, true> (gate/up)",
                            lambda n: "mfma_kernel<1, 8, 2, true>" in n, (0, 2)),
    "moe_decode_m64": ("gate_up", "gemv_kernel<1, 1> (gate/up)", lambda n: "gemv_kernel<1, 1>" in n, (0, 2)),
    "moe_prefill_m2048": ("mfma_gate_up", "mfma_kernel<1, 4, 3, false> (gate/up)",
                          lambda n: "mfma_kernel<1, 4, 3, false>" in n, (0, 2)),
    "gemm_m2048_hot_expert": ("wide", "wide_kernel", lambda n: "wide_kernel" in n, None),
    "mlp_decode_m4_tp8": ("gate_up", "gemv_kernel<1, 2> (gate/up)", lambda n: "gemv_kernel<1, 2>" in n, (0, 2)),
    "mlp_verify_m64_bf16_tp8": ("mfma_gate_up", "mfma_kernel<1, 8, 2, true> (gate/up)",
                                lambda n: "mfma_kernel<1, 8, 2, true>" in n, (0, 2)),
}


# ---------------------------------------------------------------- CPU baseline

def cpu_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count()
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "cpus_usable": aff}


def _blas_threads():
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])


def time_oracle(fn, repeats):
    """Median seconds of `repeats` calls of fn, first with every BLAS thread,
    then with one; returns (seconds_all, threads_all, seconds_1)."""
    from threadpoolctl import threadpool_limits
    fn()  # untimed: first-touch and BLAS start-up
    t_all = []
    for _ in range(repeats):
        t = time.perf_counter()
        fn()
        t_all.append(time.perf_counter() - t)
    threads = _blas_threads()
    t_one = []
    with threadpool_limits(limits=1):
        for _ in range(max(1, repeats // 2)):
            t = time.perf_counter()
            fn()
            t_one.append(time.perf_counter() - t)
    return statistics.median(t_all), threads, statistics.median(t_one)


def _baseline(amount, unit, scale, sec_all, threads, sec_one, sample, repeats):
    d = {"value": round(amount / sec_all / scale, 6), "unit": unit, "cores": threads, "kind": "oracle",
         "sample": sample, "seconds": round(sec_all, 4),
         "value_1core": round(amount / sec_one / scale, 6), "seconds_1core": round(sec_one, 4),
         "repeats": repeats}
    d.update(cpu_info())
    return d


def cpu_baseline_gemm(cfg, x, big, repeats=5):
    """The oracle's float64 GEMM on the workload (rows bounded to 256 for the
    2048-row GEMM), weights drawn by the same generator and quantized by the
    oracle (not timed); TFLOP/s when M >= 512, else GB/s."""
    import oracle as O
    import workloads as W

    K, N = cfg.K, cfg.N
    rows = min(cfg.M, 256)
    qw, sc = O.quantize_w4a16(W.weights(K, N, cfg.index, W.TAG_GATE, 0, device="cuda").cpu().numpy())
    xs = x[:rows].float().cpu().numpy()
    s_all, th, s_one = time_oracle(lambda: O.gemm64(xs, qw, sc), repeats)
    xbytes = 4 if cfg.x_dtype == "f32" else 2
    if big:
        amount, unit, scale = 2.0 * rows * K * N, "TFLOP/s", 1e12
    else:
        amount, unit, scale = K * N * 5 // 8 + rows * K * xbytes + rows * N * 4, "GB/s", 1e9
    return _baseline(amount, unit, scale, s_all, th, s_one,
                     f"{rows} of the {cfg.M} rows of the {cfg.name} GEMM, numpy float64 dequantize-then-matmul",
                     repeats)


def cpu_baseline_mlp(cfg, cols=2048, repeats=5):
    """The oracle's float64 SwiGLU MLP on the workload's activations over a
    slice of the intermediate dimension (gate/up columns [0, cols) and the
    matching rows of down: the step's work scales linearly with it), weights
    drawn by the same generator and quantized by the oracle (not timed)."""
    import numpy as np
    import oracle as O
    import workloads as W

    H, I, M = cfg.K, cfg.N, cfg.M
    g = W.weights(H, I, cfg.index, W.TAG_GATE, device="cuda")[:, :cols].cpu().numpy()
    u = W.weights(H, I, cfg.index, W.TAG_UP, device="cuda")[:, :cols].cpu().numpy()
    d = W.weights(I, H, cfg.index, W.TAG_DOWN, device="cuda")[:cols].cpu().numpy()
    codes = [O.quantize_w4a16(np.ascontiguousarray(a)) for a in (g, u, d)]
    x = W.activations(M, H, cfg.index, cfg.x_dtype, device="cuda").float().cpu().numpy()
    s_all, th, s_one = time_oracle(lambda: O.swiglu_mlp64(x, *codes), repeats)
    xbytes = 4 if cfg.x_dtype == "f32" else 2
    amount = mlp_bytes(M, H, cols, xbytes)
    return _baseline(amount, "GB/s", 1e9, s_all, th, s_one,
                     f"the {cfg.name} step over {cols} of the {I} intermediate columns ({amount} algorithmic bytes), "
                     f"numpy float64 dequantize-then-matmul", repeats)


def cpu_baseline_moe(cfg, ids_np, wts, x, tokens=1, repeats=3):
    """The oracle's float64 MoE layer on the first `tokens` tokens through the
    experts they are routed to (weights drawn by the same generator and
    quantized by the oracle, not timed)."""
    import numpy as np
    import oracle as O
    import workloads as W

    E, H, I = cfg.experts, cfg.K, cfg.N
    sample = np.arange(tokens)
    experts = np.unique(ids_np[sample])
    codes = {int(e): tuple(O.quantize_w4a16(W.weights(K, N, cfg.index, tag, int(e), device="cuda").cpu().numpy())
                           for tag, (K, N) in ((W.TAG_GATE, (H, I)), (W.TAG_UP, (H, I)), (W.TAG_DOWN, (I, H))))
             for e in experts}
    xs = x.float().cpu().numpy()
    w_np = wts.cpu().numpy()
    s_all, th, s_one = time_oracle(lambda: O.moe64(xs, ids_np, w_np, lambda e: codes[e], E, tokens=sample), repeats)
    xbytes = 4 if cfg.x_dtype == "f32" else 2
    amount = len(experts) * 3 * H * I * 5 // 8 + tokens * H * (xbytes + 4)
    return _baseline(amount, "GB/s", 1e9, s_all, th, s_one,
                     f"{tokens} of the {cfg.M} tokens through their {len(experts)} experts ({amount} algorithmic "
                     f"bytes), numpy float64 dequantize-then-matmul", repeats)


# ---------------------------------------------------------------- workloads

def mlp_bytes(M, H, I, xbytes):
    weights = 3 * H * I * 5 // 8          # 0.5 B packed + 4/32 B scale per weight
    return weights + M * H * xbytes + M * H * 4


def gate_up_bytes(M, H, I, xbytes):
    return 2 * H * I * 5 // 8 + M * H * xbytes + M * I * 4


def _roofline(bound, kernel, achieved, peak, unit, per_launch_key, per_launch, avg_us, traffic):
    return {"bound": bound, "kernel": kernel, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, per_launch_key: per_launch,
            "avg_launch_us": round(avg_us, 2)}


def _line(args, value, unit, ms_step, pct, dtype, config, roofline, kern, extra=None):
    d = {"metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
         "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
         "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": config, "ms_per_step_pct": pct,
         "roofline": roofline, "kernels_us": {n: round(v * 1e3, 2) for n, v in kern.items()}}
    if extra:
        d.update(extra)
    return d


def run_mlp(args, cfg):
    import torch
    import int4_w4a16_group_g32_amd as L
    import workloads as W

    H, I, M = cfg.K, cfg.N, cfg.M
    xt = L.F32 if cfg.x_dtype == "f32" else L.BF16
    xbytes = 4 if cfg.x_dtype == "f32" else 2
    base = []
    for K, N, tag in ((H, I, W.TAG_GATE), (H, I, W.TAG_UP), (I, H, W.TAG_DOWN)):
        w = W.weights(K, N, cfg.index, tag, device="cuda")
        base.append(L.quantize_to_weight(w))
        del w
    copies = [base]
    for _ in range(args.copies - 1):
        copies.append([L.Weight(b.qw.clone(), b.scales.clone(), b.K, b.N, b.num_experts, b.layout) for b in base])
    x = W.activations(M, H, cfg.index, cfg.x_dtype, device="cuda")
    y = torch.empty((M, H), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(L.swiglu_mlp_workspace_bytes(M, xt, *base))
    lib = L.load_library()
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cap = 10

    def step(i, evs=None):
        g, u, d = copies[i % len(copies)]
        rec = ctypes.c_int32(0)
        st = lib.w4a16_swiglu_mlp_timed(L._ptr(x), xt, M, ctypes.byref(g.desc()), ctypes.byref(u.desc()),
                                        ctypes.byref(d.desc()), L._ptr(y), L._ptr(ws),
                                        ws.numel(), sptr, evs, 0 if evs is None else cap, ctypes.byref(rec))
        if st != 0:
            raise L.W4A16Error(st, "w4a16_swiglu_mlp_timed")
        return rec.value

    # decode sizes: fused gate/up + SwiGLU GEMV, then the down GEMV; larger M:
    # activation pieces, gate/up MFMA tiles, pieces of h, down MFMA tiles
    gemv = M <= (16 if xt == L.BF16 else 8)
    # (with K splits the tiles leave per-split sums: h is formed in prep_h, and
    # a last kernel sums the down projection's splits)
    names = ["gate_up", "down"] if gemv else ["prep_x", "gate_up", "prep_h", "down", "down_sum"]
    for i in range(args.warmup):
        step(i)
    ms_step = timed_steps_ms(args.steps, step)
    pct = step_percentiles(args.steps, step)
    kern = kernel_ms(args.steps, names, step, cap)
    step_bytes = mlp_bytes(M, H, I, xbytes)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    dom_bytes = gate_up_bytes(M, H, I, xbytes)
    k_dom = kern["gate_up"]
    kernel = ("gemv_kernel" if gemv else "mfma_kernel") + " (fused gate/up + SwiGLU epilogue)"
    key, kname = ("gate_up", "gemv") if gemv else ("mfma_gate_up", "mfma")
    roof = _roofline("hbm", kernel, dom_bytes / (k_dom * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", "bytes_per_launch",
                     dom_bytes, k_dom * 1e3, stored_traffic(cfg.name, key, kname))
    config = {"workload": cfg.name, "M": M, "hidden": H, "intermediate": I, "group_size": 32,
              "x_dtype": cfg.x_dtype, "weight_copies": args.copies, "bytes_per_step": step_bytes,
              "flops_per_step": 6 * M * H * I}
    out = _line(args, value, "GB/s", ms_step, pct, cfg.x_dtype, config, roof, kern,
                {"pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1)})
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_mlp(cfg)
    return out


def run_moe(args, cfg):
    """One routed MoE layer per step (route, grouped gate/up + SwiGLU, grouped
    down, combine).  Expert weights are drawn and quantized on the GPU; the
    expert stacks (10.6 GB) are far larger than any cache."""
    import numpy as np
    import torch
    import int4_w4a16_group_g32_amd as L
    import workloads as W

    E, H, I, M, k = cfg.experts, cfg.K, cfg.N, cfg.M, cfg.top_k
    xt = L.F32 if cfg.x_dtype == "f32" else L.BF16
    xbytes = 4 if cfg.x_dtype == "f32" else 2
    stacks = []
    for tag, (K, N) in ((W.TAG_GATE, (H, I)), (W.TAG_UP, (H, I)), (W.TAG_DOWN, (I, H))):
        qw = torch.empty((E, K // 8, N), dtype=torch.int32, device="cuda")
        sc = torch.empty((E, K // 32, N), dtype=torch.float32, device="cuda")
        for e in range(E):
            L.quantize(W.weights(K, N, cfg.index, tag, e, device="cuda"), qw[e], sc[e])
        stacks.append(L.prepack(L.Weight(qw, sc, K, N, E, L.LAYOUT_CANONICAL), torch.empty_like(qw)))
        del qw
    if cfg.routing == "zipf":
        ids_np = W.topk_zipf(M, E, k, cfg.zipf_alpha, cfg.index)
    else:
        ids_np = W.topk_uniform(M, E, k, cfg.index)
    ids = torch.as_tensor(ids_np).cuda()
    wts = torch.as_tensor(W.gate_weights(M, k, cfg.index)).cuda()
    x = W.activations(M, H, cfg.index, cfg.x_dtype, device="cuda")
    y = torch.empty((M, H), dtype=torch.float32, device="cuda")
    if cfg.shared:
        return run_moe_shared(args, cfg, stacks, ids, ids_np, wts, x, y)
    ws = L.new_workspace(L.moe_workspace_bytes(M, k, xt, *stacks))
    lib = L.load_library()
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # the kernels of one layer: light experts (at most 8 rows with float32
    # activations, 16 with bf16) on the GEMV; when an expert can be heavier,
    # activation pieces and 64-row tiles as well
    mfma = M > (16 if xt == L.BF16 else 8)
    names = (["route", "gate_up_gemv", "prep_x", "gate_up_mfma", "down_gemv", "prep_h", "down_mfma", "combine"]
             if mfma else ["route", "gate_up_gemv", "down_gemv", "combine"])
    cap = 2 * len(names)

    def step(i, evs=None):
        rec = ctypes.c_int32(0)
        st = lib.w4a16_moe_grouped_timed(L._ptr(x), xt, M, L._ptr(ids), L._ptr(wts), k,
                                         ctypes.byref(stacks[0].desc()), ctypes.byref(stacks[1].desc()),
                                         ctypes.byref(stacks[2].desc()), L._ptr(y), L._ptr(ws), ws.numel(),
                                         sptr, evs, 0 if evs is None else cap, ctypes.byref(rec))
        if st != 0:
            raise L.W4A16Error(st, "w4a16_moe_grouped_timed")
        return rec.value

    for i in range(args.warmup):
        step(i)
    ms_step = timed_steps_ms(args.steps, step)
    pct = step_percentiles(args.steps, step)
    kern = kernel_ms(args.steps, names, step, cap)
    counts = np.bincount(ids_np.ravel(), minlength=E)
    active = int((counts > 0).sum())
    step_bytes = active * 3 * H * I * 5 // 8 + M * H * xbytes + M * H * 4
    flops = 2 * 3 * H * I * M * k
    value = step_bytes / (ms_step * 1e-3) / 1e9
    gemv_rows = 16 if xt == L.BF16 else 8
    light, heavy = counts[(counts > 0) & (counts <= gemv_rows)], counts[counts > gemv_rows]
    if mfma and heavy.size:
        # the gate/up tiles: 2 * H * 2I flops per row of the heavy experts
        k_dom = kern["gate_up_mfma"]
        fl = 2 * H * 2 * I * int(heavy.sum())
        roof = _roofline("mfma", "mfma_kernel (grouped gate/up + SwiGLU, experts above "
                         f"{gemv_rows} rows)", fl / (k_dom * 1e-3) / 1e12, MFMA_PEAK_TFLOPS, "TFLOP/s",
                         "flops_per_launch", fl, k_dom * 1e3, stored_traffic(cfg.name, "mfma_gate_up", "mfma"))
        wbytes = heavy.size * 2 * H * I * 5 // 8
        roof["weight_bytes_per_launch"] = wbytes
        roof["weight_gbs"] = round(wbytes / (k_dom * 1e-3) / 1e9, 1)
    else:
        k_dom = kern["gate_up_gemv"]
        b = light.size * 2 * H * I * 5 // 8 + M * H * xbytes + int(light.sum()) * I * 4
        roof = _roofline("hbm", "gemv_kernel (grouped gate/up + SwiGLU, experts up to "
                         f"{gemv_rows} rows)", b / (k_dom * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", "bytes_per_launch", b,
                         k_dom * 1e3, stored_traffic(cfg.name, "gate_up", "gemv"))
    config = {"workload": cfg.name, "M": M, "experts": E, "top_k": k, "hidden": H, "intermediate": I,
              "routing": cfg.routing, "active_experts": active, "bytes_per_step": step_bytes,
              "flops_per_step": flops}
    out = _line(args, value, "GB/s", ms_step, pct, cfg.x_dtype, config, roof, kern,
                {"tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
                 "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1)})
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_moe(cfg, ids_np, wts, x)
    return out


def run_moe_shared(args, cfg, stacks, ids, ids_np, wts, x, y):
    """One MoE layer with a shared expert per step, the shared expert running
    inside the routed experts' grouped launches.  Also times the same work as
    two calls (routed layer, then the shared expert as a dense MLP) to show
    what the overlap saves."""
    import numpy as np
    import torch
    import int4_w4a16_group_g32_amd as L
    import workloads as W

    E, H, I, M, k = cfg.experts, cfg.K, cfg.N, cfg.M, cfg.top_k
    xt = L.F32 if cfg.x_dtype == "f32" else L.BF16
    xbytes = 4 if cfg.x_dtype == "f32" else 2
    shared = []
    for tag, (K, N) in ((W.TAG_GATE, (H, I)), (W.TAG_UP, (H, I)), (W.TAG_DOWN, (I, H))):
        qw = torch.empty((1, K // 8, N), dtype=torch.int32, device="cuda")
        sc = torch.empty((1, K // 32, N), dtype=torch.float32, device="cuda")
        L.quantize(W.weights(K, N, cfg.index, tag, W.SHARED_EXPERT_INDEX, device="cuda"), qw[0], sc[0])
        shared.append(L.prepack(L.Weight(qw, sc, K, N, 1, L.LAYOUT_CANONICAL), torch.empty_like(qw)))
    ws = L.new_workspace(L.moe_shared_workspace_bytes(M, k, xt, *stacks, *shared))

    def step(i):
        L.moe_grouped_shared(x, ids, wts, *stacks, *shared, y, ws)

    for i in range(args.warmup):
        step(i)
    ms_step = timed_steps_ms(args.steps, step)
    pct = step_percentiles(args.steps, step)
    ws_r = L.new_workspace(L.moe_workspace_bytes(M, k, xt, *stacks))
    dense = [L.Weight(w.qw[0], w.scales[0], w.K, w.N, 1, w.layout) for w in shared]
    ws_d = L.new_workspace(L.swiglu_mlp_workspace_bytes(M, xt, *dense))
    y2 = torch.empty_like(y)

    def step2(i):
        L.moe_grouped(x, ids, wts, *stacks, y, ws_r)
        L.swiglu_mlp(x, *dense, y2, ws_d)

    for i in range(args.warmup):
        step2(i)
    ms_two = timed_steps_ms(args.steps, step2)
    active = int((np.bincount(ids_np.ravel(), minlength=E) > 0).sum()) + 1
    step_bytes = active * 3 * H * I * 5 // 8 + M * H * xbytes + M * H * 4
    flops = 2 * 3 * H * I * M * (k + 1)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    config = {"workload": cfg.name, "M": M, "experts": E, "top_k": k, "hidden": H, "intermediate": I,
              "routing": cfg.routing, "shared_experts": 1, "active_experts_with_shared": active,
              "bytes_per_step": step_bytes}
    return _line(args, value, "GB/s", ms_step, pct, cfg.x_dtype, config, None, {},
                 {"tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
                  "ms_routed_then_shared_mlp": round(ms_two, 5),
                  "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1)})


def run_gemm(args, cfg, cold=None):
    """One w4a16_gemm call per step (dense weight, M x K x N).  TFLOP/s
    against the bf16 dense MFMA peak when M >= 512, else GB/s.  Weight copies
    are rotated; for the single GEMM (M = 1) the cold figure rotates 4096
    copies (over 300 MB, more than the Infinity Cache) and the warm one
    re-uses one copy."""
    import torch
    import int4_w4a16_group_g32_amd as L
    import workloads as W

    M, K, N = cfg.M, cfg.K, cfg.N
    xt = L.F32 if cfg.x_dtype == "f32" else L.BF16
    xbytes = 4 if cfg.x_dtype == "f32" else 2
    small = K * N <= 1 << 20
    n_copies = 4096 if small else max(1, args.copies)
    first = L.quantize_to_weight(W.weights(K, N, cfg.index, W.TAG_GATE, 0, device="cuda"))
    if small:
        qa = first.qw.expand(n_copies, *first.qw.shape[1:]).contiguous()
        sa = first.scales.expand(n_copies, *first.scales.shape[1:]).contiguous()
        copies = [L.Weight(qa[c:c + 1], sa[c:c + 1], K, N, 1, first.layout) for c in range(n_copies)]
    else:
        copies = [first] + [L.quantize_to_weight(W.weights(K, N, cfg.index, W.TAG_GATE, c, device="cuda"))
                            for c in range(1, n_copies)]
    x = W.activations(M, K, cfg.index, cfg.x_dtype, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(L.gemm_workspace_bytes(M, first, xt))
    lib = L.load_library()
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cap = 6

    def run(rotate):
        def step(i, evs=None):
            w = copies[i % len(copies)] if rotate else copies[0]
            rec = ctypes.c_int32(0)
            st = lib.w4a16_gemm_timed(L._ptr(x), xt, M, ctypes.byref(w.desc()), L._ptr(y), L._ptr(ws), ws.numel(),
                                      sptr, evs, 0 if evs is None else cap, ctypes.byref(rec))
            if st != 0:
                raise L.W4A16Error(st, "w4a16_gemm_timed")
            return rec.value
        for i in range(args.warmup):
            step(i)
        ms = timed_steps_ms(args.steps, step)
        pct = step_percentiles(args.steps, step)
        names = ["gemv"] if M <= (16 if xt == L.BF16 else 8) else ["prep_x", "tiles", "split_sum"]
        return ms, pct, kernel_ms(args.steps, names, step, cap)

    ms_step, pct, kern = run(True)
    flops = 2.0 * M * K * N
    step_bytes = K * N * 5 // 8 + M * K * xbytes + M * N * 4
    tflops = flops / (ms_step * 1e-3) / 1e12
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    big = M >= 512
    if big:
        k_dom = kern["tiles"]
        roof = _roofline("mfma", "wide_kernel", flops / (k_dom * 1e-3) / 1e12, MFMA_PEAK_TFLOPS, "TFLOP/s",
                         "flops_per_launch", int(flops), k_dom * 1e3, stored_traffic(cfg.name, "wide", "wide"))
    else:
        k_dom = kern.get("gemv", kern.get("tiles"))
        roof = _roofline("hbm", "gemv_kernel", step_bytes / (k_dom * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                         "bytes_per_launch", step_bytes, k_dom * 1e3, stored_traffic(cfg.name, "gemv", "gemv"))
    config = {"workload": cfg.name, "M": M, "K": K, "N": N, "bytes_per_step": step_bytes,
              "flops_per_step": int(flops), "weight_copies": n_copies}
    extra = {"pct_mfma_peak_bf16": round(100 * tflops / MFMA_PEAK_TFLOPS, 1), "gbs": round(gbs, 1),
             "us_per_step": round(ms_step * 1e3, 2)}
    if small:
        ms_w, pct_w, kern_w = run(False)
        extra["warm"] = {"ms_per_step": round(ms_w, 5), "ms_per_step_pct": pct_w,
                         "kernels_us": {n: round(v * 1e3, 2) for n, v in kern_w.items()},
                         "value": round(step_bytes / (ms_w * 1e-3) / 1e9, 2), "unit": "GB/s"}
        extra["cold_note"] = "value and ms_per_step: 4096 rotated weight copies (cold); warm: one copy re-used"
    out = _line(args, tflops if big else gbs, "TFLOP/s" if big else "GB/s", ms_step, pct, cfg.x_dtype, config,
                roof, kern, extra)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_gemm(cfg, x, big)
    return out


def run_router(args, cfg):
    """One router call per step: float32 logits [M][E] -> top-k ids and
    softmax gate weights.  A few MB at most, so the figure is latency."""
    import torch
    import int4_w4a16_group_g32_amd as L
    import workloads as W

    M, E, k = cfg.M, cfg.experts, cfg.top_k
    logits = W.router_logits(M, E, cfg.index, device="cuda")
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((M, k), dtype=torch.float32, device="cuda")

    def step(i):
        L.moe_topk(logits, k, ids, wts)

    for i in range(args.warmup):
        step(i)
    ms_step = timed_steps_ms(args.steps, step)
    pct = step_percentiles(args.steps, step)
    step_bytes = M * E * 4 + M * k * 8
    value = step_bytes / (ms_step * 1e-3) / 1e9
    config = {"workload": cfg.name, "M": M, "experts": E, "top_k": k, "bytes_per_step": step_bytes}
    return _line(args, value, "GB/s", ms_step, pct, "f32", config, None, {},
                 {"pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)})


def run_workload(args, name):
    import workloads as W
    cfg = W.CONFIGS[name]
    runner = {"mlp": run_mlp, "moe": run_moe, "router": run_router, "gemm": run_gemm}.get(cfg.kind)
    if runner is None:
        print(f"workload {cfg.name} has no bench line", file=sys.stderr)
        sys.exit(2)
    return runner(args, cfg)


SUMMARY_KEYS = ("value", "unit", "ms_per_step", "ms_per_step_pct", "dtype", "config", "roofline", "kernels_us",
                "cpu_baseline", "pct_hbm_peak", "pct_mfma_peak_bf16", "tflops", "gbs", "us_per_step", "warm",
                "cold_note")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="one workload's line only (default: all)")
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--traffic-summary", metavar="DIR", default=None,
                    help="write the workload's traffic summary from counter runs under DIR (no GPU)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr, flush=True)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    if args.traffic_summary:
        traffic_summary(args.traffic_summary, args.workload or "mlp_decode_m4")
        return

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.workload:
        print(json.dumps(run_workload(args, args.workload)), flush=True)
        return
    result = run_workload(args, "mlp_decode_m4")
    result["workloads"] = {}
    for name in OTHER_WORKLOADS:
        torch.cuda.empty_cache()
        line = run_workload(args, name)
        result["workloads"][name] = {k: line[k] for k in SUMMARY_KEYS if k in line}
        print(f"bench: {name} {line['value']} {line['unit']} ({line['ms_per_step']} ms per step)", file=sys.stderr,
              flush=True)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
