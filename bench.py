#!/usr/bin/env python3
"""Benchmark of the W4A16 group-32 path on one MI355X.

Default workload: the dense SwiGLU MLP at decode size (M = 4 tokens, hidden
7168, intermediate 18432, float32 activations), one w4a16_swiglu_mlp call per
step.  Weights are drawn on the GPU (seeded), quantized and prepacked by the
library, and several copies are rotated across steps so the 256 MB Infinity
Cache cannot serve them.  Inputs are resident in HBM before timing starts.

Prints one JSON line with the step throughput (algorithmic HBM bytes per
second over a timed region of plain calls), the roofline of the dominant
kernel (fused gate/up GEMV, timed live in a second pass with HIP events the
library records between its kernels) and the CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))

METRIC = "W4A16 GEMM/MoE µs + achieved HBM GB/s (% of 8 TB/s) at decode M; TFLOP/s at M≥512"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


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


# Sources of the dominant decode kernel; a stored counter summary is only used
# while they are unchanged.
TRAFFIC_SOURCES = ("int4_w4a16_group_g32_amd/csrc/gemv.hip", "int4_w4a16_group_g32_amd/csrc/gemv.h",
                   "int4_w4a16_group_g32_amd/csrc/mfma_ops.h")


def sources_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, kernel_key):
    """HBM bytes per launch from profiles/traffic_<kernel>_<workload>.txt: the
    FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch) each scaled by the
    factor the same counter shows on a plain copy of known size.  None if the
    file is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_key}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha") != sources_sha(TRAFFIC_SOURCES):
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


def mlp_bytes(M, H, I, xbytes):
    weights = 3 * H * I * 5 // 8          # 0.5 B packed + 4/32 B scale per weight
    return weights + M * H * xbytes + M * H * 4


def gate_up_bytes(M, H, I, xbytes):
    return 2 * H * I * 5 // 8 + M * H * xbytes + M * I * 4


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
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    # kernels the library launches for one MLP call: decode sizes run the fused
    # gate/up + SwiGLU GEMV then the down GEMV; larger M runs activation pieces,
    # gate/up MFMA, pieces of h, down MFMA.  The timed entry point brackets each
    # kernel with a start and a stop event taken from its own dispatch.
    cap = 8

    def step(i, evs=None):
        g, u, d = copies[i % len(copies)]
        rec = ctypes.c_int32(0)
        st = lib.w4a16_swiglu_mlp_timed(L._ptr(x), xt, M, ctypes.byref(g.desc()), ctypes.byref(u.desc()),
                                        ctypes.byref(d.desc()), L._ptr(y), L._ptr(ws),
                                        ws.numel(), sptr, evs, 0 if evs is None else cap, ctypes.byref(rec))
        if st != 0:
            raise L.W4A16Error(st, "w4a16_swiglu_mlp_timed")
        return rec.value

    probe = _events(cap)
    marks = step(0, _handles(probe))
    names = {4: ["gate_up", "down"], 8: ["prep_x", "gate_up", "prep_h", "down"]}[marks]

    for i in range(args.warmup):
        step(i)
    ms_step = timed_steps_ms(args, lambda i: step(i))
    kern, ms_marked = per_kernel_ms(args, names, lambda i, h: step(i, h), cap, paired=True)
    step_bytes = mlp_bytes(M, H, I, xbytes)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    # dominant kernel: the fused gate/up + SwiGLU launch
    k_dom = kern["gate_up"]
    dom_bytes = gate_up_bytes(M, H, I, xbytes)
    achieved = dom_bytes / (k_dom * 1e-3) / 1e9
    dom_name = ("gemv_kernel" if M <= 8 else "mfma_kernel") + " (fused gate/up + SwiGLU epilogue)"
    dom_key = "gate_up"

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.x_dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "M": M, "hidden": H, "intermediate": I, "group_size": 32,
                   "x_dtype": cfg.x_dtype, "weight_copies": args.copies, "bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "kernel": dom_name,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(cfg.name, dom_key) if M <= 8 else None,
                     "bytes_per_launch": dom_bytes, "avg_launch_us": round(k_dom * 1e3, 2)},
        "kernels_us": {n: round(v * 1e3, 2) for n, v in kern.items()},
        "ms_per_step_marked": round(ms_marked, 5),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_mlp(cfg, base)
    return result


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
    nev = len(names) + 1

    def step(evs=None):
        rec = ctypes.c_int32(0)
        st = lib.w4a16_moe_grouped_timed(L._ptr(x), xt, M, L._ptr(ids), L._ptr(wts), k,
                                         ctypes.byref(stacks[0].desc()), ctypes.byref(stacks[1].desc()),
                                         ctypes.byref(stacks[2].desc()), L._ptr(y), L._ptr(ws), ws.numel(),
                                         sptr, evs, 0 if evs is None else nev, ctypes.byref(rec))
        if st != 0:
            raise L.W4A16Error(st, "w4a16_moe_grouped_timed")

    for _ in range(args.warmup):
        step()
    ms_step = timed_steps_ms(args, lambda i: step())
    kern, ms_marked = per_kernel_ms(args, names, lambda i, h: step(h))
    active = int((np.bincount(ids_np.ravel(), minlength=E) > 0).sum())
    step_bytes = active * 3 * H * I * 5 // 8 + M * H * xbytes + M * H * 4
    flops = 2 * 3 * H * I * M * k
    value = step_bytes / (ms_step * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.x_dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "M": M, "experts": E, "top_k": k, "hidden": H, "intermediate": I,
                   "routing": cfg.routing, "active_experts": active, "bytes_per_step": step_bytes},
        "tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "kernels_us": {n: round(v * 1e3, 2) for n, v in kern.items()},
        "ms_per_step_marked": round(ms_marked, 5),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
        **({} if args.no_cpu_baseline else {"cpu_baseline": cpu_baseline_moe(cfg, ids_np, wts, x)}),
    }


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
    ms_step = timed_steps_ms(args, step)
    # the same work in two calls: routed layer, then the shared MLP (dense entry point)
    ws_r = L.new_workspace(L.moe_workspace_bytes(M, k, xt, *stacks))
    dense = [L.Weight(w.qw[0], w.scales[0], w.K, w.N, 1, w.layout) for w in shared]
    ws_d = L.new_workspace(L.swiglu_mlp_workspace_bytes(M, xt, *dense))
    y2 = torch.empty_like(y)

    def step2(i):
        L.moe_grouped(x, ids, wts, *stacks, y, ws_r)
        L.swiglu_mlp(x, *dense, y2, ws_d)

    for i in range(args.warmup):
        step2(i)
    ms_two = timed_steps_ms(args, step2)
    active = int((np.bincount(ids_np.ravel(), minlength=E) > 0).sum()) + 1
    step_bytes = active * 3 * H * I * 5 // 8 + M * H * xbytes + M * H * 4
    flops = 2 * 3 * H * I * M * (k + 1)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.x_dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "M": M, "experts": E, "top_k": k, "hidden": H, "intermediate": I,
                   "routing": cfg.routing, "shared_experts": 1, "active_experts_with_shared": active,
                   "bytes_per_step": step_bytes},
        "tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "ms_routed_then_shared_mlp": round(ms_two, 5),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
    }


def run_gemm(args, cfg):
    """One w4a16_gemm call per step (dense weight, M x K x N).  Reported as
    TFLOP/s against the bf16 dense MFMA peak when M >= 512, else as GB/s."""
    import torch
    import int4_w4a16_group_g32_amd as L
    import workloads as W

    M, K, N = cfg.M, cfg.K, cfg.N
    xt = L.F32 if cfg.x_dtype == "f32" else L.BF16
    xbytes = 4 if cfg.x_dtype == "f32" else 2
    copies = []
    for c in range(max(1, args.copies)):
        copies.append(L.quantize_to_weight(W.weights(K, N, cfg.index, W.TAG_GATE, c, device="cuda")))
    x = W.activations(M, K, cfg.index, cfg.x_dtype, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(L.gemm_workspace_bytes(M, copies[0], xt))

    def step(i):
        L.gemm(x, copies[i % len(copies)], y, ws)

    for i in range(args.warmup):
        step(i)
    ms_step = timed_steps_ms(args, step)
    flops = 2.0 * M * K * N
    step_bytes = K * N * 5 // 8 + M * K * xbytes + M * N * 4
    tflops = flops / (ms_step * 1e-3) / 1e12
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    big = M >= 512
    return {
        "metric": METRIC, "value": round(tflops if big else gbs, 2), "unit": "TFLOP/s" if big else "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.x_dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "M": M, "K": K, "N": N, "bytes_per_step": step_bytes, "flops_per_step": flops},
        "pct_mfma_peak_bf16": round(100 * tflops / 2500.0, 1), "gbs": round(gbs, 1),
        **({} if args.no_cpu_baseline else {"cpu_baseline": cpu_baseline_gemm(cfg, x, big)}),
    }


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
    ms_step = timed_steps_ms(args, step)
    step_bytes = M * E * 4 + M * k * 8
    value = step_bytes / (ms_step * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "M": M, "experts": E, "top_k": k, "bytes_per_step": step_bytes},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
    }


def timed_steps_ms(args, step):
    """The timed region: exactly args.steps plain steps between two events,
    with a device synchronization on both sides."""
    import torch
    t0, t1 = _events(2)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / args.steps


def per_kernel_ms(args, names, step, cap=None, paired=False):
    """A second pass of args.steps steps through the *_timed entry point.
    paired: the library brackets kernel j with events 2j and 2j + 1, taken
    from the kernel's own dispatch (its execution time).  Otherwise it records
    an event before each of its kernels and one after the last, on the stream
    the kernels run on, and each interval also holds that kernel's dispatch
    gap.  Returns the mean milliseconds per kernel and the step time of this
    pass (the events themselves cost a few microseconds)."""
    import torch
    evs = [_events(cap or len(names) + 1) for _ in range(args.steps)]
    handles = [_handles(e) for e in evs]
    t0, t1 = _events(2)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i, handles[i])
    t1.record()
    torch.cuda.synchronize()
    if paired:
        kern = {n: statistics.mean(e[2 * j].elapsed_time(e[2 * j + 1]) for e in evs) for j, n in enumerate(names)}
    else:
        kern = {n: statistics.mean(e[j].elapsed_time(e[j + 1]) for e in evs) for j, n in enumerate(names)}
    return kern, t0.elapsed_time(t1) / args.steps


def _blas_threads():
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])


def cpu_baseline_moe(cfg, ids_np, wts, x, tokens=2, repeats=3):
    """The oracle's float64 MoE layer on a bounded sample: the first `tokens`
    tokens, through every expert they are routed to (weights drawn by the
    same generator and quantized by the oracle, not timed).  Value in the
    metric's unit: the sample's algorithmic bytes (its experts' weights, its
    activations and outputs) per second of oracle time."""
    import numpy as np
    import oracle as O
    import workloads as W

    E, H, I = cfg.experts, cfg.K, cfg.N
    sample = np.arange(tokens)
    experts = np.unique(ids_np[sample])
    codes = {}
    for e in experts:
        codes[int(e)] = tuple(O.quantize_w4a16(W.weights(K, N, cfg.index, tag, int(e), device="cuda").cpu().numpy())
                              for tag, (K, N) in ((W.TAG_GATE, (H, I)), (W.TAG_UP, (H, I)), (W.TAG_DOWN, (I, H))))
    xs = x.float().cpu().numpy()
    w_np = wts.cpu().numpy()
    times = []
    for _ in range(repeats):
        t = time.perf_counter()
        O.moe64(xs, ids_np, w_np, lambda e: codes[e], E, tokens=sample)
        times.append(time.perf_counter() - t)
    sec = statistics.median(times)
    xbytes = 4 if cfg.x_dtype == "f32" else 2
    nbytes = len(experts) * 3 * H * I * 5 // 8 + tokens * H * (xbytes + 4)
    return {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"{tokens} of the {cfg.M} tokens through their {len(experts)} experts ({nbytes} algorithmic "
                      f"bytes), numpy float64 dequantize-then-matmul, median of {repeats} runs of {sec:.2f}s",
            "seconds": round(sec, 3)}


def cpu_baseline_gemm(cfg, x, big, repeats=3):
    """The oracle's float64 GEMM (dequantize, then matmul) on the whole
    workload, the weights drawn by the same generator and quantized by the
    oracle (not timed); in TFLOP/s when M >= 512, else GB/s."""
    import oracle as O
    import workloads as W

    M, K, N = cfg.M, cfg.K, cfg.N
    qw, sc = O.quantize_w4a16(W.weights(K, N, cfg.index, W.TAG_GATE, 0, device="cuda").cpu().numpy())
    xs = x.float().cpu().numpy()
    times = []
    for _ in range(repeats):
        t = time.perf_counter()
        O.gemm64(xs, qw, sc)
        times.append(time.perf_counter() - t)
    sec = statistics.median(times)
    xbytes = 4 if cfg.x_dtype == "f32" else 2
    nbytes = K * N * 5 // 8 + M * K * xbytes + M * N * 4
    value = 2.0 * M * K * N / sec / 1e12 if big else nbytes / sec / 1e9
    return {"value": round(value, 6), "unit": "TFLOP/s" if big else "GB/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"the whole {cfg.name} GEMM, numpy float64 dequantize-then-matmul, median of {repeats} runs "
                      f"of {sec:.3f}s", "seconds": round(sec, 4)}


def cpu_baseline_mlp(cfg, base, repeats=7):
    """The oracle's float64 SwiGLU MLP (dequantize, then matmul) on the same
    weights and activations, median of `repeats` runs, after the oracle has
    quantized the weights itself (not timed).  Value in the metric's unit:
    algorithmic bytes of the workload per second of oracle time."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle as O
    import workloads as W

    H, I, M = cfg.K, cfg.N, cfg.M
    Is = I
    g = W.weights(H, I, cfg.index, W.TAG_GATE, device="cuda").cpu().numpy()
    u = W.weights(H, I, cfg.index, W.TAG_UP, device="cuda").cpu().numpy()
    d = W.weights(I, H, cfg.index, W.TAG_DOWN, device="cuda").cpu().numpy()
    codes = [O.quantize_w4a16(np.ascontiguousarray(a)) for a in (g, u, d)]
    del g, u, d
    x = W.activations(M, H, cfg.index, cfg.x_dtype, device="cuda").float().cpu().numpy()
    times = []
    for _ in range(repeats):
        t = time.perf_counter()
        O.swiglu_mlp64(x, *codes)
        times.append(time.perf_counter() - t)
    sec = statistics.median(times)
    xbytes = 4 if cfg.x_dtype == "f32" else 2
    nbytes = mlp_bytes(M, H, Is, xbytes)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole {cfg.name} step ({nbytes} algorithmic bytes), numpy float64 "
                      f"dequantize-then-matmul, median of {repeats} runs of {sec:.2f}s",
            "seconds": round(sec, 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mlp_decode_m4")
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr, flush=True)
        sys.exit(2)

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    cfg = W.CONFIGS[args.workload]
    if cfg.kind == "mlp":
        result = run_mlp(args, cfg)
    elif cfg.kind == "moe":
        result = run_moe(args, cfg)
    elif cfg.kind == "router":
        result = run_router(args, cfg)
    elif cfg.kind == "gemm":
        result = run_gemm(args, cfg)
    else:
        print(f"workload {cfg.name} has no bench line", file=sys.stderr)
        sys.exit(2)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
