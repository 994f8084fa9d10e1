"""Element-wise error bounds for the parity tests, and a process pool that
evaluates the oracle's independent per-expert MLPs in parallel.

Imports only numpy and the oracle, so worker processes start quickly.

The bound on one output element.  A computed dot product differs from the
exact one by at most a small multiple of the sum of the magnitudes of its
terms (oracle.gemm_abs64 computes that sum).  The library's arithmetic gives
per product a relative error of about 2^-22 with float32 activations (two f16
pieces of each activation, exact codes, float32 scales and accumulation) and
about 2^-10 with bf16 activations on the tiles (scale folded into an f16
weight, the intermediate h as one f16 piece).  The tolerance factors below
sit 8x above those, and each bound also carries a floor of
2^-11 * tau * (the row's largest term sum) for the activations that the
power-of-two staging leaves more than 2^17 below their row's largest one.
A single wrong element is typically mag / sqrt(K) away from the reference,
more than ten times any of these bounds at the tested sizes.

For a SwiGLU MLP the gate and up errors are carried through h = silu(g) * u
(|silu'| <= 1.1 everywhere) into the down projection, whose own error is
added on top.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

import oracle as O

TAU = {"f32": 2.0 ** -19, "bf16": 2.0 ** -8}
SILU_SLOPE_MAX = 1.1  # max over z of |d/dz z / (1 + e^-z)| is 1.0998
POOL_WORKERS = 16


def floor_bound(mag: np.ndarray, tau: float) -> np.ndarray:
    """tau * (mag + 2^-11 * row max of mag): the per-element bound from the
    term-magnitude sums mag[..., n]."""
    mag = np.asarray(mag, dtype=np.float64)
    if mag.size == 0:
        return mag
    return tau * (mag + 2.0 ** -11 * mag.max(axis=-1, keepdims=True))


def gemm_bound(x, qw, sc, tau) -> np.ndarray:
    return floor_bound(O.gemm_abs64(x, qw, sc), tau)


def dequant_f32(qw, sc) -> np.ndarray:
    """float32(q * s) from the words' bytes (byte j of word i holds rows
    8i + 2j in its low nibble and 8i + 2j + 1 in its high one).  Equal to
    oracle.dequant32 bit for bit (a CPU test checks it) and several times
    faster; the bounds use it, the parity references never do."""
    qw = np.ascontiguousarray(qw, dtype=np.int32)
    Kw, N = qw.shape
    b = qw.view(np.uint8).reshape(Kw, N, 4)
    q = np.empty((Kw, 4, 2, N), dtype=np.float32)
    q[:, :, 0, :] = (b & 0xF).transpose(0, 2, 1)
    q[:, :, 1, :] = (b >> 4).transpose(0, 2, 1)
    q -= 8.0
    sc = np.asarray(sc, dtype=np.float32)
    q = q.reshape(sc.shape[0], -1, N)
    q *= sc[:, None, :]
    return q.reshape(Kw * 8, N)


def mlp_bound(x, gate, up, down, tau) -> np.ndarray:
    """Per-element bound of the SwiGLU MLP's output (float32 arithmetic: a
    bound needs no more)."""
    x = np.asarray(x, dtype=np.float32)
    dg, du = dequant_f32(*gate), dequant_f32(*up)
    g, u = (x @ dg).astype(np.float64), (x @ du).astype(np.float64)
    ax = np.abs(x)
    eg = floor_bound(ax @ np.abs(dg), tau)
    eu = floor_bound(ax @ np.abs(du), tau)
    s = O.silu64(g)
    h = s * u
    eh = SILU_SLOPE_MAX * eg * (np.abs(u) + eu) + np.abs(s) * eu + tau * np.abs(h)
    ad = np.abs(dequant_f32(*down))
    return (eh.astype(np.float32) @ ad + floor_bound(((np.abs(h) + eh).astype(np.float32) @ ad), tau)) * (1 + 2.0 ** -10)


def _value_and_bound(args):
    fn, job, tau = args
    xs, gate, up, down = job
    return fn(job), mlp_bound(xs, gate, up, down, tau)


class ExpertPool:
    """map_fn for oracle.moe64: runs the oracle's per-expert function in worker
    processes (spawned, one BLAS thread each; workers=0 runs them in this
    process) and keeps, in the same order, each expert's per-element bound."""

    def __init__(self, tau: float, workers: int = POOL_WORKERS, batch: int = 32):
        self.tau = tau
        self.batch = batch
        self.bounds = []
        self.ex = None
        if workers == 0:
            return
        saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
        for k in saved:
            os.environ[k] = "1"
        try:
            n = max(1, min(workers, os.cpu_count() or 1))
            self.ex = ProcessPoolExecutor(n, mp_context=mp.get_context("spawn"))
            list(self.ex.map(int, range(n)))  # start the workers while the environment says one thread
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    def __call__(self, fn, jobs):
        pending = []
        for job in jobs:
            pending.append((fn, job, self.tau))
            if len(pending) == self.batch:
                yield from self._run(pending)
                pending = []
        if pending:
            yield from self._run(pending)

    def _run(self, items):
        results = map(_value_and_bound, items) if self.ex is None else self.ex.map(_value_and_bound, items)
        for value, bound in results:
            self.bounds.append(bound)
            yield value

    def close(self):
        if self.ex is not None:
            self.ex.shutdown()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def moe_bound_from(pool_bounds, topk_ids, topk_w, tokens=None) -> np.ndarray:
    """Per-element bound of a MoE layer's output from the per-expert bounds
    that ExpertPool collected while oracle.moe64 ran (same expert order: sorted
    ids, rows in token order): the sum over slots of |w| * the bound of that
    slot's expert row.  (The combine's own float32 rounding, about 2^-21 of
    sum |w| |o|, lies far inside the tau * |o| that each expert bound holds.)"""
    ids = np.asarray(topk_ids, dtype=np.int64)
    wts = np.abs(np.asarray(topk_w, dtype=np.float64))
    M, k = ids.shape
    rows = np.arange(M) if tokens is None else np.asarray(tokens, dtype=np.int64)
    sub = ids[rows]
    experts = np.unique(sub)
    assert len(experts) == len(pool_bounds)
    H = pool_bounds[0].shape[1]
    out = np.zeros((len(rows), H))
    for e, b in zip(experts, pool_bounds):
        sel = np.argwhere(sub == e)
        for (r, s), v in zip(sel, b):
            out[r] += wts[rows[r], s] * v
    return out


def check_elementwise(y, ref, bound, what: str) -> float:
    """Every |y - ref| <= bound; returns the largest ratio |y - ref| / bound."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape == bound.shape, (y.shape, ref.shape, bound.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    d = np.abs(y - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, d / bound, np.where(d > 0, np.inf, 0.0))
    worst = float(r.max()) if r.size else 0.0
    bad = int((d > bound).sum())
    assert bad == 0, f"{what}: {bad} of {d.size} elements exceed the element-wise bound (worst ratio {worst:.3g})"
    return worst
