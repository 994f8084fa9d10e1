"""GPU parity on a seeded sweep of shapes that no other test picks by hand:
w4a16_gemm and w4a16_swiglu_mlp at random row counts (the GEMV, the 64-row
tiles with and without K splits, the wide tiles from 256 bf16 rows) and
random K and N (multiples of 64), and w4a16_moe_grouped at random token,
expert and top-k counts under uniform and Zipf routing, all with random code
words (every nibble, q = -8 included) and scales, against the oracle's
float64 result: relative Frobenius error and the element-wise bound."""
import numpy as np
import pytest
import torch

import int4_w4a16_group_g32_amd as L
import oracle as O
import workloads as W
from helpers import rel_err, tol_for, weight_from_codes, x_for_dtype, x_values
from oracle_pool import TAU, check_elementwise, gemm_bound, mlp_bound

pytestmark = pytest.mark.gpu


def _codes(K, N, rng):
    qw = rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint64).astype(np.uint32).view(np.int32)
    sc = (rng.random((K // 32, N)) * 0.006 + 0.002).astype(np.float32)
    return qw, sc


def _gemm_cases():
    rng = np.random.default_rng(20260)
    cases = []
    for i in range(24):
        M = int(rng.choice([1, 2, 4, 7, 8, 12, 16, 20, 33, 64, 70, 100, 128, 200, 256, 300]))
        K = 64 * int(rng.integers(1, 33))
        N = 64 * int(rng.integers(1, 33))
        cases.append((i, M, K, N, "bf16" if i % 2 else "f32"))
    return cases


def _mlp_cases():
    rng = np.random.default_rng(20261)
    cases = []
    for i in range(12):
        M = int(rng.choice([1, 3, 8, 9, 16, 17, 40, 64, 96, 130]))
        H = 64 * int(rng.integers(1, 25))
        I = 64 * int(rng.integers(1, 25))
        cases.append((i, M, H, I, "bf16" if i % 2 else "f32"))
    return cases


@pytest.mark.parametrize("i,M,K,N,dtype", _gemm_cases())
def test_gemm_shape_sweep(i, M, K, N, dtype):
    rng = np.random.default_rng(700 + i)
    qw, sc = _codes(K, N, rng)
    w = weight_from_codes(qw, sc)
    x = x_for_dtype(W.activations(M, K, 700 + i).cuda(), dtype)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(L.gemm_workspace_bytes(M, w, L.F32 if dtype == "f32" else L.BF16))
    L.gemm(x, w, y, ws)
    torch.cuda.synchronize()
    xv = x_values(x)
    ref = O.gemm64(xv, qw, sc)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, gemm_bound(xv, qw, sc, TAU[dtype]),
                              f"gemm sweep M={M} K={K} N={N} {dtype}")
    print(f"gemm sweep M={M} K={K} N={N} {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)


@pytest.mark.parametrize("i,M,H,I,dtype", _mlp_cases())
def test_mlp_shape_sweep(i, M, H, I, dtype):
    rng = np.random.default_rng(800 + i)
    codes = [_codes(H, I, rng), _codes(H, I, rng), _codes(I, H, rng)]
    g, u, d = (weight_from_codes(*c) for c in codes)
    x = x_for_dtype(W.activations(M, H, 800 + i).cuda(), dtype)
    xt = L.F32 if dtype == "f32" else L.BF16
    y = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(L.swiglu_mlp_workspace_bytes(M, xt, g, u, d))
    L.swiglu_mlp(x, g, u, d, y, ws)
    torch.cuda.synchronize()
    xv = x_values(x)
    ref = O.swiglu_mlp64(xv, *codes)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, mlp_bound(xv, *codes, TAU[dtype]),
                              f"mlp sweep M={M} H={H} I={I} {dtype}")
    print(f"mlp sweep M={M} H={H} I={I} {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)


def _moe_cases():
    rng = np.random.default_rng(20262)
    cases = []
    for i in range(10):
        M = int(rng.choice([1, 4, 9, 16, 17, 40, 64, 100, 200, 300]))
        E = int(rng.integers(2, 65))
        k = int(rng.integers(1, min(8, E) + 1))
        H = 64 * int(rng.integers(1, 9))
        I = 64 * int(rng.integers(1, 9))
        cases.append((i, M, E, k, H, I, "zipf" if i % 3 == 0 else "uniform", "bf16" if i % 2 else "f32"))
    return cases


@pytest.mark.parametrize("i,M,E,k,H,I,routing,dtype", _moe_cases())
def test_moe_shape_sweep(i, M, E, k, H, I, routing, dtype):
    from test_gpu_moe import _moe_gpu, _moe_ref, _random_expert_codes
    from helpers import to_dev

    cfg = 900 + i
    (gq, gs), (uq, us), (dq, ds) = _random_expert_codes(E, H, I, cfg)
    g, u, d = (weight_from_codes(*c) for c in ((gq, gs), (uq, us), (dq, ds)))
    ids = W.topk_zipf(M, E, k, 1.1, cfg) if routing == "zipf" else W.topk_uniform(M, E, k, cfg)
    wts = W.gate_weights(M, k, cfg)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    y = _moe_gpu(x, to_dev(ids), to_dev(wts), g, u, d)
    ref, bound = _moe_ref(x, ids, wts, lambda e: ((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])), E, dtype)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, bound, f"moe sweep M={M} E={E} k={k} {dtype}")
    rows = np.bincount(ids.ravel(), minlength=E)
    print(f"moe sweep M={M} E={E} k={k} H={H} I={I} {routing} {dtype} rows/expert {rows.min()}..{rows.max()} "
          f"relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)
