"""Group sizes 64 and 128 (one scale per 64 or 128 rows) on every path:
quantizer and dequant bit-exact, GEMM / MLP / MoE within the relative
Frobenius bounds (1e-5 float32, 1e-2 bf16) of the oracle at the same group
size."""
import ctypes

import numpy as np
import pytest
import torch

import int4_w4a16_group_g32_amd as L
import oracle as O
import workloads as W
from helpers import oracle_quantize_stack, rel_err, to_dev, tol_for, weight_from_codes, x_for_dtype, x_values

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("K,N,E", [(256, 64, 1), (1024, 192, 2), (7168, 128, 1)])
def test_quantizer_bit_exact(group, K, N, E):
    w = torch.stack([W.weights(K, N, 950 + group, W.TAG_GATE, e) for e in range(E)])
    qw = torch.empty((E, K // 8, N), dtype=torch.int32, device="cuda")
    sc = torch.empty((E, K // group, N), dtype=torch.float32, device="cuda")
    L.quantize(w.cuda(), qw, sc, group_size=group)
    torch.cuda.synchronize()
    for e in range(E):
        rq, rs = O.quantize_w4a16(w[e].numpy(), group)
        assert np.array_equal(qw[e].cpu().numpy(), rq)
        assert np.array_equal(sc[e].cpu().numpy().view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("group", [64, 128])
def test_dequant_bit_exact_both_layouts(group):
    K, N = 512, 128
    qw, sc = O.quantize_w4a16(W.weights(K, N, 951, W.TAG_UP).numpy(), group)
    grouped = weight_from_codes(qw, sc)
    canon = L.Weight(to_dev(qw[None]), to_dev(sc[None]), K, N, 1, L.LAYOUT_CANONICAL, group)
    want = O.dequant32(qw, sc)
    for w in (canon, grouped):
        out = torch.empty((1, K, N), dtype=torch.float32, device="cuda")
        L.dequantize(w, out)
        torch.cuda.synchronize()
        assert np.array_equal(out[0].cpu().numpy().view(np.uint32), want.view(np.uint32))


def _gemm(x, w, N):
    y = torch.full((x.shape[0], N), float("nan"), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(L.gemm_workspace_bytes(x.shape[0], w, L.F32 if x.dtype == torch.float32 else L.BF16))
    L.gemm(x, w, y, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("M,K,N", [(1, 256, 512), (4, 7168, 256), (8, 1024, 192), (9, 1024, 64), (64, 7168, 256),
                                   (130, 512, 320), (300, 1024, 192), (513, 7168, 256)])
def test_gemm_other_group_sizes(M, K, N, group, dtype):
    """Every GEMM path (GEMV, 64-row tiles, and from 256 bf16 rows the wide
    tiles, with K splits at K = 7168) reads scale row k / group."""
    qw, sc = O.quantize_w4a16(W.weights(K, N, 960 + K + N, W.TAG_GATE).numpy(), group)
    w = weight_from_codes(qw, sc)
    x = x_for_dtype(W.activations(M, K, 961 + M).cuda(), dtype)
    y = _gemm(x, w, N)
    err = rel_err(y, O.gemm64(x_values(x), qw, sc))
    print(f"gemm g={group} M={M} K={K} N={N} {dtype} relF={err:.3e}", flush=True)
    assert err <= tol_for(dtype)


@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("M", [1, 4, 64])
def test_gemm_one_hot_rows_bit_exact(group, M):
    """Unit rows reproduce float32(q * s) of the row's group, on both paths."""
    K, N = 1024, 256
    qw, sc = O.quantize_w4a16(W.weights(K, N, 962, W.TAG_DOWN).numpy(), group)
    w = weight_from_codes(qw, sc)
    ks = np.random.default_rng(M + group).choice(K, size=M, replace=False)
    x = torch.zeros((M, K), dtype=torch.float32)
    x[torch.arange(M), torch.as_tensor(ks)] = 1.0
    y = _gemm(x.cuda(), w, N)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), O.dequant32(qw, sc)[ks].view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [3, 64])
def test_mlp_group_128(M, dtype):
    H, I = 512, 1024
    codes = [O.quantize_w4a16(W.weights(K, N, 963, tag).numpy(), 128)
             for K, N, tag in ((H, I, W.TAG_GATE), (H, I, W.TAG_UP), (I, H, W.TAG_DOWN))]
    ws_ = [weight_from_codes(*c) for c in codes]
    x = x_for_dtype(W.activations(M, H, 964 + M).cuda(), dtype)
    xt = L.F32 if dtype == "f32" else L.BF16
    y = torch.empty((M, H), dtype=torch.float32, device="cuda")
    L.swiglu_mlp(x, *ws_, y, L.new_workspace(L.swiglu_mlp_workspace_bytes(M, xt, *ws_)))
    torch.cuda.synchronize()
    err = rel_err(y, O.swiglu_mlp64(x_values(x), *codes))
    print(f"mlp g=128 M={M} {dtype} relF={err:.3e}", flush=True)
    assert err <= tol_for(dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_moe_group_64_mixed_paths_and_shared(dtype):
    """Zipf routing (heavy experts on MFMA tiles, light ones on the GEMV), with
    and without a shared expert, all at 64 rows per scale."""
    M, E, k, H, I, cfg = 300, 32, 4, 256, 128, 965
    stacks = []
    for tag, (K, N) in ((W.TAG_GATE, (H, I)), (W.TAG_UP, (H, I)), (W.TAG_DOWN, (I, H))):
        stacks.append(oracle_quantize_stack([W.weights(K, N, cfg, tag, e).numpy() for e in range(E + 1)], 64))
    routed = [weight_from_codes(q[:E], s[:E]) for q, s in stacks]
    shared = [weight_from_codes(q[E:], s[E:]) for q, s in stacks]
    ids = W.topk_zipf(M, E, k, 1.1, cfg)
    wts = W.gate_weights(M, k, cfg)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    xt = L.F32 if dtype == "f32" else L.BF16
    expert = lambda e: tuple((q[e], s[e]) for q, s in stacks)
    y = torch.empty((M, H), dtype=torch.float32, device="cuda")
    L.moe_grouped(x, to_dev(ids), to_dev(wts), *routed, y,
                  L.new_workspace(L.moe_workspace_bytes(M, k, xt, *routed)))
    torch.cuda.synchronize()
    err = rel_err(y, O.moe64(x_values(x), ids, wts, expert, E))
    assert err <= tol_for(dtype)
    L.moe_grouped_shared(x, to_dev(ids), to_dev(wts), *routed, *shared, y,
                         L.new_workspace(L.moe_shared_workspace_bytes(M, k, xt, *routed, *shared)))
    torch.cuda.synchronize()
    err2 = rel_err(y, O.moe_shared64(x_values(x), ids, wts, expert, E, expert(E)))
    print(f"moe g=64 {dtype} relF={err:.3e}, with shared {err2:.3e}", flush=True)
    assert err2 <= tol_for(dtype)


def test_mixed_group_sizes_in_one_launch_are_rejected():
    """Gate and up stream through one launch, so they must share a group size
    (checked on the host before anything is launched)."""
    H, I = 256, 128
    g = weight_from_codes(*O.quantize_w4a16(W.weights(H, I, 966, W.TAG_GATE).numpy(), 64))
    u = weight_from_codes(*O.quantize_w4a16(W.weights(H, I, 966, W.TAG_UP).numpy(), 32))
    d = weight_from_codes(*O.quantize_w4a16(W.weights(I, H, 966, W.TAG_DOWN).numpy(), 32))
    assert L.load_library().w4a16_swiglu_mlp_workspace_bytes(4, L.F32, ctypes.byref(g.desc()),
                                                             ctypes.byref(u.desc()), ctypes.byref(d.desc())) == 0
