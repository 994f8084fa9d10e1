"""GPU parity of the MoE layer with a shared expert (w4a16_moe_grouped_shared)
against the oracle's moe_shared64: relative Frobenius error <= 1e-5 for
float32 activations and <= 1e-2 for bf16; with all-zero shared scales the
result is bitwise that of w4a16_moe_grouped (the shared term adds +0)."""
import numpy as np
import pytest
import torch

import int4_w4a16_group_g32_amd as L
import oracle as O
import workloads as W
from helpers import oracle_quantize_stack, rel_err, to_dev, tol_for, weight_from_codes, x_for_dtype, x_values
from oracle_pool import TAU, ExpertPool, check_elementwise, mlp_bound, moe_bound_from

pytestmark = pytest.mark.gpu

SHARED_INDEX = W.SHARED_EXPERT_INDEX


def _stacks(E, H, I, cfg, first=0):
    gs = [W.weights(H, I, cfg, W.TAG_GATE, first + e).numpy() for e in range(E)]
    us = [W.weights(H, I, cfg, W.TAG_UP, first + e).numpy() for e in range(E)]
    ds = [W.weights(I, H, cfg, W.TAG_DOWN, first + e).numpy() for e in range(E)]
    return oracle_quantize_stack(gs), oracle_quantize_stack(us), oracle_quantize_stack(ds)


def _run_shared(x, ids, wts, routed, shared):
    M, k = ids.shape
    xt = L.F32 if x.dtype == torch.float32 else L.BF16
    ws = L.new_workspace(L.moe_shared_workspace_bytes(M, k, xt, *routed, *shared))
    y = torch.full((M, routed[0].K), float("nan"), dtype=torch.float32, device="cuda")
    L.moe_grouped_shared(x, ids, wts, *routed, *shared, y, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,E,k,H,I", [(1, 4, 2, 64, 128), (5, 6, 2, 128, 64), (9, 8, 3, 128, 64),
                                       (64, 16, 8, 64, 64), (130, 6, 2, 256, 128), (300, 8, 2, 128, 64)])
def test_moe_shared_small(M, E, k, H, I, dtype):
    """M <= 64: the shared expert is GEMV items of 8 rows; M > 64: MFMA tiles
    (130 rows: a ragged last tile) next to the routed experts' items (M = 300:
    five tiles)."""
    cfg = 700 + M
    (gq, gs), (uq, us), (dq, ds) = _stacks(E, H, I, cfg)
    (sgq, sgs), (suq, sus), (sdq, sds) = _stacks(1, H, I, cfg, first=SHARED_INDEX)
    routed = (weight_from_codes(gq, gs), weight_from_codes(uq, us), weight_from_codes(dq, ds))
    shared = (weight_from_codes(sgq, sgs), weight_from_codes(suq, sus), weight_from_codes(sdq, sds))
    ids = W.topk_uniform(M, E, k, cfg)
    wts = W.gate_weights(M, k, cfg)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    y = _run_shared(x, to_dev(ids), to_dev(wts), routed, shared)
    sh = ((sgq[0], sgs[0]), (suq[0], sus[0]), (sdq[0], sds[0]))
    ref, bound = _shared_ref(x, ids, wts, lambda e: ((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])), E, sh,
                             dtype)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, bound, f"moe+shared M={M} {dtype}")
    print(f"moe+shared M={M} E={E} k={k} H={H} I={I} {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)


def _shared_ref(x, ids, wts, expert, E, shared, dtype, tokens=None, workers=0):
    """The oracle's routed-plus-shared output and its per-element bound."""
    xv = x_values(x)
    with ExpertPool(TAU[dtype], workers=workers) as pool:
        ref = O.moe_shared64(xv, ids, wts, expert, E, shared, tokens=tokens, map_fn=pool)
        bound = moe_bound_from(pool.bounds, ids, wts, tokens)
    rows = np.arange(xv.shape[0]) if tokens is None else np.asarray(tokens)
    return ref, bound + mlp_bound(xv[rows], *shared, TAU[dtype])


@pytest.mark.parametrize("M", [4, 64])
def test_moe_shared_zero_scales_equal_routed_only(M):
    E, k, H, I = 8, 2, 128, 64
    cfg = 800 + M
    (gq, gs), (uq, us), (dq, ds) = _stacks(E, H, I, cfg)
    (sgq, sgs), (suq, sus), (sdq, sds) = _stacks(1, H, I, cfg, first=SHARED_INDEX)
    routed = (weight_from_codes(gq, gs), weight_from_codes(uq, us), weight_from_codes(dq, ds))
    shared = (weight_from_codes(sgq, sgs), weight_from_codes(suq, sus),
              weight_from_codes(sdq, np.zeros_like(sds)))
    ids = to_dev(W.topk_uniform(M, E, k, cfg))
    wts = to_dev(W.gate_weights(M, k, cfg))
    x = W.activations(M, H, cfg).cuda()
    y_sh = _run_shared(x, ids, wts, routed, shared)
    ws = L.new_workspace(L.moe_workspace_bytes(M, k, L.F32, *routed))
    y = torch.empty_like(y_sh)
    L.moe_grouped(x, ids, wts, *routed, y, ws)
    torch.cuda.synchronize()
    assert torch.equal(y_sh, y)


def test_moe_shared_decode_full_size():
    """The MoE decode layer (64 tokens, 384 experts of 7168 -> 2048, top-8,
    bf16) with a shared expert of the same shape, quantized on the GPU; the
    oracle, on two tokens, quantizes the same float32 weights itself."""
    cfg = W.CONFIGS["moe_decode_m64"]
    E, H, I, M, k = cfg.experts, cfg.K, cfg.N, cfg.M, cfg.top_k
    ids = W.topk_uniform(M, E, k, cfg.index)
    wts = W.gate_weights(M, k, cfg.index)
    tags = ((W.TAG_GATE, (H, I)), (W.TAG_UP, (H, I)), (W.TAG_DOWN, (I, H)))
    stacks, shared = [], []
    for tag, (K, N) in tags:
        qw = torch.empty((E, K // 8, N), dtype=torch.int32, device="cuda")
        sc = torch.empty((E, K // 32, N), dtype=torch.float32, device="cuda")
        for e in range(E):
            L.quantize(W.weights(K, N, cfg.index, tag, e, device="cuda"), qw[e], sc[e])
        stacks.append(L.prepack(L.Weight(qw, sc, K, N, E, L.LAYOUT_CANONICAL), torch.empty_like(qw)))
        sq = torch.empty((1, K // 8, N), dtype=torch.int32, device="cuda")
        ss = torch.empty((1, K // 32, N), dtype=torch.float32, device="cuda")
        L.quantize(W.weights(K, N, cfg.index, tag, SHARED_INDEX, device="cuda"), sq[0], ss[0])
        shared.append(L.prepack(L.Weight(sq, ss, K, N, 1, L.LAYOUT_CANONICAL), torch.empty_like(sq)))
        del qw
    x = x_for_dtype(W.activations(M, H, cfg.index).cuda(), cfg.x_dtype)
    y = _run_shared(x, to_dev(ids), to_dev(wts), stacks, shared)
    cache = {}

    def weights_of(index):
        if index not in cache:
            cache[index] = tuple(O.quantize_w4a16(W.weights(K, N, cfg.index, tag, index, device="cuda").cpu().numpy())
                                 for tag, (K, N) in tags)
        return cache[index]

    tokens = [3, 50]
    ref = O.moe_shared64(x_values(x), ids, wts, weights_of, E, weights_of(SHARED_INDEX), tokens=tokens)
    err = rel_err(y[torch.as_tensor(tokens, device="cuda")], ref)
    print(f"moe_decode_m64 + shared relF={err:.3e} on tokens {tokens}", flush=True)
    assert err <= tol_for(cfg.x_dtype)
    assert torch.isfinite(y).all()


def test_moe_shared_decode_full_size_every_token():
    """The same layer with random code words (q = -8 included) drawn on the
    GPU: every token against the oracle, with the element-wise bound; the
    oracle's experts run in worker processes."""
    cfg = W.CONFIGS["moe_decode_m64"]
    E, H, I, M, k = cfg.experts, cfg.K, cfg.N, cfg.M, cfg.top_k
    ids = W.topk_uniform(M, E, k, cfg.index)
    wts = W.gate_weights(M, k, cfg.index)
    tags = ((W.TAG_GATE, (H, I)), (W.TAG_UP, (H, I)), (W.TAG_DOWN, (I, H)))
    canon, stacks, shared_dev, shared_np = {}, [], [], []
    for tag, (K, N) in tags:
        qw = torch.empty((E, K // 8, N), dtype=torch.int32, device="cuda")
        sc = torch.empty((E, K // 32, N), dtype=torch.float32, device="cuda")
        for e in range(E):
            qw[e] = W.code_words(K, N, cfg.index, tag, e, device="cuda")
            sc[e] = W.scale_values(K // 32, N, cfg.index, tag, e, device="cuda")
        canon[tag] = (qw, sc)
        stacks.append(L.prepack(L.Weight(qw, sc, K, N, E, L.LAYOUT_CANONICAL), torch.empty_like(qw)))
        sq = W.code_words(K, N, cfg.index, tag, SHARED_INDEX, device="cuda")[None].contiguous()
        ss = W.scale_values(K // 32, N, cfg.index, tag, SHARED_INDEX, device="cuda")[None].contiguous()
        shared_dev.append(L.prepack(L.Weight(sq, ss, K, N, 1, L.LAYOUT_CANONICAL), torch.empty_like(sq)))
        shared_np.append((sq[0].cpu().numpy(), ss[0].cpu().numpy()))
    torch.cuda.synchronize()
    x = x_for_dtype(W.activations(M, H, cfg.index).cuda(), cfg.x_dtype)
    y = _run_shared(x, to_dev(ids), to_dev(wts), stacks, shared_dev)

    def expert(e):
        return tuple((canon[t][0][e].cpu().numpy(), canon[t][1][e].cpu().numpy()) for t, _ in tags)

    ref, bound = _shared_ref(x, ids, wts, expert, E, tuple(shared_np), cfg.x_dtype, workers=16)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, bound, "moe_decode_m64 + shared")
    print(f"moe_decode_m64 + shared random codes relF={err:.3e} worst/bound={worst:.2e} on all {M} tokens",
          flush=True)
    assert err <= tol_for(cfg.x_dtype)
