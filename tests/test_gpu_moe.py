"""GPU parity of expert routing (bit-exact) and of the routed MoE layer
(relative Frobenius error vs the oracle's float64 MoE)."""
import numpy as np
import pytest
import torch

import int4_w4a16_group_g32_amd as L
import oracle as O
import workloads as W
from helpers import oracle_quantize_stack, rel_err, to_dev, tol_for, weight_from_codes, x_for_dtype, x_values

pytestmark = pytest.mark.gpu


def _route_gpu(ids_np, E):
    M, k = ids_np.shape
    ids = to_dev(ids_np.astype(np.int32))
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    sp = torch.full((max(1, M * k),), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((max(1, M * k),), -7, dtype=torch.int32, device="cuda")
    L.moe_route(ids, E, counts, offsets, sp, inv)
    torch.cuda.synchronize()
    return (counts.cpu().numpy(), offsets.cpu().numpy(), sp.cpu().numpy()[:M * k], inv.cpu().numpy()[:M * k])


@pytest.mark.parametrize("M,E,k,kind", [(1, 8, 2, "uniform"), (64, 384, 8, "uniform"),
                                        (2048, 384, 8, "zipf"), (300, 16, 4, "uniform"),
                                        (5000, 1000, 6, "uniform"), (4096, 3, 1, "uniform")])
def test_route_bit_exact(M, E, k, kind):
    ids = (W.topk_zipf(M, E, k, 1.1, 900) if kind == "zipf" else W.topk_uniform(M, E, k, 900 + M))
    got = _route_gpu(ids, E)
    want = O.route(ids, E)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


def test_route_skips_out_of_range_ids():
    ids = np.array([[0, 5], [9, 1], [-1, 2], [3, 4]], dtype=np.int32)
    counts, offsets, sp, inv = _route_gpu(ids, 6)
    ok = (ids >= 0) & (ids < 6)
    c, o, s, i = O.route(np.where(ok, ids, 0), 6)
    # the oracle on the valid pairs only: drop the two invalid pairs from its lists
    valid_pairs = np.flatnonzero(ok.reshape(-1))
    want_sp = [p for p in np.argsort(np.where(ok, ids, 99).reshape(-1), kind="stable") if p in valid_pairs]
    assert sp[:len(want_sp)].tolist() == want_sp
    assert inv[~ok.reshape(-1)].tolist() == [-1, -1]
    assert counts.tolist() == np.bincount(ids[ok], minlength=6).tolist()


def _experts(E, H, I, cfg):
    gs = [W.weights(H, I, cfg, W.TAG_GATE, e).numpy() for e in range(E)]
    us = [W.weights(H, I, cfg, W.TAG_UP, e).numpy() for e in range(E)]
    ds = [W.weights(I, H, cfg, W.TAG_DOWN, e).numpy() for e in range(E)]
    return oracle_quantize_stack(gs), oracle_quantize_stack(us), oracle_quantize_stack(ds)


def _moe_gpu(x, ids, wts, g, u, d):
    M, k = ids.shape
    xt = L.F32 if x.dtype == torch.float32 else L.BF16
    ws = L.new_workspace(L.moe_workspace_bytes(M, k, xt, g, u, d))
    y = torch.full((M, g.K), float("nan"), dtype=torch.float32, device="cuda")
    L.moe_grouped(x, ids, wts, g, u, d, y, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,E,k,H,I,routing", [
    (1, 4, 2, 64, 128, "uniform"), (9, 8, 3, 128, 64, "uniform"), (40, 6, 2, 256, 128, "uniform"),
    (64, 16, 8, 64, 64, "uniform"),
    (24, 16, 8, 128, 128, "uniform"),   # 9-16 rows per expert: GEMV items for bf16, tiles for float32
    (40, 16, 8, 128, 128, "uniform"),   # 14-26 rows per expert: 64-row tiles with one or two live row blocks
    (200, 4, 2, 128, 256, "uniform"),   # every expert heavy: MFMA tiles only, ragged last tile
    (300, 64, 4, 256, 128, "zipf"),     # heavy head, light tail: both paths in one call
])
def test_moe_small(M, E, k, H, I, routing, dtype):
    cfg = 500 + M
    (gq, gs), (uq, us), (dq, ds) = _experts(E, H, I, cfg)
    g, u, d = weight_from_codes(gq, gs), weight_from_codes(uq, us), weight_from_codes(dq, ds)
    ids = W.topk_zipf(M, E, k, 1.1, cfg) if routing == "zipf" else W.topk_uniform(M, E, k, cfg)
    counts = np.bincount(ids.ravel(), minlength=E)
    if routing == "zipf":
        assert counts.max() > 64 and (counts[counts > 0] <= 8).any()
    wts = W.gate_weights(M, k, cfg)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    y = _moe_gpu(x, to_dev(ids), to_dev(wts), g, u, d)
    ref = O.moe64(x_values(x), ids, wts, lambda e: ((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])), E)
    err = rel_err(y, ref)
    print(f"moe M={M} E={E} k={k} H={H} I={I} {dtype} relF={err:.3e}", flush=True)
    assert err <= tol_for(dtype)


@pytest.mark.parametrize("M,E,k,H,I", [(600, 4, 2, 256, 192), (1000, 8, 3, 128, 128)])
def test_moe_all_heavy_bf16(M, E, k, H, I):
    """bf16 activations with every expert above 128 rows: only MFMA items, the
    last of each expert ragged, I = 192 not a multiple of the tile's 128 h
    columns."""
    cfg = 520 + M
    (gq, gs), (uq, us), (dq, ds) = _experts(E, H, I, cfg)
    g, u, d = weight_from_codes(gq, gs), weight_from_codes(uq, us), weight_from_codes(dq, ds)
    ids = W.topk_uniform(M, E, k, cfg)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.min() >= 128 and (counts % 256 != 0).all()
    wts = W.gate_weights(M, k, cfg)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), "bf16")
    y = _moe_gpu(x, to_dev(ids), to_dev(wts), g, u, d)
    ref = O.moe64(x_values(x), ids, wts, lambda e: ((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])), E)
    err = rel_err(y, ref)
    print(f"moe all-heavy M={M} E={E} k={k} H={H} I={I} bf16 relF={err:.3e}", flush=True)
    assert err <= tol_for("bf16")


def _full_moe(name, sample_tokens):
    """Full expert stacks drawn and quantized on the GPU; the oracle regenerates
    and quantizes only the experts that the sampled tokens use."""
    cfg = W.CONFIGS[name]
    E, H, I, M, k = cfg.experts, cfg.K, cfg.N, cfg.M, cfg.top_k
    if cfg.routing == "zipf":
        ids = W.topk_zipf(M, E, k, cfg.zipf_alpha, cfg.index)
    else:
        ids = W.topk_uniform(M, E, k, cfg.index)
    wts = W.gate_weights(M, k, cfg.index)
    stacks = {}
    for tag, (K, N) in ((W.TAG_GATE, (H, I)), (W.TAG_UP, (H, I)), (W.TAG_DOWN, (I, H))):
        qw = torch.empty((E, K // 8, N), dtype=torch.int32, device="cuda")
        sc = torch.empty((E, K // 32, N), dtype=torch.float32, device="cuda")
        for e in range(E):
            w = W.weights(K, N, cfg.index, tag, e, device="cuda")
            L.quantize(w, qw[e], sc[e])
        canon = L.Weight(qw, sc, K, N, E, L.LAYOUT_CANONICAL)
        stacks[tag] = L.prepack(canon, torch.empty_like(qw))
        del canon, qw
    torch.cuda.synchronize()
    x = x_for_dtype(W.activations(M, H, cfg.index).cuda(), cfg.x_dtype)
    y = _moe_gpu(x, to_dev(ids), to_dev(wts), stacks[W.TAG_GATE], stacks[W.TAG_UP], stacks[W.TAG_DOWN])
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = tuple(O.quantize_w4a16(W.weights(K, N, cfg.index, tag, e, device="cuda").cpu().numpy())
                             for tag, (K, N) in ((W.TAG_GATE, (H, I)), (W.TAG_UP, (H, I)), (W.TAG_DOWN, (I, H))))
        return cache[e]

    ref = O.moe64(x_values(x), ids, wts, expert, E, tokens=sample_tokens)
    err = rel_err(y[torch.as_tensor(sample_tokens, device="cuda")], ref)
    print(f"{name} relF={err:.3e} on tokens {list(sample_tokens)} ({len(cache)} experts)", flush=True)
    assert err <= tol_for(cfg.x_dtype)
    assert torch.isfinite(y).all()


def test_moe_decode_full_size():
    _full_moe("moe_decode_m64", [0, 37])


def test_moe_prefill_full_size():
    """2048 tokens, Zipf(1.1) routing: the sampled tokens include one routed to
    the most popular expert (over a thousand rows, MFMA tiles) and their other
    experts cover the light tail."""
    cfg = W.CONFIGS["moe_prefill_m2048"]
    ids = W.topk_zipf(cfg.M, cfg.experts, cfg.top_k, cfg.zipf_alpha, cfg.index)
    counts = np.bincount(ids.ravel(), minlength=cfg.experts)
    hot = int(np.argmax(counts))
    t_hot = int(np.argwhere((ids == hot).any(axis=1))[0, 0])
    _full_moe("moe_prefill_m2048", [t_hot, 2047])
