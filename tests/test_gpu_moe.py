"""GPU parity of expert routing (bit-exact) and of the routed MoE layer
against the oracle's float64 MoE: relative Frobenius error and a bound on
every output element (tests/oracle_pool.py)."""
import numpy as np
import pytest
import torch

import int4_w4a16_group_g32_amd as L
import oracle as O
import workloads as W
from helpers import oracle_quantize_stack, rel_err, to_dev, tol_for, weight_from_codes, x_for_dtype, x_values
from oracle_pool import TAU, ExpertPool, check_elementwise, moe_bound_from

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
                                        (5000, 1000, 6, "uniform"), (4096, 3, 1, "uniform"),
                                        # more experts than the route kernel's 1024 threads: its scans
                                        # over experts run in several blocks with a carry
                                        (3000, 2500, 4, "uniform"), (1024, 6144, 8, "zipf")])
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
    ref, bound = _moe_ref(x, ids, wts, lambda e: ((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])), E, dtype)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, bound, f"moe M={M} E={E} k={k} {dtype}")
    print(f"moe M={M} E={E} k={k} H={H} I={I} {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)


def _moe_ref(x, ids, wts, expert, E, dtype, tokens=None, workers=0):
    """The oracle's MoE output and the per-element bound for it."""
    with ExpertPool(TAU[dtype], workers=workers) as pool:
        ref = O.moe64(x_values(x), ids, wts, expert, E, tokens=tokens, map_fn=pool)
        bound = moe_bound_from(pool.bounds, ids, wts, tokens)
    return ref, bound


def _random_expert_codes(E, H, I, seed):
    rng = np.random.default_rng(seed)
    out = []
    for K, N in ((H, I), (H, I), (I, H)):
        qw = rng.integers(0, 2 ** 32, size=(E, K // 8, N), dtype=np.uint64).astype(np.uint32).view(np.int32)
        out.append((qw, (rng.random((E, K // 32, N)) * 0.005 + 0.004).astype(np.float32)))
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_moe_more_experts_than_route_threads(dtype):
    """1500 experts under Zipf routing: the work-item scans over experts run
    in two blocks of 1024, with both GEMV and MFMA items."""
    M, E, k, H, I = 300, 1500, 4, 64, 64
    cfg = 660
    ids = W.topk_zipf(M, E, k, 1.1, cfg)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.max() > 64 and ((counts > 0) & (counts <= 8)).sum() > 100
    (gq, gs), (uq, us), (dq, ds) = _experts(E, H, I, cfg)
    g, u, d = weight_from_codes(gq, gs), weight_from_codes(uq, us), weight_from_codes(dq, ds)
    wts = W.gate_weights(M, k, cfg)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    y = _moe_gpu(x, to_dev(ids), to_dev(wts), g, u, d)
    ref, bound = _moe_ref(x, ids, wts, lambda e: ((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])), E, dtype)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, bound, f"moe E={E} {dtype}")
    print(f"moe E={E} M={M} k={k} {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)


# Rows per expert on both sides of every item boundary: the GEMV limit
# (8 rows with float32 activations, 16 with bf16), the partial 64-row tile
# classes (1-16, 17-32, 33-63 rows) and whole tiles (64, 128) plus one row.
_ROW_COUNTS = [1, 8, 9, 15, 16, 17, 31, 32, 33, 42, 63, 64, 65, 127, 128, 129]


def _ids_with_counts(counts, M, k):
    """Top-k ids [M][k] in which expert e appears counts[e] times, never twice
    in one token: the pairs of expert 0, then 1, ... are dealt column-major
    (pair j to token j % M), so a run of at most M pairs covers distinct
    tokens."""
    pairs = np.repeat(np.arange(len(counts)), counts)
    assert len(pairs) == M * k and max(counts) <= M
    ids = np.empty((M, k), dtype=np.int32)
    for j, e in enumerate(pairs):
        ids[j % M, j // M] = e
    return ids


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_moe_item_boundaries(dtype):
    """Experts whose row counts sit on both sides of every item boundary, so
    the route kernel emits GEMV items, whole 64-row items and partial items
    of each class, in one layer."""
    M, k, H, I = 130, 6, 128, 128
    E = len(_ROW_COUNTS)
    assert sum(_ROW_COUNTS) == M * k
    cfg = 650
    ids = _ids_with_counts(_ROW_COUNTS, M, k)
    assert (np.bincount(ids.ravel(), minlength=E) == np.array(_ROW_COUNTS)).all()
    assert all(len(set(r)) == k for r in ids.tolist())
    (gq, gs), (uq, us), (dq, ds) = _experts(E, H, I, cfg)
    g, u, d = weight_from_codes(gq, gs), weight_from_codes(uq, us), weight_from_codes(dq, ds)
    wts = W.gate_weights(M, k, cfg)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    y = _moe_gpu(x, to_dev(ids), to_dev(wts), g, u, d)
    ref, bound = _moe_ref(x, ids, wts, lambda e: ((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])), E, dtype)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, bound, f"moe item boundaries {dtype}")
    print(f"moe item boundaries {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,E,k,H,I", [(5, 8, 3, 128, 64), (24, 16, 8, 128, 128), (200, 4, 2, 128, 256)])
def test_moe_random_codes_include_nibble_zero(M, E, k, H, I, dtype):
    """Code words with every bit uniform (q = -8 included) on the GEMV items,
    the 64-row tiles and both together."""
    cfg = 560 + M
    (gq, gs), (uq, us), (dq, ds) = _random_expert_codes(E, H, I, cfg)
    g, u, d = weight_from_codes(gq, gs), weight_from_codes(uq, us), weight_from_codes(dq, ds)
    ids = W.topk_uniform(M, E, k, cfg)
    wts = W.gate_weights(M, k, cfg)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    y = _moe_gpu(x, to_dev(ids), to_dev(wts), g, u, d)
    ref, bound = _moe_ref(x, ids, wts, lambda e: ((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])), E, dtype)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, bound, f"moe random codes M={M} {dtype}")
    print(f"moe random codes M={M} E={E} k={k} {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [5, 20])
def test_moe_repeated_ids_within_a_token(M, dtype):
    """A token that names one expert in two or three of its slots gets that
    expert's output once per slot.  At M = 5 the layer has no MFMA launch, yet
    an expert can collect up to 15 rows (more than the GEMV's item size); at
    M = 20 with float32 activations such experts take the tiles."""
    E, k, H, I = 4, 3, 128, 64
    cfg = 580 + M
    (gq, gs), (uq, us), (dq, ds) = _experts(E, H, I, cfg)
    g, u, d = weight_from_codes(gq, gs), weight_from_codes(uq, us), weight_from_codes(dq, ds)
    rng = np.random.default_rng(cfg)
    ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
    ids[:, 0] = ids[:, 1] = 2  # expert 2 twice in every token
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.max() > 2 * M - 1
    wts = W.gate_weights(M, k, cfg)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    y = _moe_gpu(x, to_dev(ids), to_dev(wts), g, u, d)
    ref, bound = _moe_ref(x, ids, wts, lambda e: ((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])), E, dtype)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, bound, f"moe repeated ids M={M} {dtype}")
    print(f"moe repeated ids M={M} {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
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
    ref, bound = _moe_ref(x, ids, wts, lambda e: ((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])), E, "bf16")
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, bound, f"moe all-heavy M={M}")
    print(f"moe all-heavy M={M} E={E} k={k} H={H} I={I} bf16 relF={err:.3e} worst/bound={worst:.2e}", flush=True)
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


def _random_code_stacks(cfg, E, H, I):
    """Expert stacks of random code words and scales drawn on the GPU
    (workloads.code_words / scale_values), kept in both layouts: the GROUPED
    copy for the library, the canonical one for the oracle's expert slices."""
    canon, grouped = {}, {}
    for tag, (K, N) in ((W.TAG_GATE, (H, I)), (W.TAG_UP, (H, I)), (W.TAG_DOWN, (I, H))):
        qw = torch.empty((E, K // 8, N), dtype=torch.int32, device="cuda")
        sc = torch.empty((E, K // 32, N), dtype=torch.float32, device="cuda")
        for e in range(E):
            qw[e] = W.code_words(K, N, cfg.index, tag, e, device="cuda")
            sc[e] = W.scale_values(K // 32, N, cfg.index, tag, e, device="cuda")
        canon[tag] = (qw, sc)
        grouped[tag] = L.prepack(L.Weight(qw, sc, K, N, E, L.LAYOUT_CANONICAL), torch.empty_like(qw))
    torch.cuda.synchronize()
    tags = (W.TAG_GATE, W.TAG_UP, W.TAG_DOWN)

    def expert(e):
        return tuple((canon[t][0][e].cpu().numpy(), canon[t][1][e].cpu().numpy()) for t in tags)

    return [grouped[t] for t in tags], expert


def _full_moe_every_token(name):
    """Every token of a full-size MoE layer (384 experts of 7168 -> 2048,
    top-8, bf16) against the oracle, with random code words (q = -8 included)
    and the element-wise bound; the oracle's experts run in worker processes.
    A second call must reproduce the output bit for bit."""
    cfg = W.CONFIGS[name]
    E, H, I, M, k = cfg.experts, cfg.K, cfg.N, cfg.M, cfg.top_k
    if cfg.routing == "zipf":
        ids = W.topk_zipf(M, E, k, cfg.zipf_alpha, cfg.index)
    else:
        ids = W.topk_uniform(M, E, k, cfg.index)
    wts = W.gate_weights(M, k, cfg.index)
    stacks, expert = _random_code_stacks(cfg, E, H, I)
    x = x_for_dtype(W.activations(M, H, cfg.index).cuda(), cfg.x_dtype)
    y = _moe_gpu(x, to_dev(ids), to_dev(wts), *stacks)
    # deterministic: a second call (fresh workspace) gives the same bits
    assert torch.equal(y, _moe_gpu(x, to_dev(ids), to_dev(wts), *stacks))
    counts = np.bincount(ids.ravel(), minlength=E)
    print(f"{name}: {int((counts > 0).sum())} experts active, rows per expert {counts.min()}..{counts.max()}",
          flush=True)
    ref, bound = _moe_ref(x, ids, wts, expert, E, cfg.x_dtype, workers=16)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, bound, name)
    print(f"{name} random codes relF={err:.3e} worst/bound={worst:.2e} on all {M} tokens "
          f"({int((counts > 0).sum())} experts)", flush=True)
    assert err <= tol_for(cfg.x_dtype)
    return counts


def test_moe_decode_full_size_every_token():
    _full_moe_every_token("moe_decode_m64")


def test_moe_prefill_full_size_every_token():
    """Zipf(1.1) routing: every item kind at full size, among them the hot
    expert's tiles, experts of exactly 16 and 17 rows (the bf16 GEMV/tile
    boundary), experts of 65-127 rows (a ragged second tile) and expert 383."""
    cfg = W.CONFIGS["moe_prefill_m2048"]
    ids = W.topk_zipf(cfg.M, cfg.experts, cfg.top_k, cfg.zipf_alpha, cfg.index)
    counts = np.bincount(ids.ravel(), minlength=cfg.experts)
    assert (counts == 16).any() and (counts == 17).any() and ((counts > 64) & (counts < 128)).any()
    assert counts[cfg.experts - 1] > 0
    _full_moe_every_token("moe_prefill_m2048")
