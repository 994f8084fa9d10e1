"""Empty inputs (M = 0) on every entry point that takes rows: the call returns
OK and enqueues no work, and the workspace it was given still serves a later
non-empty call with the same bits as a fresh one.  The route of zero tokens
leaves every expert count and offset at zero."""
import numpy as np
import pytest
import torch

import int4_w4a16_group_g32_amd as L

pytestmark = pytest.mark.gpu

H, I, E, K_TOP = 128, 64, 6, 2


def _weights(seed, E_=E):
    g = torch.Generator(device="cpu").manual_seed(seed)

    def q(k, n):
        return L.quantize_to_weight((0.02 * torch.randn((E_, k, n), generator=g)).cuda())

    return q(H, I), q(H, I), q(I, H)


def _routing(M, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, K_TOP, replace=False) for _ in range(M)]).astype(np.int32).reshape(M, K_TOP)
    w = rng.random((M, K_TOP)).astype(np.float32)
    return torch.from_numpy(ids).cuda(), torch.from_numpy(w / w.sum(1, keepdims=True)).cuda()


def _x(M, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn((M, H), generator=g).to(dtype).cuda()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_mlp_m0_then_rows(dtype):
    gate, up, down = (w for w in _weights(11, 1))
    xt = L.F32 if dtype == torch.float32 else L.BF16
    ws = L.new_workspace(L.swiglu_mlp_workspace_bytes(5, xt, gate, up, down))
    L.swiglu_mlp(torch.empty((0, H), dtype=dtype, device="cuda"), gate, up, down,
                 torch.empty((0, H), device="cuda"), ws)
    x = _x(5, dtype, 12)
    y = torch.full((5, H), float("nan"), device="cuda")
    L.swiglu_mlp(x, gate, up, down, y, ws)
    ref = torch.full((5, H), float("nan"), device="cuda")
    L.swiglu_mlp(x, gate, up, down, ref, L.new_workspace(L.swiglu_mlp_workspace_bytes(5, xt, gate, up, down)))
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.equal(y, ref)


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_moe_m0_then_rows(dtype, shared):
    routed = _weights(21)
    sh = _weights(22, 1) if shared else ()
    xt = L.F32 if dtype == torch.float32 else L.BF16
    M = 7

    def ws_bytes(m):
        if shared:
            return L.moe_shared_workspace_bytes(m, K_TOP, xt, *routed, *sh)
        return L.moe_workspace_bytes(m, K_TOP, xt, *routed)

    def run(x, ids, w, y, ws):
        if shared:
            L.moe_grouped_shared(x, ids, w, *routed, *sh, y, ws)
        else:
            L.moe_grouped(x, ids, w, *routed, y, ws)

    assert ws_bytes(0) == 0
    ws = L.new_workspace(ws_bytes(M))
    run(torch.empty((0, H), dtype=dtype, device="cuda"), torch.empty((0, K_TOP), dtype=torch.int32, device="cuda"),
        torch.empty((0, K_TOP), device="cuda"), torch.empty((0, H), device="cuda"), ws)
    x = _x(M, dtype, 23)
    ids, w = _routing(M, 24)
    y = torch.full((M, H), float("nan"), device="cuda")
    run(x, ids, w, y, ws)
    ref = torch.full((M, H), float("nan"), device="cuda")
    run(x, ids, w, ref, L.new_workspace(ws_bytes(M)))
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.equal(y, ref)


def test_route_and_topk_of_zero_tokens():
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    empty_i = torch.empty((0,), dtype=torch.int32, device="cuda")
    L.moe_route(torch.empty((0, K_TOP), dtype=torch.int32, device="cuda"), E, counts, offsets, empty_i, empty_i)
    ids = torch.empty((0, K_TOP), dtype=torch.int32, device="cuda")
    w = torch.empty((0, K_TOP), device="cuda")
    L.moe_topk(torch.empty((0, E), device="cuda"), K_TOP, ids, w)
    torch.cuda.synchronize()
    assert (counts == 0).all() and (offsets == 0).all()
