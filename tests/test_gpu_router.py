"""GPU parity of w4a16_moe_topk against the oracle's router (moe_topk).

Expert ids are compared bit for bit: both sides compare the same float32
logits.  Gate weights are a float32 softmax on the GPU against the float64
oracle: relative Frobenius error <= 1e-6 (a few float32 roundings of exp, sum
and divide)."""
import numpy as np
import pytest
import torch

import int4_w4a16_group_g32_amd as L
import oracle as O

pytestmark = pytest.mark.gpu


def _run(logits, k):
    M, E = logits.shape
    ids = torch.full((M, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((M, k), float("nan"), dtype=torch.float32, device="cuda")
    L.moe_topk(logits, k, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("M,E,k", [(64, 384, 8), (2048, 384, 8), (5, 6, 2), (7, 1024, 32), (3, 65, 1),
                                   (1, 1, 1), (33, 130, 7)])
def test_topk_matches_oracle(M, E, k):
    g = torch.Generator().manual_seed(M * 1000 + E + k)
    logits = torch.randn((M, E), generator=g, dtype=torch.float32)
    ids, w = _run(logits.cuda(), k)
    ref_ids, ref_w = O.moe_topk(logits.numpy(), k)
    assert np.array_equal(ids, ref_ids)
    err = O.rel_frobenius(w, ref_w)
    print(f"topk M={M} E={E} k={k} weights relF={err:.3e}", flush=True)
    assert err <= 1e-6


def test_topk_ties_take_the_lower_expert_index():
    g = torch.Generator().manual_seed(5)
    logits = torch.randint(-3, 4, (200, 384), generator=g).to(torch.float32)
    ids, w = _run(logits.cuda(), 8)
    ref_ids, ref_w = O.moe_topk(logits.numpy(), 8)
    assert np.array_equal(ids, ref_ids)
    assert O.rel_frobenius(w, ref_w) <= 1e-6


def test_topk_extreme_logits_and_determinism():
    g = torch.Generator().manual_seed(6)
    logits = torch.randn((128, 384), generator=g, dtype=torch.float32) * 1000.0
    logits[0] = -3.0e38          # every logit at the bottom of the float32 range
    logits[1, :] = 0.0
    logits[1, 17] = 3.0e38
    a = _run(logits.cuda(), 8)
    b = _run(logits.cuda(), 8)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    ref_ids, ref_w = O.moe_topk(logits.numpy().astype(np.float64), 8)
    assert np.array_equal(a[0], ref_ids)
    assert O.rel_frobenius(a[1], ref_w) <= 1e-6
    np.testing.assert_allclose(a[1].sum(axis=1), 1.0, rtol=1e-6)


def test_topk_feeds_route_and_moe_contract():
    """The router's output is a valid routing: distinct ids per token, so
    w4a16_moe_route groups every pair exactly once."""
    g = torch.Generator().manual_seed(9)
    M, E, k = 257, 384, 8
    logits = torch.randn((M, E), generator=g, dtype=torch.float32).cuda()
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, k), dtype=torch.float32, device="cuda")
    L.moe_topk(logits, k, ids, w)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(M * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(M * k, dtype=torch.int32, device="cuda")
    L.moe_route(ids, E, counts, offsets, sp, inv)
    torch.cuda.synchronize()
    ids_np = ids.cpu().numpy()
    assert all(len(set(r)) == k for r in ids_np.tolist())
    rc, ro, rs, ri = O.route(ids_np, E)
    assert np.array_equal(counts.cpu().numpy(), rc) and np.array_equal(sp.cpu().numpy(), rs)
