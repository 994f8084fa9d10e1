"""GPU test of w4a16_swiglu_mlp_static, the allocation-free variant of
w4a16_swiglu_mlp: called through the C ABI twice in a row (the second call
smaller, on another path), each output bitwise equal to w4a16_swiglu_mlp's
on a fresh workspace of its own, and within the oracle's bound."""
import ctypes

import numpy as np
import pytest
import torch

import int4_w4a16_group_g32_amd as L
import oracle as O
import workloads as W
from helpers import rel_err, tol_for, weight_from_codes, x_for_dtype, x_values

pytestmark = pytest.mark.gpu


def _static_call(x, g, u, d, y):
    lib = L.load_library()
    xt = L.F32 if x.dtype == torch.float32 else L.BF16
    return lib.w4a16_swiglu_mlp_static(L._ptr(x), xt, x.shape[0], ctypes.byref(g.desc()), ctypes.byref(u.desc()),
                                       ctypes.byref(d.desc()), L._ptr(y),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _plain(x, g, u, d):
    xt = L.F32 if x.dtype == torch.float32 else L.BF16
    ws = L.new_workspace(L.swiglu_mlp_workspace_bytes(x.shape[0], xt, g, u, d))
    y = torch.full((x.shape[0], g.K), float("nan"), dtype=torch.float32, device="cuda")
    L.swiglu_mlp(x, g, u, d, y, ws)
    torch.cuda.synchronize()
    return y


@pytest.fixture(scope="module")
def dense():
    """The dense MLP shape (hidden 7168, intermediate 18432), quantized on the GPU."""
    H, I, cfg = 7168, 18432, 960
    return [L.quantize_to_weight(W.weights(K, N, cfg, tag, device="cuda"))
            for K, N, tag in ((H, I, W.TAG_GATE), (H, I, W.TAG_UP), (I, H, W.TAG_DOWN))]


def test_static_scratch_two_calls_in_a_row_match_the_workspace_entry_point(dense):
    g, u, d = dense
    # 64 rows with float32 activations (tiles, the largest plan: 48.6 MiB),
    # then 4 rows with bf16 (GEMV) and 3 with float32, on the same scratch
    for M, dtype in ((64, "f32"), (4, "bf16"), (3, "f32")):
        x = x_for_dtype(W.activations(M, g.K, 961 + M).cuda(), dtype)
        y = torch.full((M, g.K), float("nan"), dtype=torch.float32, device="cuda")
        assert _static_call(x, g, u, d, y) == L.OK
        torch.cuda.synchronize()
        y_ref = _plain(x, g, u, d)
        assert torch.isfinite(y).all()
        assert torch.equal(y, y_ref), f"M={M} {dtype}"
        print(f"static scratch M={M} {dtype}: bitwise equal to w4a16_swiglu_mlp", flush=True)


def test_static_scratch_against_the_oracle():
    H, I, M, cfg = 256, 512, 5, 962
    codes = [O.quantize_w4a16(W.weights(K, N, cfg, tag).numpy())
             for K, N, tag in ((H, I, W.TAG_GATE), (H, I, W.TAG_UP), (I, H, W.TAG_DOWN))]
    g, u, d = (weight_from_codes(*c) for c in codes)
    for dtype in ("f32", "bf16"):
        x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
        y = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
        assert _static_call(x, g, u, d, y) == L.OK
        torch.cuda.synchronize()
        err = rel_err(y, O.swiglu_mlp64(x_values(x), *codes))
        print(f"static scratch vs oracle {dtype} relF={err:.3e}", flush=True)
        assert err <= tol_for(dtype)


def test_static_scratch_rejects_a_call_beyond_its_size(dense):
    g, u, d = dense
    M = 512  # needs more than 64 MiB of workspace at this shape
    assert L.swiglu_mlp_workspace_bytes(M, L.F32, g, u, d) > 64 << 20
    x = torch.zeros((M, g.K), dtype=torch.float32, device="cuda")
    y = torch.zeros((M, g.K), dtype=torch.float32, device="cuda")
    assert _static_call(x, g, u, d, y) == L.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (y == 0).all()  # nothing was enqueued
