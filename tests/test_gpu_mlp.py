"""GPU parity of w4a16_swiglu_mlp against the oracle's float64 SwiGLU MLP,
on small shapes (several tiles, ragged row counts) and on the full dense
shape (hidden 7168, intermediate 18432) at M = 4 (float32) and M = 64
(float32 and bf16), comparing sampled output columns."""
import numpy as np
import pytest
import torch

import int4_w4a16_group_g32_amd as L
import oracle as O
import workloads as W
from helpers import canonical_words, rel_err, tol_for, weight_from_codes, x_for_dtype, x_values
from oracle_pool import TAU, check_elementwise, mlp_bound

pytestmark = pytest.mark.gpu


def _mlp_gpu(x, g, u, d):
    xt = L.F32 if x.dtype == torch.float32 else L.BF16
    ws = L.new_workspace(L.swiglu_mlp_workspace_bytes(x.shape[0], xt, g, u, d))
    y = torch.full((x.shape[0], g.K), float("nan"), dtype=torch.float32, device="cuda")
    L.swiglu_mlp(x, g, u, d, y, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H,I", [(64, 128), (256, 512), (1024, 2048)])
@pytest.mark.parametrize("M", [1, 3, 4, 8, 9, 16, 64, 100])
def test_mlp_small(M, H, I, dtype):
    cfg = 400 + H
    ws_np = [W.weights(H, I, cfg, W.TAG_GATE).numpy(), W.weights(H, I, cfg, W.TAG_UP).numpy(),
             W.weights(I, H, cfg, W.TAG_DOWN).numpy()]
    codes = [O.quantize_w4a16(w) for w in ws_np]
    g, u, d = (weight_from_codes(*c) for c in codes)
    x = x_for_dtype(W.activations(M, H, cfg + M).cuda(), dtype)
    y = _mlp_gpu(x, g, u, d)
    ref = O.swiglu_mlp64(x_values(x), *codes)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, mlp_bound(x_values(x), *codes, TAU[dtype]),
                              f"mlp M={M} H={H} I={I} {dtype}")
    print(f"mlp M={M} H={H} I={I} {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [4, 16, 64])
def test_mlp_random_codes_include_nibble_zero(M, dtype):
    """Code words with every bit uniform, so q = -8 reaches the gate/up and
    down kernels of the GEMV (M = 4; 16 with bf16) and the tiles (M = 16
    with float32, 64)."""
    H, I, cfg = 1024, 2048, 610 + M
    rng = np.random.default_rng(cfg)
    codes = []
    for K, N in ((H, I), (H, I), (I, H)):
        qw = rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint64).astype(np.uint32).view(np.int32)
        codes.append((qw, (rng.random((K // 32, N)) * 0.005 + 0.004).astype(np.float32)))
    g, u, d = (weight_from_codes(*c) for c in codes)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    y = _mlp_gpu(x, g, u, d)
    ref = O.swiglu_mlp64(x_values(x), *codes)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, mlp_bound(x_values(x), *codes, TAU[dtype]),
                              f"mlp random codes M={M} {dtype}")
    print(f"mlp random codes M={M} {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)


@pytest.fixture(scope="module")
def dense_mlp():
    """The dense SwiGLU MLP (7168 -> 18432 -> 7168), weights drawn on the GPU,
    quantized by the library and, independently, by the oracle."""
    H, I, cfg = 7168, 18432, W.CONFIGS["mlp_decode_m4"].index
    gpu, ora = [], []
    for K, N, tag in ((H, I, W.TAG_GATE), (H, I, W.TAG_UP), (I, H, W.TAG_DOWN)):
        w = W.weights(K, N, cfg, tag, device="cuda")
        gpu.append(L.quantize_to_weight(w))
        w_np = w.cpu().numpy()
        del w
        if tag == W.TAG_DOWN:
            ora.append(w_np)  # quantized per sampled column below
        else:
            ora.append(O.quantize_w4a16(w_np))
    torch.cuda.synchronize()
    return H, I, gpu, ora


def _sampled_down(w_down, cols):
    return O.quantize_w4a16(np.ascontiguousarray(w_down[:, cols]))


@pytest.mark.parametrize("name,dtype", [("mlp_decode_m4", "f32"), ("mlp_verify_m64_f32", "f32"),
                                        ("mlp_verify_m64_bf16", "bf16")])
def test_mlp_full_size(dense_mlp, name, dtype):
    H, I, (g, u, d), (gq, uq, w_down) = dense_mlp
    cfg = W.CONFIGS[name]
    x = x_for_dtype(W.activations(cfg.M, H, cfg.index).cuda(), dtype)
    y = _mlp_gpu(x, g, u, d)
    assert torch.equal(y, _mlp_gpu(x, g, u, d))  # deterministic across calls
    cols = np.sort(np.random.default_rng(cfg.M).choice(H, size=512, replace=False))
    xv = x_values(x)
    dq = _sampled_down(w_down, cols)
    ref = O.swiglu_mlp64(xv, gq, uq, dq)
    ys = y[:, torch.as_tensor(cols, device="cuda")]
    err = rel_err(ys, ref)
    worst = check_elementwise(ys.cpu().numpy(), ref, mlp_bound(xv, gq, uq, dq, TAU[dtype]), name)
    print(f"{name} relF={err:.3e} worst/bound={worst:.2e} (512 sampled columns)", flush=True)
    assert err <= tol_for(dtype)
    assert torch.isfinite(y).all()
    # the library's quantization of the same weights agrees with the oracle's
    qd = canonical_words(d.qw.cpu().numpy(), I, H)[0][:, cols]
    assert np.array_equal(qd, _sampled_down(w_down, cols)[0])


@pytest.mark.parametrize("M,dtype,H,I,kernels", [(4, "f32", 256, 512, 2), (100, "bf16", 128, 128, 4),
                                                 (64, "bf16", 2048, 4096, 5), (40, "f32", 2048, 4096, 5)])
def test_mlp_timed_brackets_each_kernel(M, dtype, H, I, kernels):
    """w4a16_swiglu_mlp_timed does the same work as w4a16_swiglu_mlp (same
    output bits) and brackets each of its kernels with a start and a stop
    event.  From M = 9 (float32) or 17 (bf16): the activation pieces, the
    gate/up tiles, the pieces of h and the down tiles (hidden and
    intermediate 128: too few groups to split K); with K split across
    workgroups (hidden 2048, intermediate 4096) the pieces of h are formed
    from the gate/up split sums and a fifth kernel adds the down projection's
    splits."""
    import ctypes

    cfg = 470
    codes = [O.quantize_w4a16(w.numpy()) for w in (W.weights(H, I, cfg, W.TAG_GATE), W.weights(H, I, cfg, W.TAG_UP),
                                                   W.weights(I, H, cfg, W.TAG_DOWN))]
    g, u, d = (weight_from_codes(*c) for c in codes)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    y_plain = _mlp_gpu(x, g, u, d)
    xt = L.F32 if dtype == "f32" else L.BF16
    ws = L.new_workspace(L.swiglu_mlp_workspace_bytes(M, xt, g, u, d))
    y = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(10)]
    for e in evs:  # torch creates the HIP event on its first record
        e.record()
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * 10)(*[e.cuda_event for e in evs])
    rec = ctypes.c_int32(-1)
    lib = L.load_library()
    st = lib.w4a16_swiglu_mlp_timed(L._ptr(x), xt, M, ctypes.byref(g.desc()), ctypes.byref(u.desc()),
                                    ctypes.byref(d.desc()), L._ptr(y), L._ptr(ws), ws.numel(),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), handles, 10,
                                    ctypes.byref(rec))
    assert st == 0
    torch.cuda.synchronize()
    assert rec.value == 2 * kernels
    assert torch.equal(y, y_plain)
    ref = O.swiglu_mlp64(x_values(x), *codes)
    assert rel_err(y, ref) <= tol_for(dtype)
    for j in range(kernels):
        assert evs[2 * j].elapsed_time(evs[2 * j + 1]) > 0.0
        if j > 0:  # kernels run in launch order on the stream
            assert evs[2 * j - 1].elapsed_time(evs[2 * j]) >= 0.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mlp_gemv_four_tile_workgroups_ragged(dtype):
    """Hidden 32768, intermediate 1920 at M = 4: the fused gate/up GEMV has 15
    SwiGLU tiles of 128 outputs and 32 K splits (480 tasks), run as 256
    workgroups of two tiles, the last with one quad past the matrix.  Sampled
    output columns against the oracle."""
    H, I, M, cfg = 32768, 1920, 4, 530
    gate = W.weights(H, I, cfg, W.TAG_GATE)
    up = W.weights(H, I, cfg, W.TAG_UP)
    down = W.weights(I, H, cfg, W.TAG_DOWN)
    gq, uq = O.quantize_w4a16(gate.numpy()), O.quantize_w4a16(up.numpy())
    g, u = weight_from_codes(*gq), weight_from_codes(*uq)
    d = L.quantize_to_weight(down.cuda())
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    y = _mlp_gpu(x, g, u, d)
    cols = np.sort(np.random.default_rng(cfg).choice(H, size=512, replace=False))
    xv = x_values(x)
    h = O.silu64(O.gemm64(xv, *gq)) * O.gemm64(xv, *uq)
    ref = h @ O.dequant64(*_sampled_down(down.numpy(), cols))
    err = rel_err(y[:, torch.as_tensor(cols, device="cuda")], ref)
    print(f"mlp H={H} I={I} M={M} {dtype} relF={err:.3e} (512 sampled columns)", flush=True)
    assert err <= tol_for(dtype)


@pytest.mark.parametrize("M,dtype", [(64, "bf16"), (40, "f32")])
def test_mlp_split_pieces_zero_and_small_ranges(M, dtype):
    """Hidden 2048, intermediate 4096: both tile launches split K, so the
    pieces of h are made per down split from the gate/up split sums (the five
    kernels of test_mlp_timed_brackets_each_kernel).  Gate columns 0..1023 are
    zero, so h is zero there and the down splits over that range get zero
    pieces and a zero row factor; up columns 2048..3071 are scaled by 2^-20,
    so those splits' largest magnitudes sit far below the row's.  Element-wise
    bound and relF against the oracle."""
    H, I, cfg = 2048, 4096, 640 + M
    gate = W.weights(H, I, cfg, W.TAG_GATE).numpy()
    up = W.weights(H, I, cfg, W.TAG_UP).numpy()
    down = W.weights(I, H, cfg, W.TAG_DOWN).numpy()
    gate[:, :1024] = 0.0
    up[:, 2048:3072] *= np.float32(2.0 ** -20)
    codes = [O.quantize_w4a16(w) for w in (gate, up, down)]
    g, u, d = (weight_from_codes(*c) for c in codes)
    x = x_for_dtype(W.activations(M, H, cfg).cuda(), dtype)
    y = _mlp_gpu(x, g, u, d)
    ref = O.swiglu_mlp64(x_values(x), *codes)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, mlp_bound(x_values(x), *codes, TAU[dtype]),
                              f"mlp split pieces M={M} {dtype}")
    print(f"mlp split pieces M={M} {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)
    assert torch.isfinite(y).all()


@pytest.mark.parametrize("name,dtype", [("mlp_decode_m4_tp8", "f32"), ("mlp_verify_m64_bf16_tp8", "bf16"),
                                        ("mlp_verify_m64_bf16_tp8", "f32")])
def test_mlp_tp8_share_full_size(name, dtype):
    """One GPU's share of the dense MLP under 8-way tensor parallelism
    (hidden 7168, intermediate 2304: gate/up column-parallel, down
    row-parallel), every output element against the oracle; the library's
    quantization of the weights is checked word for word against the
    oracle's."""
    cfg = W.CONFIGS[name]
    H, I, M = cfg.K, cfg.N, cfg.M
    gpu, codes = [], []
    for K, N, tag in ((H, I, W.TAG_GATE), (H, I, W.TAG_UP), (I, H, W.TAG_DOWN)):
        w = W.weights(K, N, cfg.index, tag, device="cuda")
        gpu.append(L.quantize_to_weight(w))
        codes.append(O.quantize_w4a16(w.cpu().numpy()))
        del w
    for wt, (qw, sc), (K, N) in zip(gpu, codes, ((H, I), (H, I), (I, H))):
        assert np.array_equal(canonical_words(wt.qw.cpu().numpy(), K, N)[0], qw)
        assert np.array_equal(wt.scales.cpu().numpy().reshape(sc.shape), sc)
    x = x_for_dtype(W.activations(M, H, cfg.index).cuda(), dtype)
    y = _mlp_gpu(x, *gpu)
    xv = x_values(x)
    ref = O.swiglu_mlp64(xv, *codes)
    err = rel_err(y, ref)
    worst = check_elementwise(y.cpu().numpy(), ref, mlp_bound(xv, *codes, TAU[dtype]), f"{name} {dtype}")
    print(f"{name} {dtype} relF={err:.3e} worst/bound={worst:.2e}", flush=True)
    assert err <= tol_for(dtype)
