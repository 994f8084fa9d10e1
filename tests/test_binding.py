"""CPU checks of the Python binding's argument validation: every wrong dtype,
shape, layout or device is rejected in Python, before the library is called
(the tensors here are host tensors, so a call that got through would fail
differently)."""
import pytest
import torch

import int4_w4a16_group_g32_amd as L


def _w(K, N, E=1):
    return L.Weight(torch.zeros((E, K // 8, N), dtype=torch.int32), torch.zeros((E, K // 32, N)), K, N, E)


def test_gemm_rejects_bad_tensors():
    w = _w(64, 128)
    ws = torch.zeros(256, dtype=torch.uint8)
    with pytest.raises(TypeError):  # float16 activations
        L.gemm(torch.zeros((2, 64), dtype=torch.float16), w, torch.zeros((2, 128)), ws)
    with pytest.raises(ValueError):  # x is [M][K] with the wrong K
        L.gemm(torch.zeros((2, 32)), w, torch.zeros((2, 128)), ws)
    with pytest.raises(ValueError):  # y of the wrong shape
        L.gemm(torch.zeros((2, 64)), w, torch.zeros((2, 64)), ws)
    with pytest.raises(TypeError):  # y not float32
        L.gemm(torch.zeros((2, 64)), w, torch.zeros((2, 128), dtype=torch.float64), ws)
    with pytest.raises(ValueError):  # non-contiguous x
        L.gemm(torch.zeros((64, 2)).t(), w, torch.zeros((2, 128)), ws)
    with pytest.raises(ValueError):  # host tensors are not device memory
        L.gemm(torch.zeros((2, 64)), w, torch.zeros((2, 128)), ws)


def test_swiglu_mlp_rejects_bad_tensors():
    g, u, d = _w(64, 128), _w(64, 128), _w(128, 64)
    ws = torch.zeros(256, dtype=torch.uint8)
    with pytest.raises(ValueError):
        L.swiglu_mlp(torch.zeros((3, 128)), g, u, d, torch.zeros((3, 64)), ws)
    with pytest.raises(ValueError):
        L.swiglu_mlp(torch.zeros((3, 64)), g, u, d, torch.zeros((3, 128)), ws)
    with pytest.raises(TypeError):
        L.swiglu_mlp(torch.zeros((3, 64)), g, u, d, torch.zeros((3, 64)), torch.zeros(64))


def test_moe_rejects_int64_ids_and_bad_shapes():
    g, u, d = _w(64, 128, 4), _w(64, 128, 4), _w(128, 64, 4)
    ws = torch.zeros(256, dtype=torch.uint8)
    x = torch.zeros((5, 64))
    y = torch.zeros((5, 64))
    ids64 = torch.zeros((5, 2), dtype=torch.int64)  # what torch.topk returns
    wts = torch.zeros((5, 2))
    with pytest.raises(TypeError):
        L.moe_grouped(x, ids64, wts, g, u, d, y, ws)
    ids = ids64.to(torch.int32)
    with pytest.raises(ValueError):  # gate weights of another shape
        L.moe_grouped(x, ids, torch.zeros((5, 3)), g, u, d, y, ws)
    with pytest.raises(ValueError):  # x rows != token rows
        L.moe_grouped(torch.zeros((4, 64)), ids, wts, g, u, d, torch.zeros((4, 64)), ws)
    with pytest.raises(ValueError):  # y of the wrong width
        L.moe_grouped(x, ids, wts, g, u, d, torch.zeros((5, 128)), ws)
    with pytest.raises(TypeError):
        L.moe_grouped_shared(x, ids64, wts, g, u, d, _w(64, 128), _w(64, 128), _w(128, 64), y, ws)
    with pytest.raises(TypeError):
        L.moe_topk(torch.zeros((5, 4)), 2, ids64, wts)
    with pytest.raises(TypeError):
        L.moe_route(ids64, 4, torch.zeros(4, dtype=torch.int32), torch.zeros(5, dtype=torch.int32),
                    torch.zeros(10, dtype=torch.int32), torch.zeros(10, dtype=torch.int32))


def test_format_calls_reject_bad_buffers():
    with pytest.raises(TypeError):
        L.quantize(torch.zeros((64, 64), dtype=torch.float64), torch.zeros((8, 64), dtype=torch.int32),
                   torch.zeros((2, 64)))
    canon = L.Weight(torch.zeros((1, 8, 64), dtype=torch.int32), torch.zeros((1, 2, 64)), 64, 64, 1,
                     L.LAYOUT_CANONICAL)
    with pytest.raises(TypeError):
        L.prepack(canon, torch.zeros((1, 8, 64), dtype=torch.int64))
    with pytest.raises(TypeError):
        L.dequantize(canon, torch.zeros((64, 64), dtype=torch.float64))
