"""Python binding of libw4a16.so, the MI355X (gfx950) W4A16 group-32 library.

Argument marshalling only: every computation runs in the HIP kernels behind
the C ABI declared in include/w4a16.h.  PyTorch supplies device memory and
streams.  There is no fallback: if the library is not built, importing a
compute function raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libw4a16.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
F32, BF16 = 0, 1
LAYOUT_CANONICAL, LAYOUT_GROUPED = 0, 1
GROUP = 32

# every symbol include/w4a16.h declares
EXPORTS = (
    "w4a16_status_string",
    "w4a16_workspace_init",
    "w4a16_quantize",
    "w4a16_quantize_group",
    "w4a16_prepacked_bytes",
    "w4a16_prepack",
    "w4a16_dequantize",
    "w4a16_gemm_workspace_bytes",
    "w4a16_gemm",
    "w4a16_gemm_timed",
    "w4a16_swiglu_mlp_workspace_bytes",
    "w4a16_swiglu_mlp",
    "w4a16_swiglu_mlp_timed",
    "w4a16_swiglu_mlp_static",
    "w4a16_moe_topk",
    "w4a16_moe_route",
    "w4a16_moe_workspace_bytes",
    "w4a16_moe_grouped",
    "w4a16_moe_shared_workspace_bytes",
    "w4a16_moe_grouped_shared",
    "w4a16_moe_grouped_timed",
)


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class WeightDesc(ctypes.Structure):
    _fields_ = [
        ("qw", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("K", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("layout", ctypes.c_int32),
    ]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libw4a16.so (built in-tree by int4_w4a16_group_g32_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m int4_w4a16_group_g32_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        dp = ctypes.POINTER(WeightDesc)
        sig = {
            "w4a16_status_string": (ctypes.c_char_p, [i32]),
            "w4a16_workspace_init": (i32, [vp, sz, vp]),
            "w4a16_quantize": (i32, [vp, i32, i32, i32, vp, sz, vp, sz, vp]),
            "w4a16_quantize_group": (i32, [vp, i32, i32, i32, i32, vp, sz, vp, sz, vp]),
            "w4a16_prepacked_bytes": (sz, [dp]),
            "w4a16_prepack": (i32, [dp, vp, sz, dp, vp]),
            "w4a16_dequantize": (i32, [dp, vp, sz, vp]),
            "w4a16_gemm_workspace_bytes": (sz, [i32, dp, i32]),
            "w4a16_gemm": (i32, [vp, i32, i32, dp, vp, vp, sz, vp]),
            "w4a16_gemm_timed": (i32, [vp, i32, i32, dp, vp, vp, sz, vp, vp, i32, ctypes.POINTER(i32)]),
            "w4a16_swiglu_mlp_workspace_bytes": (sz, [i32, i32, dp, dp, dp]),
            "w4a16_swiglu_mlp": (i32, [vp, i32, i32, dp, dp, dp, vp, vp, sz, vp]),
            "w4a16_swiglu_mlp_timed": (i32, [vp, i32, i32, dp, dp, dp, vp, vp, sz, vp, vp, i32,
                                             ctypes.POINTER(i32)]),
            "w4a16_swiglu_mlp_static": (i32, [vp, i32, i32, dp, dp, dp, vp, vp]),
            "w4a16_moe_topk": (i32, [vp, i32, i32, i32, vp, vp, vp]),
            "w4a16_moe_route": (i32, [vp, i32, i32, i32, vp, vp, vp, vp, vp]),
            "w4a16_moe_workspace_bytes": (sz, [i32, i32, i32, dp, dp, dp]),
            "w4a16_moe_grouped": (i32, [vp, i32, i32, vp, vp, i32, dp, dp, dp, vp, vp, sz, vp]),
            "w4a16_moe_shared_workspace_bytes": (sz, [i32, i32, i32, dp, dp, dp, dp, dp, dp]),
            "w4a16_moe_grouped_shared": (i32, [vp, i32, i32, vp, vp, i32, dp, dp, dp, dp, dp, dp, vp, vp, sz,
                                               vp]),
            "w4a16_moe_grouped_timed": (i32, [vp, i32, i32, vp, vp, i32, dp, dp, dp, vp, vp, sz, vp, vp,
                                              i32, ctypes.POINTER(i32)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().w4a16_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != OK:
        raise W4A16Error(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return F32
    if x.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {x.dtype}")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    """Check a tensor handed to the library: dtype, contiguity and shape."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _on_device(**tensors):
    """Every tensor the library reads or writes must be device memory."""
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor, got {t.device}")


def _need_x(x: torch.Tensor, K: int):
    _dtype_code(x)
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"activations must be [M][{K}], got {tuple(x.shape)}")
    _need(x, "x", x.dtype)


@dataclass
class Weight:
    """A W4A16 weight (or expert stack): codes, scales and their shape."""
    qw: torch.Tensor          # int32, CANONICAL [E][K/8][N] or GROUPED [E][K/32][N][4]
    scales: torch.Tensor      # float32 [E][K/group_size][N]
    K: int
    N: int
    num_experts: int = 1
    layout: int = LAYOUT_GROUPED
    group_size: int = GROUP   # rows per scale: 32, 64 or 128

    def desc(self) -> WeightDesc:
        return WeightDesc(self.qw.data_ptr(), self.scales.data_ptr(), self.K, self.N, self.group_size,
                          self.num_experts, self.layout)


def _dref(w):
    return None if w is None else ctypes.byref(w.desc() if isinstance(w, Weight) else w)


# ---------------------------------------------------------------- format

def workspace_init(ws: torch.Tensor, stream=None):
    _check(load_library().w4a16_workspace_init(_ptr(ws), ws.numel() * ws.element_size(),
                                                _stream(stream)), "w4a16_workspace_init")


def quantize(w: torch.Tensor, qw: torch.Tensor, scales: torch.Tensor, stream=None, group_size: int = GROUP):
    """w float32 [E][K][N] (or [K][N]) -> CANONICAL qw, scales [E][K/group_size][N] (caller-allocated)."""
    _need(w, "w", torch.float32)
    _need(qw, "qw", torch.int32)
    _need(scales, "scales", torch.float32)
    _on_device(w=w, qw=qw, scales=scales)
    E = 1 if w.dim() == 2 else w.shape[0]
    K, N = w.shape[-2], w.shape[-1]
    if group_size == GROUP:
        st = load_library().w4a16_quantize(_ptr(w), K, N, E, _ptr(qw), _nbytes(qw), _ptr(scales), _nbytes(scales),
                                           _stream(stream))
    else:
        st = load_library().w4a16_quantize_group(_ptr(w), K, N, E, group_size, _ptr(qw), _nbytes(qw),
                                                 _ptr(scales), _nbytes(scales), _stream(stream))
    _check(st, "w4a16_quantize")


def prepacked_bytes(src: Weight) -> int:
    """Bytes of GROUPED codes w4a16_prepack writes for `src` (0 for an unsupported descriptor)."""
    return load_library().w4a16_prepacked_bytes(_dref(src))


def prepack(src: Weight, dst_qw: torch.Tensor, stream=None) -> Weight:
    _need(dst_qw, "dst_qw", torch.int32)
    _on_device(dst_qw=dst_qw, qw=src.qw, scales=src.scales)
    out = WeightDesc()
    _check(load_library().w4a16_prepack(_dref(src), _ptr(dst_qw), _nbytes(dst_qw), ctypes.byref(out),
                                        _stream(stream)), "w4a16_prepack")
    return Weight(dst_qw, src.scales, out.K, out.N, out.num_experts, out.layout, out.group_size)


def dequantize(w: Weight, out: torch.Tensor, stream=None):
    _need(out, "out", torch.float32)
    _on_device(out=out, qw=w.qw, scales=w.scales)
    _check(load_library().w4a16_dequantize(_dref(w), _ptr(out), _nbytes(out), _stream(stream)), "w4a16_dequantize")


# ---------------------------------------------------------------- compute

def gemm_workspace_bytes(M: int, w: Weight, xt: int) -> int:
    return load_library().w4a16_gemm_workspace_bytes(M, _dref(w), xt)


def gemm(x: torch.Tensor, w: Weight, y: torch.Tensor, ws: torch.Tensor, stream=None):
    _need_x(x, w.K)
    _need(y, "y", torch.float32, (x.shape[0], w.N))
    _need(ws, "ws", torch.uint8)
    _on_device(x=x, y=y, ws=ws)
    _check(load_library().w4a16_gemm(_ptr(x), _dtype_code(x), x.shape[0], _dref(w), _ptr(y), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)), "w4a16_gemm")


def swiglu_mlp_workspace_bytes(M: int, xt: int, gate: Weight, up: Weight, down: Weight) -> int:
    return load_library().w4a16_swiglu_mlp_workspace_bytes(M, xt, _dref(gate), _dref(up), _dref(down))


def swiglu_mlp(x: torch.Tensor, gate: Weight, up: Weight, down: Weight, y: torch.Tensor,
               ws: torch.Tensor, stream=None):
    _need_x(x, gate.K)
    _need(y, "y", torch.float32, (x.shape[0], down.N))
    _need(ws, "ws", torch.uint8)
    _on_device(x=x, y=y, ws=ws)
    _check(load_library().w4a16_swiglu_mlp(_ptr(x), _dtype_code(x), x.shape[0], _dref(gate), _dref(up),
                                           _dref(down), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                           _stream(stream)), "w4a16_swiglu_mlp")


def swiglu_mlp_static(x: torch.Tensor, gate: Weight, up: Weight, down: Weight, y: torch.Tensor, stream=None):
    """swiglu_mlp on the library's static per-GPU scratch (no workspace, no allocation)."""
    _need_x(x, gate.K)
    _need(y, "y", torch.float32, (x.shape[0], down.N))
    _on_device(x=x, y=y)
    _check(load_library().w4a16_swiglu_mlp_static(_ptr(x), _dtype_code(x), x.shape[0], _dref(gate), _dref(up),
                                                  _dref(down), _ptr(y), _stream(stream)), "w4a16_swiglu_mlp_static")


def moe_topk(logits: torch.Tensor, top_k: int, topk_ids: torch.Tensor, topk_w: torch.Tensor, stream=None):
    """Top-k experts per token row of float32 logits [M][E] and their softmax gate weights."""
    _need(logits, "logits", torch.float32)
    M, E = logits.shape
    _need(topk_ids, "topk_ids", torch.int32, (M, top_k))
    _need(topk_w, "topk_w", torch.float32, (M, top_k))
    _on_device(logits=logits, topk_ids=topk_ids, topk_w=topk_w)
    _check(load_library().w4a16_moe_topk(_ptr(logits), M, E, top_k, _ptr(topk_ids), _ptr(topk_w),
                                         _stream(stream)), "w4a16_moe_topk")


def moe_route(topk_ids: torch.Tensor, num_experts: int, counts, offsets, sorted_pairs, inv, stream=None):
    _need(topk_ids, "topk_ids", torch.int32)
    M, k = topk_ids.shape
    _need(counts, "counts", torch.int32, (num_experts,))
    _need(offsets, "offsets", torch.int32, (num_experts + 1,))
    for t, name in ((sorted_pairs, "sorted_pairs"), (inv, "inv")):
        _need(t, name, torch.int32)
        if t.numel() < M * k:
            raise ValueError(f"{name} must hold at least {M * k} entries")
    _on_device(topk_ids=topk_ids, counts=counts, offsets=offsets, sorted_pairs=sorted_pairs, inv=inv)
    _check(load_library().w4a16_moe_route(_ptr(topk_ids), M, k, num_experts, _ptr(counts), _ptr(offsets),
                                          _ptr(sorted_pairs), _ptr(inv), _stream(stream)), "w4a16_moe_route")


def moe_workspace_bytes(M: int, top_k: int, xt: int, gate: Weight, up: Weight, down: Weight) -> int:
    return load_library().w4a16_moe_workspace_bytes(M, top_k, xt, _dref(gate), _dref(up), _dref(down))


def moe_shared_workspace_bytes(M: int, top_k: int, xt: int, gate: Weight, up: Weight, down: Weight,
                               shared_gate: Weight, shared_up: Weight, shared_down: Weight) -> int:
    return load_library().w4a16_moe_shared_workspace_bytes(M, top_k, xt, _dref(gate), _dref(up), _dref(down),
                                                           _dref(shared_gate), _dref(shared_up),
                                                           _dref(shared_down))


def _check_moe_args(x, topk_ids, topk_w, gate: Weight, down: Weight, y, ws):
    """topk_ids int32 [M][k] (torch.topk's int64 ids must be converted), topk_w
    float32 [M][k], x [M][H], y float32 [M][H]; returns (M, k)."""
    _need(topk_ids, "topk_ids", torch.int32)
    if topk_ids.dim() != 2:
        raise ValueError(f"topk_ids must be [M][top_k], got {tuple(topk_ids.shape)}")
    M, k = topk_ids.shape
    _need(topk_w, "topk_w", torch.float32, (M, k))
    _need_x(x, gate.K)
    if x.shape[0] != M:
        raise ValueError(f"x has {x.shape[0]} rows, topk_ids {M}")
    _need(y, "y", torch.float32, (M, down.N))
    _need(ws, "ws", torch.uint8)
    _on_device(x=x, topk_ids=topk_ids, topk_w=topk_w, y=y, ws=ws)
    return M, k


def moe_grouped_shared(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, gate: Weight, up: Weight,
                       down: Weight, shared_gate: Weight, shared_up: Weight, shared_down: Weight, y: torch.Tensor,
                       ws: torch.Tensor, stream=None):
    M, k = _check_moe_args(x, topk_ids, topk_w, gate, down, y, ws)
    _check(load_library().w4a16_moe_grouped_shared(_ptr(x), _dtype_code(x), M, _ptr(topk_ids), _ptr(topk_w), k,
                                                   _dref(gate), _dref(up), _dref(down), _dref(shared_gate),
                                                   _dref(shared_up), _dref(shared_down), _ptr(y), _ptr(ws),
                                                   ws.numel() * ws.element_size(), _stream(stream)),
           "w4a16_moe_grouped_shared")


def moe_grouped(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, gate: Weight, up: Weight,
                down: Weight, y: torch.Tensor, ws: torch.Tensor, stream=None):
    M, k = _check_moe_args(x, topk_ids, topk_w, gate, down, y, ws)
    _check(load_library().w4a16_moe_grouped(_ptr(x), _dtype_code(x), M, _ptr(topk_ids), _ptr(topk_w), k,
                                            _dref(gate), _dref(up), _dref(down), _ptr(y), _ptr(ws),
                                            ws.numel() * ws.element_size(), _stream(stream)),
           "w4a16_moe_grouped")


# ---------------------------------------------------------------- helpers

def new_workspace(nbytes: int, device="cuda", stream=None) -> torch.Tensor:
    """A zero-filled workspace of at least `nbytes` bytes (16-byte aligned by torch)."""
    ws = torch.empty(max(16, (int(nbytes) + 15) // 16 * 16), dtype=torch.uint8, device=device)
    workspace_init(ws, stream)
    return ws


def quantize_to_weight(w: torch.Tensor, stream=None) -> Weight:
    """Quantize float32 device weights [E][K][N] or [K][N] and prepack them (GROUPED)."""
    E = 1 if w.dim() == 2 else w.shape[0]
    K, N = w.shape[-2], w.shape[-1]
    qw = torch.empty((E, K // 8, N), dtype=torch.int32, device=w.device)
    sc = torch.empty((E, K // GROUP, N), dtype=torch.float32, device=w.device)
    quantize(w, qw, sc, stream)
    canon = Weight(qw, sc, K, N, E, LAYOUT_CANONICAL)
    dst = torch.empty_like(qw)
    return prepack(canon, dst, stream)
