"""Shared helpers for the tests (no test functions here).

GPU-side objects are built through the library's own entry points; the oracle
side always recomputes from the same float32 inputs with oracle/ only.
"""
from __future__ import annotations

import numpy as np
import torch

import int4_w4a16_group_g32_amd as L
import oracle as O

TOL = {"f32": 1e-5, "bf16": 1e-2}  # relative Frobenius bounds on outputs


def tol_for(dtype: str) -> float:
    return TOL[dtype]


def to_dev(a, dtype=None):
    t = torch.as_tensor(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def weight_from_codes(qw_np: np.ndarray, sc_np: np.ndarray) -> L.Weight:
    """Upload oracle-made CANONICAL codes [E][K/8][N] (or [K/8][N]) and prepack on the GPU."""
    qw_np = np.asarray(qw_np, dtype=np.int32)
    sc_np = np.asarray(sc_np, dtype=np.float32)
    if qw_np.ndim == 2:
        qw_np, sc_np = qw_np[None], sc_np[None]
    E, Kw, N = qw_np.shape
    group = Kw * 8 // sc_np.shape[1]  # rows per scale, from the scales' shape
    canon = L.Weight(to_dev(qw_np), to_dev(sc_np), Kw * 8, N, E, L.LAYOUT_CANONICAL, group)
    return L.prepack(canon, torch.empty_like(canon.qw))


def oracle_quantize_stack(ws, group=32):
    """Oracle-quantize a list of float32 [K][N] matrices into stacked codes and scales."""
    qs, ss = zip(*(O.quantize_w4a16(w, group) for w in ws))
    return np.stack(qs), np.stack(ss)


def x_for_dtype(x_f32: torch.Tensor, dtype: str) -> torch.Tensor:
    return x_f32.to(torch.bfloat16) if dtype == "bf16" else x_f32


def x_values(x: torch.Tensor) -> np.ndarray:
    """The exact values the GPU sees, as float32 numpy (bf16 widened exactly)."""
    return x.detach().float().cpu().numpy()


def rel_err(y_gpu: torch.Tensor, y_ref: np.ndarray) -> float:
    return O.rel_frobenius(y_gpu.detach().cpu().numpy().astype(np.float64), y_ref)


def grouped_words(qw_canon: np.ndarray) -> np.ndarray:
    """The GROUPED layout of canonical codes qw[E][K/8][N], as the header
    describes it: for group g and 64-column block j, 16-byte slot 16b + l holds
    canonical word 4g + b of columns 64j + 4l .. 64j + 4l + 3.  Returns
    [E][K/32][N/64][64][4] int32."""
    E, W, N = qw_canon.shape
    G = W // 4
    v = qw_canon.reshape(E, G, 4, N // 64, 16, 4)          # e, g, b, j, l, c
    return np.ascontiguousarray(v.transpose(0, 1, 3, 2, 4, 5)).reshape(E, G, N // 64, 64, 4)


def canonical_words(qw_grouped: np.ndarray, K: int, N: int) -> np.ndarray:
    """Inverse of grouped_words: canonical qw[E][K/8][N] from GROUPED words."""
    E = qw_grouped.size // (K * N // 8)
    v = qw_grouped.reshape(E, K // 32, N // 64, 4, 16, 4)  # e, g, j, b, l, c
    return np.ascontiguousarray(v.transpose(0, 1, 3, 2, 4, 5)).reshape(E, K // 8, N)

