"""Seeded synthetic inputs for the W4A16 group-32 path.

This module only draws random numbers; it holds none of the method's
arithmetic (no quantization, packing or matmul).  The same generators feed both
the library under test and the CPU oracle: a tensor is drawn once and handed to
both sides.

Every tensor is drawn from a torch generator seeded by
``SeedSequence([0, config, tag, index])``, on the device that will hold it.
Draws on the CPU and on the GPU use different streams, so a caller draws on one
device and copies to the other; the same key always gives the same values on
the same kind of device.

Workload shapes follow the synthetic stand-ins for the pages' model shapes
(hidden 7168, dense intermediate 18432, expert intermediate 2048, 384 experts,
top-8): see ``CONFIGS``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

WEIGHT_STD = 0.02

# tensor tags, so that every (config, tensor) pair has its own stream
TAG_X, TAG_GATE, TAG_UP, TAG_DOWN, TAG_TOPK, TAG_GATEW, TAG_ZIPF, TAG_LOGITS = range(8)
# streams of random code words and scales (drawn directly, not quantized)
TAG_CODES, TAG_SCALES = 8, 9


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    kind: str            # "gemm" | "mlp" | "moe" | "router"
    M: int
    K: int               # hidden size (input dim of gate/up, output dim of down)
    N: int               # output dim of a plain gemm, else the intermediate size
    x_dtype: str         # "f32" | "bf16"
    experts: int = 0
    top_k: int = 0
    routing: str = ""    # "uniform" | "zipf"
    zipf_alpha: float = 0.0
    shared: bool = False  # MoE layer with one shared expert of the experts' shape


CONFIGS = {
    "gemm_m1": Config("gemm_m1", 0, "gemm", 1, 256, 512, "f32"),
    "mlp_decode_m4": Config("mlp_decode_m4", 1, "mlp", 4, 7168, 18432, "f32"),
    "mlp_verify_m64_f32": Config("mlp_verify_m64_f32", 2, "mlp", 64, 7168, 18432, "f32"),
    "mlp_verify_m64_bf16": Config("mlp_verify_m64_bf16", 2, "mlp", 64, 7168, 18432, "bf16"),
    "moe_decode_m64": Config("moe_decode_m64", 3, "moe", 64, 7168, 2048, "bf16", 384, 8, "uniform"),
    "moe_prefill_m2048": Config("moe_prefill_m2048", 4, "moe", 2048, 7168, 2048, "bf16", 384, 8, "zipf", 1.1),
    "moe_decode_m64_shared": Config("moe_decode_m64_shared", 3, "moe", 64, 7168, 2048, "bf16", 384, 8, "uniform",
                                    shared=True),
    "moe_prefill_m2048_shared": Config("moe_prefill_m2048_shared", 4, "moe", 2048, 7168, 2048, "bf16", 384, 8,
                                       "zipf", 1.1, shared=True),
    "gemm_m2048_hot_expert": Config("gemm_m2048_hot_expert", 5, "gemm", 2048, 7168, 4096, "bf16"),
    # one GPU's share of the dense MLP under 8-way tensor parallelism: gate/up
    # column-parallel (N = 18432 / 8), down row-parallel (K = 18432 / 8)
    "mlp_decode_m4_tp8": Config("mlp_decode_m4_tp8", 6, "mlp", 4, 7168, 2304, "f32"),
    "mlp_verify_m64_bf16_tp8": Config("mlp_verify_m64_bf16_tp8", 6, "mlp", 64, 7168, 2304, "bf16"),
    # router (top-k gating) ahead of the two MoE layers: float32 logits [M][384]
    "router_m64": Config("router_m64", 3, "router", 64, 0, 0, "f32", 384, 8),
    "router_m2048": Config("router_m2048", 4, "router", 2048, 0, 0, "f32", 384, 8),
}


# expert index of a shared expert's weight streams (the routed experts use 0 .. E-1)
SHARED_EXPERT_INDEX = 10_000


def seed_of(config: int, tag: int, index: int = 0) -> int:
    """63-bit seed for one tensor of one workload."""
    st = np.random.SeedSequence([0, int(config), int(tag), int(index)]).generate_state(2, np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std, config, tag, index=0, device="cpu") -> torch.Tensor:
    """float32 N(0, std^2) samples, drawn as N(0,1) and multiplied by std in float32."""
    g = _gen(device, seed_of(config, tag, index))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def activations(M, K, config, dtype="f32", index=0, device="cpu") -> torch.Tensor:
    """x[M][K] ~ N(0,1) in float32; for bf16 runs rounded to nearest-even bf16."""
    x = normal((M, K), 1.0, config, TAG_X, index, device)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def weights(K, N, config, tag, index=0, device="cpu") -> torch.Tensor:
    """Unquantized weights W[K][N] ~ N(0, 0.02^2) in float32."""
    return normal((K, N), WEIGHT_STD, config, tag, index, device)


def router_logits(M, E, config, index=0, device="cpu") -> torch.Tensor:
    """Router logits[M][E] ~ N(0,1) in float32."""
    return normal((M, E), 1.0, config, TAG_LOGITS, index, device)


def topk_uniform(M, E, k, config, index=0) -> np.ndarray:
    """k distinct expert ids per token, uniformly at random (int32 [M][k])."""
    rng = np.random.default_rng(seed_of(config, TAG_TOPK, index))
    keys = rng.random((M, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def topk_zipf(M, E, k, alpha, config, index=0) -> np.ndarray:
    """k distinct expert ids per token with Zipf(alpha) popularity.

    Expert of popularity rank r (1..E) has weight r^-alpha; ranks are assigned
    to ids by a seeded permutation.  Each token draws k distinct ids without
    replacement, proportionally to the weights (int32 [M][k]).
    """
    rng = np.random.default_rng(seed_of(config, TAG_ZIPF, index))
    p = np.arange(1, E + 1, dtype=np.float64) ** (-alpha)
    p /= p.sum()
    ids_by_rank = rng.permutation(E)
    out = np.empty((M, k), dtype=np.int32)
    for t in range(M):
        r = rng.choice(E, size=k, replace=False, p=p)
        out[t] = ids_by_rank[r]
    return out


def gate_weights(M, k, config, index=0) -> np.ndarray:
    """Per-token gate weights: softmax over the k chosen slots of N(0,1) logits (float32 [M][k])."""
    rng = np.random.default_rng(seed_of(config, TAG_GATEW, index))
    z = rng.standard_normal((M, k))
    z = np.exp(z - z.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def code_words(K, N, config, tag, index=0, device="cpu") -> torch.Tensor:
    """Random 32-bit words [K/8][N] as int32, every bit uniform: each nibble is
    uniform over 0..15, so code 0 (value -8) appears as often as any other.
    ``tag`` names the matrix (TAG_GATE, TAG_UP, TAG_DOWN)."""
    g = _gen(device, seed_of(config, TAG_CODES * 16 + tag, index))
    w = torch.randint(-(2 ** 31), 2 ** 31, (K // 8, N), generator=g, device=device, dtype=torch.int64)
    return w.to(torch.int32)


def scale_values(G, N, config, tag, index=0, lo=0.004, hi=0.009, device="cpu") -> torch.Tensor:
    """Random float32 scales [G][N], uniform in [lo, hi) (the range that
    max|w| / 7 takes for 32 draws of N(0, 0.02^2))."""
    g = _gen(device, seed_of(config, TAG_SCALES * 16 + tag, index))
    return torch.rand((G, N), generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo
