"""Plain, slow, obviously correct numpy definition of the W4A16 group-32 path.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.

Sources (web pages, cited by title and section):
  [WP] "The Weight of Precision: Building Native INT4 Quantization for a Custom
       Speculative Decoding Engine"
  [FL] "The First Line of Code: Implementing W4A16 Quantization in a Native
       Speculative Decoding Engine"
  [FW] "The Final Wire: How a Single Edit Integrated INT4 Quantization into a
       Native DDTree Inference Engine"

Everything is float64 unless a function says otherwise.  Where the pages leave
a step open the reading taken is stated in the function's docstring.

Parity status: every function here is pinned by tests/test_oracle_pins.py
against closed forms, brute force or hand-worked fixtures.
"""
from __future__ import annotations

import numpy as np

GROUP = 32  # [WP] "The Kernel: w4a16_gemm": per-group scales at group size 32.
_NIB_PER_WORD = 8  # [WP] "The Kernel": 8 nibbles per int32 along the input dim.


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """Pack unsigned nibbles nib[K][N] (0..15) into int32 words [K/8][N].

    [WP] "The Kernel: w4a16_gemm" and [FL] "What the Edit Actually Does": eight
    4-bit values per int32 (two per byte) along the input dimension K.  Reading
    taken where the pages are silent on order: nibble j of word (i, n) holds
    row k = 8*i + j, lowest k in the least significant nibble.
    """
    nib = np.asarray(nib)
    K, N = nib.shape
    assert K % _NIB_PER_WORD == 0
    assert nib.min(initial=0) >= 0 and nib.max(initial=0) <= 15
    v = nib.astype(np.uint64).reshape(K // _NIB_PER_WORD, _NIB_PER_WORD, N)
    word = np.zeros((K // _NIB_PER_WORD, N), dtype=np.uint64)
    for j in range(_NIB_PER_WORD):
        word |= v[:, j, :] << np.uint64(4 * j)
    return word.astype(np.uint32).view(np.int32)


def unpack(qw: np.ndarray) -> np.ndarray:
    """Signed INT4 values q[K][N] from packed words qw[K/8][N].

    [WP] "The Kernel: w4a16_gemm": symmetric, value = nibble - 8, range [-8, 7].
    The shift is logical (the word is read as unsigned), so word -1 gives +7.
    """
    u = np.asarray(qw, dtype=np.int32).view(np.uint32).astype(np.int64)
    Kw, N = u.shape
    q = np.empty((Kw, _NIB_PER_WORD, N), dtype=np.int8)
    for j in range(_NIB_PER_WORD):
        q[:, j, :] = ((u >> (4 * j)) & 0xF) - 8
    return q.reshape(Kw * _NIB_PER_WORD, N)


def quantize_w4a16(w: np.ndarray, group: int = GROUP):
    """Quantize float32 weights w[K][N] to (qw int32[K/8][N], sc float32[K/group][N]).

    [WP] "The Reference and Bundle Pipeline" names the reference quantizer and
    its outputs (packed int32 words and float32 per-group scales); [FL] "What
    the Edit Actually Does" fixes symmetric groups of input rows sharing one
    scale per output column.  The pages do not print the scale rule or the
    rounding mode.  Readings taken:
      scale  s = max|w| over the group / 7, one IEEE float32 division;
      code   q = clamp(round_half_even(w / s), -8, 7), quotient taken in float64
             from the float32 operands; an all-zero group gives s = 0, q = 0.
    With s = max|w|/7 every |w/s| <= 7, so the clamp never fires and nibble 0
    (q = -8) is never produced by this quantizer.
    """
    w = np.asarray(w, dtype=np.float32)
    K, N = w.shape
    assert K % group == 0 and group % _NIB_PER_WORD == 0
    assert np.all(np.isfinite(w)), "non-finite weights are outside the format"
    g = w.reshape(K // group, group, N)
    m = np.max(np.abs(g), axis=1)                      # exact in float32
    s = (m / np.float32(7.0)).astype(np.float32)       # float32 / float32
    s64 = s.astype(np.float64)[:, None, :]
    safe = np.where(s64 == 0.0, 1.0, s64)
    r = np.where(s64 == 0.0, 0.0, g.astype(np.float64) / safe)
    q = np.clip(np.rint(r), -8, 7).astype(np.int64)    # rint: ties to even
    return pack_nibbles((q + 8).reshape(K, N)), s


def _expand_scales(sc: np.ndarray, K: int) -> np.ndarray:
    sc = np.asarray(sc, dtype=np.float32)
    G, N = sc.shape
    assert K % G == 0
    return np.repeat(sc, K // G, axis=0)


def dequant64(qw: np.ndarray, sc: np.ndarray) -> np.ndarray:
    """Exact dequantized weights q*s in float64 ([WP] "The Kernel": value = nibble - 8
    times the group's scale).  q has 4 significant bits and s 24, so the float64
    product is exact."""
    q = unpack(qw)
    return q.astype(np.float64) * _expand_scales(sc, q.shape[0]).astype(np.float64)


def dequant32(qw: np.ndarray, sc: np.ndarray) -> np.ndarray:
    """Dequantized weights rounded once to float32: float32(q*s).

    [FL] "What the Edit Actually Does": the dequantization arithmetic must be
    identical between the reference and the GPU.  This is the bit-exact
    contract for any kernel that materialises dequantized weights.
    """
    return dequant64(qw, sc).astype(np.float32)


def gemm64(x: np.ndarray, qw: np.ndarray, sc: np.ndarray) -> np.ndarray:
    """y = x @ dequant(W) in float64.

    [FW] "The Multi-Step Integration Chain": the kernel takes activations
    x[M][K], packed INT4 weights and float32 group scales and produces y[M][N];
    the reference is the dequantize-then-matmul forward.
    """
    x = np.asarray(x, dtype=np.float64)
    return x @ dequant64(qw, sc)


def gemm_abs64(a: np.ndarray, qw: np.ndarray, sc: np.ndarray) -> np.ndarray:
    """|a| @ |dequant(W)| in float64: the sum of the magnitudes of the terms of
    every dot product of gemm64.

    Not a step of the method: it is the scale against which the rounding error
    of one output element is bounded (a computed dot product differs from
    the exact one by at most a small multiple of this sum), so that a parity
    test can hold every element to a bound instead of only the norm.
    """
    a = np.abs(np.asarray(a, dtype=np.float64))
    return a @ np.abs(dequant64(qw, sc))


def silu64(z: np.ndarray) -> np.ndarray:
    """SiLU, z / (1 + exp(-z)).  The pages name SwiGLU ([WP] "The Context That
    Produced This Message"); the gate activation is read as SiLU."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_mlp64(x, gate, up, down) -> np.ndarray:
    """y = (silu(x Wg) * (x Wu)) Wd, each W given as a (qw, sc) pair.

    [FW] "What the Edit Actually Changes": the dense MLP's gate, up and down
    projections all run through the W4A16 path.  No intermediate rounding.
    """
    g = gemm64(x, *gate)
    u = gemm64(x, *up)
    h = silu64(g) * u
    return h @ dequant64(*down)


def route(topk_ids: np.ndarray, num_experts: int):
    """Group (token, slot) pairs by expert.

    [FW] "What the Edit Actually Changes": the router picks top-k experts per
    token and each chosen expert runs its gate, up and down projections.  The
    pages give no data layout; the reading taken is a stable sort of the pairs
    p = t*top_k + slot by expert id, so ties keep token order.  Returns
      counts[E], offsets[E+1] (exclusive prefix sum), sorted_pairs[M*top_k]
      (pair ids, grouped by expert, ascending token inside a group) and
      inv[M*top_k] (position of each pair in sorted_pairs).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    assert ids.ndim == 2
    flat = ids.reshape(-1)
    assert flat.size == 0 or (flat.min() >= 0 and flat.max() < num_experts)
    counts = np.bincount(flat, minlength=num_experts).astype(np.int32)
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_pairs = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty_like(sorted_pairs)
    inv[sorted_pairs] = np.arange(flat.size, dtype=np.int32)
    return counts, offsets, sorted_pairs, inv


def moe_topk(logits: np.ndarray, top_k: int):
    """Router: the top-k experts of every token and their gate weights.

    [FW] "What the Edit Actually Changes": for each token the router selects
    top-k experts.  The pages give no gating rule; the reading taken is the
    plainest one the configurations support (softmax-normalised gate weights
    over the chosen experts): the k largest logits of the token, in descending
    order with equal logits taken in ascending expert index, and weights
    softmax over those k logits, exp(l_i - l_max) / sum_j exp(l_j - l_max).
    Logits must be finite.  Returns topk_ids [M][k] int32 and topk_w [M][k]
    float64.
    """
    lg = np.asarray(logits, dtype=np.float64)
    assert lg.ndim == 2
    M, E = lg.shape
    assert 1 <= top_k <= E
    ids = np.empty((M, top_k), dtype=np.int32)
    w = np.empty((M, top_k), dtype=np.float64)
    for t in range(M):
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))
        sel = order[:top_k]
        ids[t] = sel
        z = np.exp(lg[t, sel] - lg[t, sel[0]])
        w[t] = z / z.sum()
    return ids, w


def _expert_job(job):
    xs, gate, up, down = job
    return swiglu_mlp64(xs, gate, up, down)


def moe64(x, topk_ids, topk_w, expert, num_experts, tokens=None, map_fn=map) -> np.ndarray:
    """Routed-expert SwiGLU MoE layer in float64.

    [FW] "What the Edit Actually Changes": for each token the router selects
    top-k experts and each expert applies its own gate/up/down projections.
    The pages do not state how expert outputs are combined; the reading taken
    is y[t] = sum_slot topk_w[t, slot] * expert_{topk_ids[t, slot]}(x[t]),
    summed in slot order, with the gate weights given as inputs.

    ``expert(e)`` returns ((qw_g, sc_g), (qw_u, sc_u), (qw_d, sc_d)) for expert
    e, so only experts that are used are ever dequantized.  ``tokens`` limits
    the evaluation to a subset of token rows (returned in that order).
    ``map_fn`` evaluates the experts' MLPs, which are independent of one
    another (the builtin map by default; a process pool's map runs them in
    parallel without changing any arithmetic).
    """
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids, dtype=np.int64)
    wts = np.asarray(topk_w, dtype=np.float64)
    M, top_k = ids.shape
    rows = np.arange(M) if tokens is None else np.asarray(tokens, dtype=np.int64)
    sub_ids = ids[rows]
    out = {}  # (row index in ``rows``, slot) -> expert output
    experts = np.unique(sub_ids)
    sels = [np.argwhere(sub_ids == e) for e in experts]  # (row, slot), row-major = token order
    jobs = ((x[rows[sel[:, 0]]], *expert(int(e))) for e, sel in zip(experts, sels))
    for sel, o in zip(sels, map_fn(_expert_job, jobs)):
        for (r, s), v in zip(sel, o):
            out[(int(r), int(s))] = v
    H = None
    y = None
    for r in range(len(rows)):
        for s in range(top_k):
            v = out[(r, s)]
            if y is None:
                H = v.shape[0]
                y = np.zeros((len(rows), H), dtype=np.float64)
            y[r] += wts[rows[r], s] * v
    if y is None:
        return np.zeros((len(rows), 0), dtype=np.float64)
    return y


def moe_shared64(x, topk_ids, topk_w, expert, num_experts, shared, tokens=None, map_fn=map) -> np.ndarray:
    """Routed experts plus one shared expert, float64.

    [WP] section "The Engine Dispatch: Model::linear" puts the shared expert
    on the INT4 path beside the routed experts, and [FL] section "Assumptions
    and Knowledge Boundaries" names an MoE with a shared expert.  The pages
    do not say how it joins the layer; the reading taken is the plain sum
    y[t] = (routed
    experts' weighted sum, as in moe64) + shared(x[t]) with weight 1, the
    shared term added last.  ``shared`` is ((qw_g, sc_g), (qw_u, sc_u),
    (qw_d, sc_d)) for one SwiGLU MLP of the experts' shape.
    """
    x = np.asarray(x, dtype=np.float64)
    rows = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens, dtype=np.int64)
    routed = moe64(x, topk_ids, topk_w, expert, num_experts, tokens, map_fn)
    return routed + swiglu_mlp64(x[rows], *shared)


def rel_frobenius(y, ref) -> float:
    """||y - ref||_F / ||ref||_F, computed in float64."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(y - ref)
    return float(num / den) if den > 0 else float(num)
