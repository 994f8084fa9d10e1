"""Pins for the CPU oracle against facts that do not come from the oracle itself:
hand-worked fixtures, exhaustive enumeration, exact rational brute force, closed
forms and invariants.  Each test names the plausible oracle mistake it catches.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def _u32_to_i32(h):
    v = int(h, 16)
    return v - (1 << 32) if v >= (1 << 31) else v


# ---------------------------------------------------------------- pack / unpack

def test_unpack_every_nibble_at_every_position():
    """Exhaustive: nibble v at position j decodes to v - 8 at row 8i+j and leaves
    the others at 0.  Catches a wrong nibble order, a missing -8 or a sign slip."""
    for j in range(8):
        for v in range(16):
            word = 0x88888888 & ~(0xF << (4 * j)) | (v << (4 * j))
            qw = np.array([[_u32_to_i32(hex(word))]], dtype=np.int32)
            q = O.unpack(qw)[:, 0]
            want = np.zeros(8, dtype=np.int64)
            want[j] = v - 8
            assert q.tolist() == want.tolist(), (j, v)


def test_unpack_special_words():
    """-1 must give +7 everywhere (logical shift), 0 gives -8, 0x88888888 gives 0,
    0x76543210 gives -8..-1 in row order.  Catches an arithmetic shift."""
    words = np.array([[-1, 0, _u32_to_i32("0x88888888"), 0x76543210]], dtype=np.int32)
    q = O.unpack(words)
    assert (q[:, 0] == 7).all()
    assert (q[:, 1] == -8).all()
    assert (q[:, 2] == 0).all()
    assert q[:, 3].tolist() == list(range(-8, 0))


def test_pack_unpack_round_trip_random_words():
    rng = np.random.default_rng(1234)
    words = rng.integers(-(2 ** 31), 2 ** 31, size=(4096, 25), dtype=np.int64).astype(np.int32)
    q = O.unpack(words)
    assert q.min() >= -8 and q.max() <= 7
    again = O.pack_nibbles(q.astype(np.int64) + 8)
    assert np.array_equal(again, words)


# ---------------------------------------------------------------- quantizer

def test_quantize_hand_worked_fixture():
    """The hand-worked group in tests/golden/quantize_hand.txt: codes, words and
    scales.  Catches high-nibble-first packing, a +8 offset slip, round-half-away,
    a wrong scale rule (e.g. max/8) and NaN on an all-zero group."""
    fx = _read_fixture("quantize_hand.txt")
    s0, s2 = 2.0 ** -6, 2.0 ** -3
    w = np.zeros((32, 3), dtype=np.float32)
    w[:, 0] = np.array([float(v) for v in fx["w_over_scale_col0"]]) * s0
    w[:, 2] = np.array([float(v) for v in fx["w_over_scale_col2"]]) * s2
    qw, sc = O.quantize_w4a16(w)
    assert qw.shape == (4, 3) and sc.shape == (1, 3)
    assert sc[0].tolist() == [s0, 0.0, s2]
    for c in range(3):
        want = [_u32_to_i32(h) for h in fx[f"words_col{c}"]]
        assert qw[:, c].tolist() == want, c
    assert O.unpack(qw)[:, 0].tolist() == [int(v) for v in fx["codes_col0"]]


def test_quantizer_invariants_on_weight_distribution():
    """N(0, 0.02) weights: every nonzero group reaches |q| = 7, nibbles stay in
    1..15 (q = -8 cannot occur with scale = max/7) and |w - q*s| <= s/2."""
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((1024, 96)) * 0.02).astype(np.float32)
    qw, sc = O.quantize_w4a16(w)
    q = O.unpack(qw).astype(np.int64)
    g = np.abs(q).reshape(32, 32, 96).max(axis=1)
    assert (g == 7).all()
    assert q.min() >= -7 and q.max() <= 7
    s = np.repeat(sc, 32, axis=0).astype(np.float64)
    err = np.abs(w.astype(np.float64) - q * s)
    assert (err <= 0.5 * s * (1 + 1e-12)).all()
    assert float((err / s).max()) > 0.45  # the bound is attained, not vacuous


def test_quantizer_zero_and_single_value_groups():
    w = np.zeros((64, 2), dtype=np.float32)
    w[40, 1] = -3.0
    qw, sc = O.quantize_w4a16(w)
    assert sc[:, 0].tolist() == [0.0, 0.0] and sc[0, 1] == 0.0
    assert sc[1, 1] == np.float32(3.0) / np.float32(7.0)
    q = O.unpack(qw)
    assert (q[:, 0] == 0).all()
    assert q[40, 1] == -7 and np.count_nonzero(q[:, 1]) == 1


def test_quantizer_power_of_two_groups_are_exact():
    """Integer codes times a power-of-two scale, with max |code| = 7, quantize back
    to exactly those codes and that scale."""
    rng = np.random.default_rng(3)
    K, N = 256, 16
    q = rng.integers(-7, 8, size=(K, N))
    q[::32, :] = 7 * np.where(rng.random((K // 32, N)) < 0.5, 1, -1)
    e = rng.integers(-12, 0, size=(K // 32, N))
    s = np.ldexp(1.0, e)
    w = (q * np.repeat(s, 32, axis=0)).astype(np.float32)
    qw, sc = O.quantize_w4a16(w)
    assert np.array_equal(O.unpack(qw), q)
    assert np.array_equal(sc.astype(np.float64), s)


# ---------------------------------------------------------------- dequant

def test_dequant32_is_one_float32_multiply():
    """float32(q*s) equals IEEE float32 multiplication of the two float32 values
    (numpy's float32 multiply), on a full K=7168 slab."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((7168, 64)) * 0.02).astype(np.float32)
    qw, sc = O.quantize_w4a16(w)
    d = O.dequant32(qw, sc)
    lib = O.unpack(qw).astype(np.float32) * np.repeat(sc, 32, axis=0)
    assert d.dtype == np.float32
    assert np.array_equal(d.view(np.uint32), lib.view(np.uint32))


def test_dequant_power_of_two_closed_form():
    nib = np.tile(np.arange(16), 4).reshape(64, 1)
    qw = O.pack_nibbles(nib)
    sc = np.array([[2.0 ** -5], [2.0 ** -9]], dtype=np.float32)
    d = O.dequant64(qw, sc)[:, 0]
    want = np.concatenate([np.ldexp(np.arange(-8, 8, dtype=np.float64), -5)] * 2
                          + [np.ldexp(np.arange(-8, 8, dtype=np.float64), -9)] * 2)
    assert np.array_equal(d, want)


# ---------------------------------------------------------------- gemm

def _dyadic(rng, shape, bits, lo_exp, hi_exp):
    m = rng.integers(-(2 ** bits), 2 ** bits, size=shape)
    e = rng.integers(lo_exp, hi_exp, size=shape)
    return np.ldexp(m.astype(np.float64), e).astype(np.float32)


@pytest.mark.parametrize("M,K,N", [(1, 32, 1), (3, 64, 8), (2, 64, 5)])
def test_gemm64_matches_exact_rational_brute_force(M, K, N):
    """Scalar Fraction loop, y[m][n] = sum_k x*q*s, exact.  Inputs carry few
    significant bits so the float64 result must be exact too.  Catches a
    transposed operand, a dropped group scale or a wrong group index."""
    rng = np.random.default_rng(M * 100 + K + N)
    x = _dyadic(rng, (M, K), 6, -3, 3)
    q = rng.integers(-8, 8, size=(K, N))
    qw = O.pack_nibbles(q + 8)
    sc = _dyadic(rng, (K // 32, N), 6, -8, -2)
    sc = np.abs(sc) + np.float32(2.0 ** -8)
    y = O.gemm64(x, qw, sc)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(x[m, k])) * int(q[k, n]) * Fraction(float(sc[k // 32, n]))
            assert Fraction(float(y[m, n])) == acc, (m, n)


def test_gemm64_constant_nibble_closed_form():
    K, N = 7168, 4
    for c in (0, 3, 8, 15):
        qw = O.pack_nibbles(np.full((K, N), c))
        sc = np.full((K // 32, N), 2.0 ** -7, dtype=np.float32)
        y = O.gemm64(np.ones((2, K), dtype=np.float32), qw, sc)
        assert (y == K * (c - 8) * 2.0 ** -7).all()


def test_quantization_is_real():
    """INT4 output differs from the unquantized product by far more than any
    kernel tolerance (about 10 %), so a no-op path cannot pass parity."""
    rng = np.random.default_rng(5)
    K, N = 7168, 128
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    x = rng.standard_normal((4, K)).astype(np.float32)
    qw, sc = O.quantize_w4a16(w)
    r = O.rel_frobenius(O.gemm64(x, qw, sc), x.astype(np.float64) @ w.astype(np.float64))
    assert 0.05 < r < 0.2, r


# ---------------------------------------------------------------- SwiGLU MLP

def _rand_weights(rng, K, N, std=0.02):
    return O.quantize_w4a16((rng.standard_normal((K, N)) * std).astype(np.float32))


def test_swiglu_zero_up_or_gate_gives_zero():
    rng = np.random.default_rng(9)
    H, I = 64, 96
    x = rng.standard_normal((3, H)).astype(np.float32)
    g, u, d = _rand_weights(rng, H, I), _rand_weights(rng, H, I), _rand_weights(rng, I, H)
    zero = (O.pack_nibbles(np.full((H, I), 8)), np.ones((H // 32, I), dtype=np.float32))
    assert (O.swiglu_mlp64(x, g, zero, d) == 0).all()
    assert (O.swiglu_mlp64(x, zero, u, d) == 0).all()


def test_swiglu_scalar_loop_brute_force():
    """Pure-Python loops with math.exp on H=32, I=32.  Catches a swapped gate and
    up, a sign slip in the SiLU, or a missing down projection."""
    rng = np.random.default_rng(21)
    H, I = 32, 32
    x = rng.standard_normal((2, H)).astype(np.float32)
    g, u, d = _rand_weights(rng, H, I, 0.3), _rand_weights(rng, H, I, 0.3), _rand_weights(rng, I, H, 0.3)
    qg, qu, qd = O.unpack(g[0]), O.unpack(u[0]), O.unpack(d[0])
    y = O.swiglu_mlp64(x, g, u, d)
    for m in range(2):
        h = []
        for i in range(I):
            a = sum(float(x[m, k]) * int(qg[k, i]) * float(g[1][k // 32, i]) for k in range(H))
            b = sum(float(x[m, k]) * int(qu[k, i]) * float(u[1][k // 32, i]) for k in range(H))
            h.append(a / (1.0 + math.exp(-a)) * b)
        for n in range(H):
            want = sum(h[i] * int(qd[i, n]) * float(d[1][i // 32, n]) for i in range(I))
            assert abs(y[m, n] - want) <= 1e-12 * max(1.0, abs(want)), (m, n)


# ---------------------------------------------------------------- routing

def test_route_hand_worked_fixture():
    fx = _read_fixture("route_hand.txt")
    E = int(fx["num_experts"][0])
    ids = np.array([int(v) for v in fx["topk_ids"]]).reshape(3, 2)
    counts, offsets, sp, inv = O.route(ids, E)
    assert counts.tolist() == [int(v) for v in fx["counts"]]
    assert offsets.tolist() == [int(v) for v in fx["offsets"]]
    assert sp.tolist() == [int(v) for v in fx["sorted_pairs"]]
    assert inv.tolist() == [int(v) for v in fx["inv"]]


def test_route_against_python_loops():
    rng = np.random.default_rng(17)
    M, E, k = 200, 40, 8
    ids = np.stack([rng.permutation(E)[:k] for _ in range(M)])
    counts, offsets, sp, inv = O.route(ids, E)
    brute = [t * k + s for e in range(E) for t in range(M) for s in range(k) if ids[t, s] == e]
    assert sp.tolist() == brute
    assert counts.sum() == M * k and (np.diff(offsets) == counts).all()
    assert (inv[sp] == np.arange(M * k)).all()


# ---------------------------------------------------------------- MoE

def _experts(rng, E, H, I):
    ws = [(_rand_weights(rng, H, I), _rand_weights(rng, H, I), _rand_weights(rng, I, H)) for _ in range(E)]
    return lambda e: ws[e]


def test_moe_matches_per_token_per_slot_loop():
    """Grouped-by-expert evaluation equals the per-(token, slot) definition,
    summed in slot order."""
    rng = np.random.default_rng(31)
    M, E, k, H, I = 9, 6, 3, 64, 32
    x = rng.standard_normal((M, H)).astype(np.float32)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(M)])
    w = rng.random((M, k)).astype(np.float32)
    ex = _experts(rng, E, H, I)
    y = O.moe64(x, ids, w, ex, E)
    for t in range(M):
        want = np.zeros(H)
        for s in range(k):
            want += float(w[t, s]) * O.swiglu_mlp64(x[t:t + 1], *ex(int(ids[t, s])))[0]
        assert np.allclose(y[t], want, rtol=0, atol=1e-13 * np.abs(want).max())


def test_moe_special_cases():
    rng = np.random.default_rng(37)
    M, E, k, H, I = 7, 5, 2, 32, 64
    x = rng.standard_normal((M, H)).astype(np.float32)
    ex = _experts(rng, E, H, I)
    # one expert, top-1, weight 1: the dense MLP
    y = O.moe64(x, np.zeros((M, 1), dtype=np.int64), np.ones((M, 1)), ex, 1)
    assert np.array_equal(y, O.swiglu_mlp64(x, *ex(0)))
    # one-hot gate weights select a single expert per token
    ids = np.stack([rng.permutation(E)[:k] for _ in range(M)])
    w = np.zeros((M, k))
    w[:, 1] = 1.0
    y = O.moe64(x, ids, w, ex, E)
    for t in range(M):
        want = O.swiglu_mlp64(x[t:t + 1], *ex(int(ids[t, 1])))[0]
        assert np.allclose(y[t], want, rtol=1e-13, atol=1e-13 * np.abs(want).max())
    # permuting tokens permutes output rows; a token subset gives those rows
    wr = rng.random((M, k))
    perm = rng.permutation(M)
    y0 = O.moe64(x, ids, wr, ex, E)
    y1 = O.moe64(x[perm], ids[perm], wr[perm], ex, E)
    assert np.allclose(y1, y0[perm], rtol=1e-14, atol=1e-15)
    sub = O.moe64(x, ids, wr, ex, E, tokens=[5, 2])
    assert np.allclose(sub, y0[[5, 2]], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- router (top-k gating)

def _topk_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "topk_hand.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"k": int(vals[0])}
                cases.append(cur)
            else:
                cur[key] = vals
    return cases


def _closed_form(expr):
    """Evaluate a fixture weight written in e = exp(1): only 1, 2, e and / + ( )."""
    assert set(expr) <= set("0123456789e/+() ")
    return eval(expr, {"__builtins__": {}}, {"e": math.e})


def test_topk_hand_worked_fixture():
    for c in _topk_cases():
        logits = np.array([[float(v) for v in c["logits"]]])
        ids, w = O.moe_topk(logits, c["k"])
        assert ids[0].tolist() == [int(v) for v in c["ids"]]
        np.testing.assert_allclose(w[0], [_closed_form(v) for v in c["weights"]], rtol=1e-14, atol=0)


def test_topk_all_experts_is_a_full_softmax_in_descending_order():
    rng = np.random.default_rng(7)
    lg = rng.standard_normal((5, 37))
    ids, w = O.moe_topk(lg, 37)
    for t in range(5):
        assert sorted(ids[t].tolist()) == list(range(37))
        assert np.all(np.diff(lg[t, ids[t]]) <= 0)
        full = np.exp(lg[t] - lg[t].max())
        full /= full.sum()
        np.testing.assert_allclose(w[t], full[ids[t]], rtol=1e-13, atol=0)


def test_topk_brute_force_selection_and_ties():
    """Integer logits with many ties: every chosen logit is >= every unchosen
    one, equal logits are taken in ascending index, and the weights are a
    softmax over the chosen logits (sum 1, shift invariant)."""
    rng = np.random.default_rng(8)
    lg = rng.integers(-3, 4, size=(40, 16)).astype(np.float64)
    for k in (1, 3, 8, 16):
        ids, w = O.moe_topk(lg, k)
        shifted_ids, shifted_w = O.moe_topk(lg + 123.0, k)
        assert np.array_equal(ids, shifted_ids)
        np.testing.assert_allclose(w, shifted_w, rtol=1e-12)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-13)
        for t in range(lg.shape[0]):
            chosen = set(ids[t].tolist())
            rest = [e for e in range(16) if e not in chosen]
            if rest:
                assert lg[t, ids[t]].min() >= lg[t, rest].max()
            for a, b in zip(ids[t][:-1], ids[t][1:]):
                assert lg[t, a] > lg[t, b] or (lg[t, a] == lg[t, b] and a < b)
            # the boundary: an unchosen expert tied with the last chosen one has a larger index
            last = ids[t][-1]
            for e in rest:
                if lg[t, e] == lg[t, last]:
                    assert e > last


# ---------------------------------------------------------------- shared expert

def test_moe_shared_special_cases():
    """The shared expert adds one SwiGLU MLP with weight 1: zero routed gate
    weights leave exactly the shared MLP; an all-zero shared expert (zero
    scales) leaves exactly the routed sum; a per-token loop agrees."""
    rng = np.random.default_rng(41)
    M, E, k, H, I = 6, 5, 2, 32, 64
    x = rng.standard_normal((M, H)).astype(np.float32)
    ex = _experts(rng, E, H, I)
    sh = _experts(rng, 1, H, I)(0)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(M)])
    w = rng.random((M, k))
    y0 = O.moe_shared64(x, ids, np.zeros((M, k)), ex, E, sh)
    assert np.array_equal(y0, O.swiglu_mlp64(x, *sh))
    zero = tuple((qw, np.zeros_like(sc)) for qw, sc in sh)
    assert np.array_equal(O.moe_shared64(x, ids, w, ex, E, zero), O.moe64(x, ids, w, ex, E))
    y = O.moe_shared64(x, ids, w, ex, E, sh)
    for t in range(M):
        want = np.zeros(H)
        for s in range(k):
            want += w[t, s] * O.swiglu_mlp64(x[t:t + 1], *ex(int(ids[t, s])))[0]
        want += O.swiglu_mlp64(x[t:t + 1], *sh)[0]
        assert np.allclose(y[t], want, rtol=0, atol=1e-13 * np.abs(want).max())
    sub = O.moe_shared64(x, ids, w, ex, E, sh, tokens=[4, 1])
    assert np.allclose(sub, y[[4, 1]], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- other group sizes (64, 128)

@pytest.mark.parametrize("group", [64, 128])
def test_quantizer_invariants_other_group_sizes(group):
    """One scale per `group` rows: every nonzero group reaches |q| = 7, the
    scale is the group's max|w| / 7 in float32, and |w - q*s| <= s/2."""
    rng = np.random.default_rng(group)
    K, N = 1024, 48
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    qw, sc = O.quantize_w4a16(w, group)
    assert sc.shape == (K // group, N)
    q = O.unpack(qw).astype(np.int64)
    assert (np.abs(q).reshape(K // group, group, N).max(axis=1) == 7).all()
    m = np.abs(w).reshape(K // group, group, N).max(axis=1)
    assert np.array_equal(sc, (m / np.float32(7.0)).astype(np.float32))
    s = np.repeat(sc, group, axis=0).astype(np.float64)
    err = np.abs(w.astype(np.float64) - q * s)
    assert (err <= 0.5 * s * (1 + 1e-12)).all()


@pytest.mark.parametrize("group", [64, 128])
def test_quantizer_power_of_two_groups_are_exact_other_sizes(group):
    rng = np.random.default_rng(group + 1)
    K, N = 512, 8
    q = rng.integers(-7, 8, size=(K, N))
    q[::group, :] = 7
    s = np.ldexp(1.0, rng.integers(-12, 0, size=(K // group, N)))
    w = (q * np.repeat(s, group, axis=0)).astype(np.float32)
    qw, sc = O.quantize_w4a16(w, group)
    assert np.array_equal(O.unpack(qw), q)
    assert np.array_equal(sc.astype(np.float64), s)


@pytest.mark.parametrize("M,K,N,group", [(2, 128, 3, 64), (1, 256, 2, 128), (2, 256, 3, 64)])
def test_gemm64_brute_force_other_group_sizes(M, K, N, group):
    """The scale of row k is sc[k // group]: a Fraction loop with that index."""
    rng = np.random.default_rng(M * 7 + K + group)
    x = _dyadic(rng, (M, K), 6, -3, 3)
    q = rng.integers(-8, 8, size=(K, N))
    qw = O.pack_nibbles(q + 8)
    sc = np.abs(_dyadic(rng, (K // group, N), 6, -8, -2)) + np.float32(2.0 ** -8)
    y = O.gemm64(x, qw, sc)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(x[m, k])) * int(q[k, n]) * Fraction(float(sc[k // group, n]))
            assert Fraction(float(y[m, n])) == acc, (m, n)


# ---------------------------------------------------------------- error-bound scale, metric, map_fn

@pytest.mark.parametrize("M,K,N", [(1, 32, 1), (3, 64, 8), (2, 96, 5)])
def test_gemm_abs64_matches_exact_rational_brute_force(M, K, N):
    """sum_k |x| * |q| * |s| by a scalar Fraction loop, exact on dyadic inputs
    (negative scales included, so a dropped abs on either factor fails)."""
    rng = np.random.default_rng(7 * M + K + N)
    x = _dyadic(rng, (M, K), 6, -3, 3)
    q = rng.integers(-8, 8, size=(K, N))
    qw = O.pack_nibbles(q + 8)
    sc = _dyadic(rng, (K // 32, N), 6, -8, -2)
    y = O.gemm_abs64(x, qw, sc)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += abs(Fraction(float(x[m, k]))) * abs(int(q[k, n])) * abs(Fraction(float(sc[k // 32, n])))
            assert Fraction(float(y[m, n])) == acc, (m, n)


def test_gemm_abs64_bounds_gemm64_and_equals_it_for_nonnegative_terms():
    rng = np.random.default_rng(41)
    K, N = 256, 64
    x = rng.standard_normal((5, K)).astype(np.float32)
    q = rng.integers(-8, 8, size=(K, N))
    sc = (rng.random((K // 32, N)) + 0.5).astype(np.float32)
    qw = O.pack_nibbles(q + 8)
    assert (np.abs(O.gemm64(x, qw, sc)) <= O.gemm_abs64(x, qw, sc)).all()
    assert np.array_equal(O.gemm_abs64(-x, qw, sc), O.gemm_abs64(x, qw, sc))
    # every term nonnegative (x >= 0, q >= 0, s > 0): the two coincide
    qp = O.pack_nibbles(np.minimum(np.abs(q), 7) + 8)
    assert np.array_equal(O.gemm_abs64(np.abs(x), qp, sc), O.gemm64(np.abs(x), qp, sc))


def test_rel_frobenius_hand_values():
    """||y - ref||_F / ||ref||_F worked by hand: y = [3, 4], ref = [0, 5] gives
    ||[3, -1]|| / 5 = sqrt(10) / 5; a matrix case; equal inputs give 0; a zero
    reference returns the absolute norm."""
    assert O.rel_frobenius([3.0, 4.0], [0.0, 5.0]) == pytest.approx(np.sqrt(10.0) / 5.0, rel=1e-15)
    assert O.rel_frobenius([[1.0, 2.0], [2.0, 0.0]], [[1.0, 0.0], [0.0, 0.0]]) == pytest.approx(np.sqrt(8.0),
                                                                                              rel=1e-15)
    assert O.rel_frobenius([[1.0, -2.0]], [[1.0, -2.0]]) == 0.0
    assert O.rel_frobenius([0.0, 3.0, 4.0], [0.0, 0.0, 0.0]) == 5.0


def test_moe_map_fn_and_repeated_ids():
    """The experts' MLPs are independent: evaluating them in another order
    gives the same bits.  A token that names one expert twice gets that
    expert's output once per slot (the per-(token, slot) definition)."""
    rng = np.random.default_rng(43)
    M, E, k, H, I = 6, 4, 3, 32, 64
    x = rng.standard_normal((M, H)).astype(np.float32)
    ex = _experts(rng, E, H, I)
    ids = rng.integers(0, E, size=(M, k))
    ids[0] = [2, 2, 1]
    ids[1] = [3, 3, 3]
    w = rng.random((M, k)).astype(np.float32)
    y = O.moe64(x, ids, w, ex, E)

    def reversed_map(fn, it):
        jobs = list(it)
        return [fn(j) for j in jobs[::-1]][::-1]

    assert np.array_equal(O.moe64(x, ids, w, ex, E, map_fn=reversed_map), y)
    for t in range(M):
        want = np.zeros(H)
        for s in range(k):
            want += float(w[t, s]) * O.swiglu_mlp64(x[t:t + 1], *ex(int(ids[t, s])))[0]
        assert np.allclose(y[t], want, rtol=0, atol=1e-13 * np.abs(want).max())
