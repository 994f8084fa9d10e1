"""CPU checks of the parity tests' element-wise bound machinery
(tests/oracle_pool.py): its fast dequantization equals the oracle's float32
dequantization bit for bit, the bounds hold for a float32 evaluation of the
same products, and a wrong element exceeds them."""
import numpy as np

import oracle as O
import oracle_pool as P


def _codes(rng, K, N):
    qw = rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint64).astype(np.uint32).view(np.int32)
    sc = (rng.random((K // 32, N)) * 0.005 + 0.004).astype(np.float32)
    return qw, sc


def test_fast_dequant_equals_oracle_dequant32():
    rng = np.random.default_rng(1)
    for K, N, g in ((256, 64, 32), (512, 128, 64), (1024, 64, 128)):
        qw = rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint64).astype(np.uint32).view(np.int32)
        sc = (rng.standard_normal((K // g, N))).astype(np.float32)
        assert np.array_equal(P.dequant_f32(qw, sc).view(np.uint32), O.dequant32(qw, sc).view(np.uint32))


def test_bounds_hold_for_float32_evaluation_and_catch_a_wrong_element():
    rng = np.random.default_rng(2)
    H, I, M = 512, 256, 6
    gate, up, down = _codes(rng, H, I), _codes(rng, H, I), _codes(rng, I, H)
    x = rng.standard_normal((M, H)).astype(np.float32)
    ref = O.swiglu_mlp64(x, gate, up, down)
    # a float32 evaluation (inputs rounded to bf16: 8 significant bits)
    xb = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)
    g, u = xb @ P.dequant_f32(*gate), xb @ P.dequant_f32(*up)
    h = (g / (1 + np.exp(-g))) * u
    y = h @ P.dequant_f32(*down)
    b = P.mlp_bound(x, gate, up, down, P.TAU["bf16"])
    assert P.check_elementwise(y, ref, b, "float32 mlp") < 1.0
    bf = P.mlp_bound(x, gate, up, down, P.TAU["f32"])
    bad = ref.copy()
    bad[2, 5] += 0.05 * np.abs(ref).max()
    assert ((np.abs(bad - ref) > bf).sum()) == 1
    gb = P.gemm_bound(x, *gate, P.TAU["f32"])
    assert (gb >= P.TAU["f32"] * O.gemm_abs64(x, *gate)).all()
