"""GPU parity of the weight-format kernels against the oracle: the quantizer
and dequantize are bit-exact, prepack is the stated permutation."""
import numpy as np
import pytest
import torch

import int4_w4a16_group_g32_amd as L
import oracle as O
import workloads as W
from helpers import canonical_words, grouped_words, to_dev, weight_from_codes

pytestmark = pytest.mark.gpu


def _gpu_quantize(w_np):
    E = 1 if w_np.ndim == 2 else w_np.shape[0]
    K, N = w_np.shape[-2:]
    w = to_dev(w_np.astype(np.float32))
    qw = torch.empty((E, K // 8, N), dtype=torch.int32, device="cuda")
    sc = torch.empty((E, K // 32, N), dtype=torch.float32, device="cuda")
    L.quantize(w, qw, sc)
    return qw.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("K,N,seed", [(32, 64, 0), (256, 512, 1), (1024, 192, 2), (7168, 128, 3)])
def test_quantize_bit_exact(K, N, seed):
    w = W.weights(K, N, 100 + seed, W.TAG_GATE).numpy()
    w[:, 5] = 0.0                      # an all-zero column
    w[:64, 7] = np.float32(1e-30)      # tiny values
    w[32:64, 9] = -w[32:64, 9]
    qw, sc = _gpu_quantize(w)
    qo, so = O.quantize_w4a16(w)
    assert np.array_equal(qw[0], qo)
    assert np.array_equal(sc[0].view(np.uint32), so.view(np.uint32))


def test_quantize_half_way_ties_and_stack():
    """Exact half-way quotients (ties to even) and a two-expert stack."""
    rng = np.random.default_rng(5)
    K, N = 64, 64
    s = np.ldexp(1.0, rng.integers(-10, -2, size=(K // 32, N)))
    t = rng.integers(-14, 15, size=(K, N)) / 2.0          # multiples of 1/2 in [-7, 7]
    t[::32] = 7.0
    w = (t * np.repeat(s, 32, axis=0)).astype(np.float32)
    stack = np.stack([w, -w])
    qw, sc = _gpu_quantize(stack)
    for e in range(2):
        qo, so = O.quantize_w4a16(stack[e])
        assert np.array_equal(qw[e], qo) and np.array_equal(sc[e], so)


def test_prepack_is_the_grouped_slot_permutation():
    rng = np.random.default_rng(9)
    E, K, N = 3, 256, 192
    qw = rng.integers(-(2 ** 31), 2 ** 31, size=(E, K // 8, N), dtype=np.int64).astype(np.int32)
    sc = rng.random((E, K // 32, N)).astype(np.float32)
    w = weight_from_codes(qw, sc)
    got = w.qw.cpu().numpy()
    assert w.layout == L.LAYOUT_GROUPED and got.size == qw.size
    assert np.array_equal(got.reshape(E, K // 32, N // 64, 64, 4), grouped_words(qw))
    assert np.array_equal(canonical_words(got, K, N), qw)


@pytest.mark.parametrize("grouped", [False, True])
def test_dequantize_bit_exact(grouped):
    K, N = 1024, 256
    qw, sc = O.quantize_w4a16(W.weights(K, N, 7, W.TAG_UP).numpy())
    canon = L.Weight(to_dev(qw[None]), to_dev(sc[None]), K, N, 1, L.LAYOUT_CANONICAL)
    w = L.prepack(canon, torch.empty_like(canon.qw)) if grouped else canon
    out = torch.empty((1, K, N), dtype=torch.float32, device="cuda")
    L.dequantize(w, out)
    ref = O.dequant32(qw, sc)
    assert np.array_equal(out[0].cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_dequantize_every_nibble_every_position():
    """Every nibble value at every word position, with scales spanning many binades."""
    K, N = 128, 64
    nib = np.zeros((K, N), dtype=np.int64)
    for n in range(N):
        for k in range(K):
            nib[k, n] = (k + 3 * n) % 16
    qw = O.pack_nibbles(nib)
    sc = np.ldexp(np.random.default_rng(1).random((K // 32, N)) + 0.5,
                  np.random.default_rng(2).integers(-40, 20, size=(K // 32, N))).astype(np.float32)
    w = weight_from_codes(qw, sc)
    out = torch.empty((1, K, N), dtype=torch.float32, device="cuda")
    L.dequantize(w, out)
    assert np.array_equal(out[0].cpu().numpy().view(np.uint32), O.dequant32(qw, sc).view(np.uint32))
