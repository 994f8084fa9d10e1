"""The test helpers that spell out the GROUPED code layout, checked element by
element against the layout's definition (slot 16b + l of block j of group g
holds word 4g + b of columns 64j + 4l .. 64j + 4l + 3)."""
import itertools

import numpy as np

from helpers import canonical_words, grouped_words


def test_grouped_words_follow_the_slot_definition():
    rng = np.random.default_rng(3)
    E, K, N = 2, 64, 128
    G = K // 32
    qw = rng.integers(-(2 ** 31), 2 ** 31, size=(E, K // 8, N), dtype=np.int64).astype(np.int32)
    flat = grouped_words(qw).reshape(-1)
    assert flat.size == qw.size
    for e, g, j, b, l, c in itertools.product(range(E), range(G), range(N // 64), range(4), range(16), range(4)):
        pos = ((e * G + g) * (N // 64) + j) * 256 + (16 * b + l) * 4 + c
        assert flat[pos] == qw[e, 4 * g + b, 64 * j + 4 * l + c]
    assert np.array_equal(canonical_words(flat, K, N), qw)
