"""Pins for the oracle's counter-based uniforms.

Philox4x64-10 is checked against numpy.random.Philox, an independent
implementation of the same generator (Salmon et al., SC'11).  numpy increments
its 256-bit counter before producing each block of four words, so block c is
obtained by seeding numpy's counter with c - 1.
"""
import numpy as np
import pytest
from scipy import stats

import oracle


def numpy_philox(ctr, key):
    c = sum(int(x) << (64 * i) for i, x in enumerate(ctr))
    c = (c - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & ((1 << 64) - 1) for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=words)
    return [int(x) for x in bg.random_raw(4)]


def test_known_answer_zero():
    # Random123 known-answer vector for philox4x64-10 at ctr = key = 0,
    # which numpy reproduces.
    want = [0x16554D9ECA36314C, 0xDB20FE9D672D0FDC, 0xD7E772CEE186176B, 0x7E68B68AEC7BA23B]
    assert numpy_philox([0, 0, 0, 0], [0, 0]) == want
    assert oracle.philox4x64_10([0, 0, 0, 0], [0, 0]) == want


def test_against_numpy_random_counters_and_keys():
    rng = np.random.default_rng(7)
    for _ in range(300):
        ctr = [int(x) for x in rng.integers(0, 2**64, size=4, dtype=np.uint64)]
        key = [int(x) for x in rng.integers(0, 2**64, size=2, dtype=np.uint64)]
        assert oracle.philox4x64_10(ctr, key) == numpy_philox(ctr, key)


def test_against_numpy_small_counters():
    for p in range(0, 64):
        for s in range(3):
            ctr = [p, s, 5, 0]
            assert oracle.philox4x64_10(ctr, [1003, 0]) == numpy_philox(ctr, [1003, 0])


def test_uniform_words_layout():
    # key = (seed, 0), counter = (p, s, c, 0)
    assert oracle.uniform_words(1003, 17, 2, 9) == numpy_philox([17, 2, 9, 0], [1003, 0])


def test_u24_is_top_24_bits():
    for w in (0, 1, (1 << 40) - 1, 1 << 40, (1 << 64) - 1, 0x123456789ABCDEF0):
        assert oracle.u24(w) == w >> 40
    assert oracle.u24((1 << 64) - 1) == (1 << 24) - 1


def test_u24_uniformity_chi_square():
    # Each of the three used words, over consecutive positions, is uniform.
    n = 1 << 16
    for word in range(3):
        bins = np.zeros(256, np.int64)
        for p in range(n):
            bins[oracle.u24(oracle.uniform_words(1003, p, 0, 0)[word]) >> 16] += 1
        chi2, pval = stats.chisquare(bins)
        assert pval > 1e-4, (word, chi2, pval)
