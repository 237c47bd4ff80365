"""Pins of the oracle's Philox4x64-10 against the published known-answer
vectors and against numpy's independent Philox implementation."""

import random

import numpy as np

from conftest import golden_path
from oracle import philox


def _load_kat():
    rows = []
    for line in open(golden_path("philox4x64_10_kat.txt")):
        if line.startswith("#") or not line.strip():
            continue
        w = [int(x, 16) for x in line.split()]
        rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_known_answer_vectors():
    rows = _load_kat()
    assert len(rows) == 3
    for ctr, key, want in rows:
        assert list(philox.philox4x64(ctr, key)) == want


def _numpy_block(ctr, key):
    # numpy's Philox increments its 256-bit counter before producing a block
    c = (ctr[0] | ctr[1] << 64 | ctr[2] << 128 | ctr[3] << 192) - 1
    c %= 1 << 256
    words = np.array([(c >> (64 * i)) & philox.MASK64 for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(counter=words, key=np.array(key, dtype=np.uint64))
    return [int(x) for x in g.random_raw(4)]


def test_agrees_with_numpy_philox():
    rng = random.Random(7)
    for i in range(300):
        ctr = [rng.getrandbits(64) for _ in range(4)]
        if i % 4 == 0:
            ctr[0] = 0  # borrow path of the numpy counter offset
        key = [rng.getrandbits(64) for _ in range(2)]
        assert list(philox.philox4x64(ctr, key)) == _numpy_block(ctr, key)


def test_stream_layout_counters():
    # block(seed, rnd, k, stream, index) is Philox at counter (rnd, k, stream, index), key (seed, 0)
    seed, rnd, k, stream, idx = 123456789, 1000, 3, 2, 5
    assert list(philox.block(seed, rnd, k, stream, idx)) == _numpy_block([rnd, k, stream, idx], [seed, 0])


def test_uniform_map_is_open_interval_and_exact():
    from fractions import Fraction
    assert philox.to_uniform(0) == 2.0 ** -53
    top = philox.to_uniform(philox.MASK64)
    assert top < 1.0 and Fraction(top) == 1 - Fraction(1, 2 ** 53)
    # every word maps to exactly ((w >> 12) + 1/2) / 2**52, no rounding
    for w in (0x123456789ABCDEF0, philox.MASK64 - 4095, 1 << 63, (1 << 63) - 1):
        assert Fraction(philox.to_uniform(w)) == (Fraction(w >> 12) + Fraction(1, 2)) / 2 ** 52
    # low 12 bits are ignored
    w = 0x123456789ABCDEF0
    assert philox.to_uniform(w | 0xFFF) == philox.to_uniform(w & ~0xFFF)


def test_uniforms_look_uniform():
    us = np.array([philox.uniform(42, r, 1, 0) for r in range(20000)])
    assert 0.0 < us.min() and us.max() < 1.0
    counts, _ = np.histogram(us, bins=20, range=(0, 1))
    from scipy.stats import chisquare
    assert chisquare(counts).pvalue > 1e-4
