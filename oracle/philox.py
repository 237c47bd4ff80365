"""Philox4x64-10, the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), written out from the
published round function in plain Python integers.

TEST INFRASTRUCTURE. Part of the float64 oracle: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The HIP library carries its own implementation of the same
published generator and shares no code with this file.

The pages of the method never name a random-number generator; the stream
layout below is this implementation's reading:

* key     = (seed_b, 0)                         one key per request
* counter = (round, position k, stream, index)  one block of four words
* streams: 0 draft sample, 1 acceptance test, 2 residual proposal / bonus,
  3 exact residual fallback
* a uniform in (0, 1) is ((w >> 12) + 0.5) * 2**-52: 52 integer bits plus a
  half need 53 significant bits, so the value is exact in float64 and lies in
  [2**-53, 1 - 2**-53].
"""

MASK64 = (1 << 64) - 1

# Round multipliers and Weyl key increments of Philox4x64 (SC'11, Sec. 5).
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B

STREAM_DRAFT = 0
STREAM_ACCEPT = 1
STREAM_RESIDUAL = 2
STREAM_FALLBACK = 3


def _mulhilo(a, b):
    p = a * b
    return p >> 64, p & MASK64


def philox4x64(counter, key, rounds=10):
    """Apply ``rounds`` Philox4x64 rounds to a 4-word counter under a 2-word key.

    Each round multiplies words 0 and 2 by the two round constants, swaps the
    high halves across and xors in the other words and the key; the key is
    bumped by the Weyl constants between rounds.
    """
    c0, c1, c2, c3 = (int(w) & MASK64 for w in counter)
    k0, k1 = (int(w) & MASK64 for w in key)
    for rnd in range(rounds):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        hi0, lo0 = _mulhilo(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo(PHILOX_M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return (c0, c1, c2, c3)


def to_uniform(word):
    """Map a 64-bit word to the float64 uniform ((w >> 12) + 0.5) / 2**52 in (0, 1)."""
    return ((int(word) >> 12) + 0.5) * (2.0 ** -52)


def block(seed, rnd, k, stream, index=0):
    """The four output words for request key ``seed`` at counter (rnd, k, stream, index)."""
    return philox4x64((rnd, k, stream, index), (seed, 0))


def uniform(seed, rnd, k, stream, index=0, word=0):
    """One uniform of the stream layout described in the module docstring."""
    return to_uniform(block(seed, rnd, k, stream, index)[word])
