"""Pins of the oracle's RNN head (Eq. 6 of the DSpark technical review,
"Instantiation 2: The RNN Head"): its bf16 rounding against library
conversions, the reductions to the Markov head and to independent
per-position softmaxes, the zero initial state, the memory beyond one step
that the Markov head lacks, and the block law by enumeration and Monte
Carlo."""

import itertools

import numpy as np
import torch
from scipy.stats import chisquare

from oracle import dspark_ref as ref


def _case(V=7, gamma=3, r=4, d=5, B=3, seed=0):
    rng = np.random.default_rng(seed)
    U = rng.normal(0, 1.0, size=(B, gamma, V)).astype(np.float32)
    W1 = rng.normal(0, 1.0, size=(V, r))
    W2 = rng.normal(0, 1.0, size=(r, V))
    Wp = rng.normal(0, 0.6, size=(3 * r, 2 * r + d))
    h = rng.normal(0, 1.0, size=(B, gamma, d)).astype(np.float32)
    x0 = rng.integers(0, V, size=B).astype(np.int32)
    seeds = np.arange(B, dtype=np.uint64) + np.uint64(3)
    return U, W1, W2, Wp, h, x0, seeds


def test_bf16_rounding_matches_library_conversions():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 1, size=4000).astype(np.float32)      # float32 values: one rounding either way
    ours = ref.round_to_bf16(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert (ours == theirs).all()
    # ties go to the even neighbour
    assert ref.round_to_bf16([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]).tolist() == [1.0, 1 + 2.0 ** -6, -1.0]


def test_zero_output_block_is_the_parallel_drafter():
    U, W1, W2, Wp, h, x0, seeds = _case()
    r = W1.shape[1]
    Wp0 = Wp.copy()
    Wp0[2 * r:] = 0.0
    d_rnn = ref.rnn_draft(U, W1, W2, Wp0, h, x0, 1.0, seeds, 5)
    d_par = ref.markov_draft(U, np.zeros_like(W1), W2, x0, 1.0, seeds, 5)
    assert (d_rnn["tokens"] == d_par["tokens"]).all()
    np.testing.assert_allclose(d_rnn["prob"], d_par["prob"], rtol=1e-13, atol=0)
    assert (d_rnn["E"] == 0).all()


def test_output_reading_only_the_embedding_is_a_markov_head():
    U, W1, W2, Wp, h, x0, seeds = _case(seed=2)
    r = W1.shape[1]
    Wp1 = Wp.copy()
    Wp1[2 * r:, :r] = 0.0          # output block: no state
    Wp1[2 * r:, 2 * r:] = 0.0      # ... and no hidden state
    emb = np.tanh(W1 @ Wp1[2 * r:, r:2 * r].T)
    for rounded in (False, True):
        W1_eff = ref.round_to_bf16(emb) if rounded else emb
        for T in (1.0, 0.7, 0.0):
            d_rnn = ref.rnn_draft(U, W1, W2, Wp1, h, x0, T, seeds, 6, bf16_operand=rounded)
            d_mk = ref.markov_draft(U, W1_eff, W2, x0, T, seeds, 6)
            assert (d_rnn["tokens"] == d_mk["tokens"]).all()
            np.testing.assert_allclose(d_rnn["prob"], d_mk["prob"], rtol=1e-12, atol=0)


def test_zero_initial_state_and_memory_beyond_one_step():
    U, W1, W2, Wp, h, x0, seeds = _case(V=6, gamma=4, seed=3)
    r = W1.shape[1]
    Wp2 = Wp.copy()
    Wp2[2 * r:, r:] = 0.0          # output block reads the state only
    forced = np.array([[1, 2, 3, 4]] * 3, dtype=np.int32)
    d = ref.rnn_draft(U, W1, W2, Wp2, h, x0, 1.0, seeds, 7, forced=forced)
    assert (d["E"][:, 0] == 0).all()                    # s_0 = 0: position 1 has no bias
    alt = forced.copy()
    alt[:, 0] = 5                                       # change x_1 only
    d2 = ref.rnn_draft(U, W1, W2, Wp2, h, x0, 1.0, seeds, 7, forced=alt)
    # s_1 summarises x_0 only, so position 2 does not see x_1; s_2 takes in
    # x_1, so positions 3 and 4 do, although a Markov head at position 3
    # would see x_2 alone (unchanged here)
    assert (d2["E"][:, :2] == d["E"][:, :2]).all()
    assert (d2["E"][:, 2] != d["E"][:, 2]).any()
    assert (d2["E"][:, 3] != d["E"][:, 3]).any()


def test_block_law_sums_to_one_and_matches_sampling():
    V, gamma = 3, 3
    U, W1, W2, Wp, h, x0, _ = _case(V=V, gamma=gamma, r=2, d=3, B=1, seed=4)
    law = {}
    for blk in itertools.product(range(V), repeat=gamma):
        d = ref.rnn_draft(U, W1, W2, Wp, h, x0, 1.0, np.zeros(1, dtype=np.uint64), 0,
                          forced=np.array([blk], dtype=np.int32))
        law[blk] = float(np.prod(d["prob"][0]))
    assert abs(sum(law.values()) - 1.0) < 1e-12
    n = 3000
    Ur, hr = np.repeat(U, n, axis=0), np.repeat(h, n, axis=0)
    x0r = np.repeat(x0, n)
    seeds = np.arange(n, dtype=np.uint64) * np.uint64(7919) + np.uint64(1)
    d = ref.rnn_draft(Ur, W1, W2, Wp, hr, x0r, 1.0, seeds, 9)
    counts = {blk: 0 for blk in law}
    for row in d["tokens"]:
        counts[tuple(int(t) for t in row)] += 1
    keys = sorted(law)
    assert chisquare([counts[k] for k in keys], [law[k] * n for k in keys]).pvalue > 1e-4


def test_precomputed_hidden_part_is_the_same_draft():
    U, W1, W2, Wp, h, x0, seeds = _case(seed=9)
    r = W1.shape[1]
    hp = np.einsum("bkd,jd->bkj", h.astype(np.float64), Wp[:, 2 * r:])
    a = ref.rnn_draft(U, W1, W2, Wp, h, x0, 1.0, seeds, 4)
    b = ref.rnn_draft(U, W1, W2, Wp[:, :2 * r], None, x0, 1.0, seeds, 4, hp=hp)
    assert (a["tokens"] == b["tokens"]).all()
    np.testing.assert_allclose(a["prob"], b["prob"], rtol=1e-12, atol=0)
