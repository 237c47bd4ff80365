"""Pins of the oracle's draft sampler (Eq. 4 / Eq. 5 of the DSpark technical
review): softmax against scipy, the inverse CDF against closed forms, the bias
indexing against the bigram special case, and the block law against
brute-force enumeration."""

import itertools

import numpy as np
import pytest
from scipy.special import logsumexp
from scipy.special import softmax as sp_softmax
from scipy.stats import chisquare

from oracle import dspark_ref as ref
from oracle import philox


def test_softmax_matches_scipy():
    rng = np.random.default_rng(0)
    for _ in range(20):
        l = rng.normal(0, 5, size=257)
        l[rng.integers(0, 257, 3)] = -np.inf
        p, z = ref.softmax(l)
        np.testing.assert_allclose(p, sp_softmax(l), rtol=1e-13, atol=0)
        assert abs(z - logsumexp(l)) < 1e-12
        assert abs(p.sum() - 1.0) < 1e-12


def test_inverse_cdf_two_outcomes_closed_form():
    # V = 2: x = 0 exactly when u < p0
    for p0 in (0.1, 0.5, 0.73):
        p = np.array([p0, 1 - p0])
        for u in np.linspace(0.001, 0.999, 101):
            x, d = ref.inverse_cdf(p, u)
            assert x == (0 if u < p0 else 1)
            assert abs(d - (min(u, p0 - u) if u < p0 else min(u - p0, 1 - u))) < 1e-15


def test_inverse_cdf_hand_values_and_zero_tail():
    p = np.array([0.25, 0.0, 0.5, 0.25, 0.0])
    assert ref.inverse_cdf(p, 0.1)[0] == 0
    assert ref.inverse_cdf(p, 0.25)[0] == 2      # strict '>' skips the zero-mass id 1
    assert ref.inverse_cdf(p, 0.74)[0] == 2
    assert ref.inverse_cdf(p, 0.75)[0] == 3
    # rounding leaves the total below u: the last id with positive mass
    q = np.array([0.5, 0.5 - 1e-12, 0.0])
    assert ref.inverse_cdf(q, 1.0 - 1e-13)[0] == 1


def _tiny(V, gamma, r, B, w_std, seed=0):
    rng = np.random.default_rng(seed)
    U = rng.normal(0, 1.5, size=(B, gamma, V)).astype(np.float32)
    W1 = rng.normal(0, w_std, size=(V, r))
    W2 = rng.normal(0, w_std, size=(r, V))
    x0 = rng.integers(0, V, size=B).astype(np.int32)
    seeds = np.arange(1, B + 1, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)
    return U, W1, W2, x0, seeds


def test_zero_bias_is_independent_softmax():
    # W1 = 0: every position is its own softmax of U_k / T (the parallel-drafter case)
    U, W1, W2, x0, seeds = _tiny(V=50, gamma=4, r=8, B=6, w_std=1.0)
    W1[:] = 0
    for T in (1.0, 0.6):
        out = ref.markov_draft(U, W1, W2, x0, T, seeds, rnd=5)
        for b in range(6):
            for k in range(4):
                p = sp_softmax(U[b, k].astype(np.float64) / T)
                x = out["tokens"][b, k]
                assert abs(out["prob"][b, k] - p[x]) < 1e-14
                assert abs(out["lse"][b, k] - logsumexp(U[b, k].astype(np.float64) / T)) < 1e-12


def test_identity_embedding_is_bigram_table_row_of_previous_token():
    # r = V and W1 = I: the bias of position k is row x_{k-1} of W2 (x_0 = anchor)
    V, gamma, B = 12, 4, 5
    U, _, _, x0, seeds = _tiny(V=V, gamma=gamma, r=V, B=B, w_std=1.0, seed=3)
    W1 = np.eye(V)
    W2 = np.random.default_rng(9).normal(0, 2.0, size=(V, V))   # not symmetric
    out = ref.markov_draft(U, W1, W2, x0, 1.0, seeds, rnd=2)
    for b in range(B):
        prev = x0[b]
        for k in range(gamma):
            p = sp_softmax(U[b, k].astype(np.float64) + W2[prev])
            x = out["tokens"][b, k]
            assert abs(out["prob"][b, k] - p[x]) < 1e-14
            prev = x


def test_temperature_divides_the_summed_logits():
    # (U + W1[x] W2) / T is unchanged when U and W1 are doubled and T is doubled
    U, W1, W2, x0, seeds = _tiny(V=40, gamma=3, r=4, B=4, w_std=1.0, seed=4)
    a = ref.markov_draft(U, W1, W2, x0, 1.0, seeds, rnd=11)
    b = ref.markov_draft(2 * U, 2 * W1, W2, x0, 2.0, seeds, rnd=11)
    assert (a["tokens"] == b["tokens"]).all()
    np.testing.assert_allclose(a["prob"], b["prob"], rtol=1e-12)


def test_position_k_uses_stream_zero_uniform_of_its_counter():
    # V = 2, zero bias: x_k = 0 iff the (rnd, k, stream 0) uniform is below p_0
    V, gamma, B = 2, 5, 3
    U = np.zeros((B, gamma, V), dtype=np.float32)
    U[:, :, 0] = 0.3
    W1, W2 = np.zeros((V, 4)), np.zeros((4, V))
    x0 = np.zeros(B, dtype=np.int32)
    seeds = np.array([11, 22, 33], dtype=np.uint64)
    p0 = float(sp_softmax(np.array([0.3, 0.0]))[0])
    out = ref.markov_draft(U, W1, W2, x0, 1.0, seeds, rnd=77)
    for b in range(B):
        for k in range(1, gamma + 1):
            u = philox.uniform(int(seeds[b]), 77, k, philox.STREAM_DRAFT)
            assert out["tokens"][b, k - 1] == (0 if u < p0 else 1)


def test_request_subset_matches_full_run():
    U, W1, W2, x0, seeds = _tiny(V=30, gamma=3, r=4, B=5, w_std=0.5, seed=8)
    full = ref.markov_draft(U, W1, W2, x0, 0.9, seeds, rnd=3)
    part = ref.markov_draft(U, W1, W2, x0, 0.9, seeds, rnd=3, requests=[1, 4])
    for b in (1, 4):
        assert (part["tokens"][b] == full["tokens"][b]).all()
    assert (part["tokens"][0] == -1).all()


def test_greedy_is_first_argmax_with_probability_one():
    V, gamma, B = 9, 3, 2
    U = np.zeros((B, gamma, V), dtype=np.float32)
    U[0, 0, [2, 5]] = 4.0          # tie: lowest index wins
    U[0, 1, 7] = 1.0
    U[0, 2, [0, 8]] = 2.0
    U[1] = np.arange(V)[None, :]
    W1, W2 = np.zeros((V, 4)), np.zeros((4, V))
    out = ref.markov_draft(U, W1, W2, np.zeros(B, dtype=np.int32), 0.0, np.zeros(B, np.uint64), rnd=0)
    assert out["tokens"][0].tolist() == [2, 7, 0]
    assert out["tokens"][1].tolist() == [8, 8, 8]
    assert (out["prob"] == 1.0).all()


@pytest.mark.slow
def test_block_law_matches_brute_force_enumeration():
    # chi-square of drafted blocks against P(X | x0) = prod_k p_k(x_k | x0, x_<k) (Eq. 4)
    V, gamma, r = 5, 3, 3
    rng = np.random.default_rng(21)
    U = rng.normal(0, 1.0, size=(1, gamma, V)).astype(np.float32)
    W1 = rng.normal(0, 1.0, size=(V, r))
    W2 = rng.normal(0, 1.0, size=(r, V))
    x0 = np.array([2], dtype=np.int32)
    T = 0.8

    law = {}
    for blk in itertools.product(range(V), repeat=gamma):
        prob, prev = 1.0, 2
        for k, x in enumerate(blk):
            prob *= sp_softmax((U[0, k].astype(np.float64) + W1[prev] @ W2) / T)[x]
            prev = x
        law[blk] = prob
    assert abs(sum(law.values()) - 1.0) < 1e-12

    n = 20000
    counts = dict.fromkeys(law, 0)
    seeds = np.array([0xABCDEF], dtype=np.uint64)
    for rnd in range(n):
        t = ref.markov_draft(U, W1, W2, x0, T, seeds, rnd=rnd)["tokens"][0]
        counts[tuple(int(v) for v in t)] += 1
    keys = list(law)
    f_obs = np.array([counts[k] for k in keys], dtype=float)
    f_exp = np.array([law[k] for k in keys]) * n
    # merge sparse cells so every expected count is at least 5
    order = np.argsort(f_exp)
    obs_m, exp_m, acc_o, acc_e = [], [], 0.0, 0.0
    for i in order:
        acc_o += f_obs[i]
        acc_e += f_exp[i]
        if acc_e >= 5:
            obs_m.append(acc_o)
            exp_m.append(acc_e)
            acc_o = acc_e = 0.0
    exp_m[-1] += acc_e
    obs_m[-1] += acc_o
    assert chisquare(obs_m, exp_m).pvalue > 1e-4
