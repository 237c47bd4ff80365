"""Pins of the oracle's verifier: the printed acceptance example (Eq. 8a-8c of
the DSpark technical review), the residual law norm(max(0, p_t - p_d)), the
bonus draw, the greedy limit, and losslessness of the whole round as a
chi-square test on a tiny vocabulary."""

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax
from scipy.stats import chisquare

from conftest import golden_path
from oracle import dspark_ref as ref
from oracle import philox


def _worked_example():
    for line in open(golden_path("acceptance_worked_example.txt")):
        if line.startswith("#") or not line.strip():
            continue
        f = [[float(x) for x in part.split()] for part in line.split("|")]
        return np.array(f[0]), np.array(f[1]), f[2][0], f[3][0], f[4][0]


def test_printed_acceptance_identity_example():
    pt, pd, sum_min, l1, one_minus_half_l1 = _worked_example()
    assert abs(ref.acceptance_rate(pd, pt) - sum_min) < 1e-15
    assert abs(np.abs(pd - pt).sum() - l1) < 1e-15
    assert abs(ref.acceptance_rate(pd, pt) - one_minus_half_l1) < 1e-15


def test_acceptance_rate_equals_one_minus_total_variation():
    rng = np.random.default_rng(1)
    for _ in range(200):
        V = int(rng.integers(2, 40))
        pd = rng.dirichlet(np.full(V, 0.5))
        pt = rng.dirichlet(np.full(V, 0.5))
        assert abs(ref.acceptance_rate(pd, pt) - (1 - 0.5 * np.abs(pd - pt).sum())) < 1e-14
    p = rng.dirichlet(np.ones(7))
    assert ref.acceptance_rate(p, p) == 1.0
    a = np.array([0.5, 0.5, 0.0, 0.0])
    b = np.array([0.0, 0.0, 0.3, 0.7])
    assert ref.acceptance_rate(a, b) == 0.0


def _two_token_round(pt, pd, gamma=1, B=1):
    """A round whose draft law is pd and whose target law is pt at every position."""
    V = len(pt)
    U = np.tile(np.log(pd).astype(np.float32), (B, gamma, 1))
    tgt = np.tile(np.log(pt).astype(np.float32), (B, gamma + 1, 1))
    W1, W2 = np.zeros((V, 2)), np.zeros((2, V))
    return U, W1, W2, tgt


@pytest.mark.slow
def test_printed_example_round_law_and_residual_support():
    # p_t = (0.7, 0.3), p_d = (0.5, 0.5): acceptance 0.8, emitted law (0.7, 0.3),
    # and every correction is A because the residual lives where p_t > p_d.
    pt, pd = np.array([0.7, 0.3]), np.array([0.5, 0.5])
    B, R = 100, 60
    U, W1, W2, tgt = _two_token_round(pt, pd, gamma=1, B=B)
    x0 = np.zeros(B, dtype=np.int32)
    seeds = np.arange(B, dtype=np.uint64) + np.uint64(1000)
    acc = first_A = rejected = 0
    for rnd in range(R):
        d = ref.markov_draft(U, W1, W2, x0, 1.0, seeds, rnd)
        v = ref.verify(U, W1, W2, x0, d["tokens"], tgt, 1.0, seeds, rnd, max_proposals=4)
        for b in range(B):
            n = v["accept_len"][b]
            acc += n
            first_A += v["out_tokens"][b, 0] == 0
            if n == 0:
                rejected += 1
                assert v["out_tokens"][b, 0] == 0
    N = B * R
    s_acc = np.sqrt(0.8 * 0.2 / N)
    assert abs(acc / N - 0.8) < 5 * s_acc
    s_a = np.sqrt(0.7 * 0.3 / N)
    assert abs(first_A / N - 0.7) < 5 * s_a
    # resampling the correction from p_t instead would give 0.5 + 0.5*0.4*0.7 = 0.64
    assert abs(first_A / N - 0.64) > 5 * s_a
    assert rejected > 0


def test_residual_inverse_cdf_when_no_proposals():
    rng = np.random.default_rng(2)
    pt = rng.dirichlet(np.ones(6))
    pd = rng.dirichlet(np.ones(6))
    res = np.maximum(0, pt - pd)
    for rnd in range(50):
        y = ref.residual_sample(pt, pd, 5, rnd, 2, 0, [])
        u = philox.uniform(5, rnd, 2, philox.STREAM_FALLBACK)
        assert y == ref.inverse_cdf(res / res.sum(), u)[0]


@pytest.mark.slow
@pytest.mark.parametrize("max_prop", [0, 1, 16, 64])
def test_residual_law(max_prop):
    rng = np.random.default_rng(3)
    pt = rng.dirichlet(np.ones(6))
    pd = rng.dirichlet(np.ones(6))
    law = ref.residual_law(pt, pd)
    n = 12000
    counts = np.zeros(6)
    for rnd in range(n):
        counts[ref.residual_sample(pt, pd, 99, rnd, 1, max_prop, [])] += 1
    assert counts[law == 0].sum() == 0
    keep = law > 0
    assert chisquare(counts[keep], law[keep] * n).pvalue > 1e-4


@pytest.mark.slow
def test_first_position_acceptance_probability_is_sum_of_minima():
    rng = np.random.default_rng(4)
    V = 6
    pd = rng.dirichlet(np.ones(V))
    pt = rng.dirichlet(np.ones(V))
    B, R = 100, 50
    U, W1, W2, tgt = _two_token_round(pt, pd, gamma=2, B=B)
    x0 = np.zeros(B, dtype=np.int32)
    seeds = np.arange(B, dtype=np.uint64) * np.uint64(7919) + np.uint64(3)
    acc = 0
    for rnd in range(R):
        d = ref.markov_draft(U, W1, W2, x0, 1.0, seeds, rnd)
        v = ref.verify(U, W1, W2, x0, d["tokens"], tgt, 1.0, seeds, rnd)
        acc += int((v["accept_len"] >= 1).sum())
    N = B * R
    a = np.minimum(pd, pt).sum()
    assert abs(acc / N - a) < 5 * np.sqrt(a * (1 - a) / N)


def test_bonus_uses_stream_two_at_position_gamma_plus_one():
    # identical laws: every draft is accepted; the bonus is the inverse CDF of
    # target row gamma+1 with the (rnd, gamma+1, 2, 0) uniform
    gamma, B = 3, 4
    p = np.array([0.35, 0.65])
    U, W1, W2, tgt = _two_token_round(p, p, gamma=gamma, B=B)
    tgt[:, gamma, :] = np.log(np.array([0.6, 0.4]))
    x0 = np.zeros(B, dtype=np.int32)
    seeds = np.array([5, 6, 7, 8], dtype=np.uint64)
    for rnd in range(20):
        d = ref.markov_draft(U, W1, W2, x0, 1.0, seeds, rnd)
        v = ref.verify(U, W1, W2, x0, d["tokens"], tgt, 1.0, seeds, rnd)
        for b in range(B):
            assert v["accept_len"][b] == gamma
            u = philox.uniform(int(seeds[b]), rnd, gamma + 1, philox.STREAM_RESIDUAL)
            assert v["out_tokens"][b, gamma] == (0 if u < 0.6 else 1)
            assert (v["out_tokens"][b, :gamma] == d["tokens"][b]).all()
            np.testing.assert_allclose(v["accept_prob"][b], 1.0, rtol=1e-12)


def test_greedy_exact_match_correction_and_bonus():
    V, gamma, B = 6, 3, 3
    U = np.zeros((B, gamma, V), dtype=np.float32)
    W1, W2 = np.zeros((V, 2)), np.zeros((2, V))
    tgt = np.zeros((B, gamma + 1, V), dtype=np.float32)
    draft = np.array([[1, 2, 3], [1, 2, 3], [4, 4, 4]], dtype=np.int32)
    tgt[0, 0, 1] = tgt[0, 1, 2] = tgt[0, 2, 3] = 1.0   # all match
    tgt[0, 3, 5] = 1.0                                  # bonus 5
    tgt[1, 0, 1] = tgt[1, 1, 0] = 1.0                   # mismatch at k=2: correction 0
    tgt[2, 0, [2, 3]] = 1.0                             # tie: argmax 2, mismatch at k=1
    v = ref.verify(U, W1, W2, np.zeros(B, np.int32), draft, tgt, 0.0, np.zeros(B, np.uint64), 0)
    assert v["accept_len"].tolist() == [3, 1, 0]
    assert v["out_tokens"].tolist() == [[1, 2, 3, 5], [1, 0, -1, -1], [2, -1, -1, -1]]
    assert v["accept_prob"][0].tolist() == [1.0, 1.0, 1.0]
    assert v["accept_prob"][1, :2].tolist() == [1.0, 0.0] and np.isnan(v["accept_prob"][1, 2])
    assert v["accept_prob"][2, 0] == 0.0 and np.isnan(v["accept_prob"][2, 1:]).all()


def _losslessness_counts(T, V=4, gamma=3, r=2, B=150, R=80, seed=5):
    """Draft with a Markov head, let a 'target' table G[k][prev] play the target
    model on the drafted prefix, verify, and count emitted tokens."""
    rng = np.random.default_rng(seed)
    U = rng.normal(0, 1.0, size=(1, gamma, V)).astype(np.float32)
    U = np.repeat(U, B, axis=0)
    W1 = rng.normal(0, 1.0, size=(V, r))
    W2 = rng.normal(0, 1.0, size=(r, V))
    G = rng.normal(0, 1.2, size=(gamma + 1, V, V)).astype(np.float32)  # G[k][prev] -> target logits
    anchor = 1
    x0 = np.full(B, anchor, dtype=np.int32)
    first = np.zeros(V)
    second = np.zeros((V, V))
    for rnd in range(R):
        seeds = (np.arange(B, dtype=np.uint64) + np.uint64(rnd * B)) * np.uint64(2654435761) + np.uint64(17)
        d = ref.markov_draft(U, W1, W2, x0, T, seeds, rnd)
        tgt = np.empty((B, gamma + 1, V), dtype=np.float32)
        for b in range(B):
            prev = anchor
            for k in range(gamma + 1):
                tgt[b, k] = G[k, prev]
                if k < gamma:
                    prev = d["tokens"][b, k]
        v = ref.verify(U, W1, W2, x0, d["tokens"], tgt, T, seeds, rnd)
        for b in range(B):
            y = v["out_tokens"][b]
            first[y[0]] += 1
            if v["accept_len"][b] >= 1:
                second[y[0], y[1]] += 1
    return G, anchor, first, second


@pytest.mark.slow
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_round_is_lossless_on_a_tiny_vocabulary(T):
    G, anchor, first, second = _losslessness_counts(T)
    law1 = sp_softmax(G[0, anchor].astype(np.float64) / T)
    assert chisquare(first, law1 * first.sum()).pvalue > 1e-4
    tested = 0
    for a in range(len(law1)):
        n = second[a].sum()
        if n < 200:
            continue
        law2 = sp_softmax(G[1, a].astype(np.float64) / T)
        assert chisquare(second[a], law2 * n).pvalue > 1e-4
        tested += 1
    assert tested >= 2
