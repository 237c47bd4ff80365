"""Pins of the oracle's prefix-survival products: the printed worked traces of
the DSpark technical review's scheduler section, bounds and monotonicity,
and the closed form P(n >= k) = prod c*_i in the position-only case."""

import numpy as np
import pytest

from conftest import golden_path
from oracle import dspark_ref as ref


def _printed_rows():
    rows = []
    for line in open(golden_path("survival_worked_examples.txt")):
        if line.startswith("#") or not line.strip():
            continue
        left, right = line.split("|")
        f = left.split()
        rows.append((f[0], [float(x) for x in f[1:]], [float(x) for x in right.split()]))
    return rows


def test_printed_survival_products():
    rows = _printed_rows()
    assert len(rows) == 5
    for mode, conf, printed in rows:
        c_star, a = ref.survival(None, None, None, None, None, None, 1.0, conf=np.array([conf]))
        assert c_star is None
        if mode == "exact":
            np.testing.assert_allclose(a[0], printed, rtol=0, atol=1e-15)
        else:
            # printed to `mode` decimals: within half a unit of the last digit
            half = 0.5 * 10.0 ** -int(mode)
            assert np.all(np.abs(a[0] - np.array(printed)) <= half + 1e-12)


def test_survival_is_non_increasing_and_bounded():
    rng = np.random.default_rng(0)
    conf = rng.random((50, 7))
    _, a = ref.survival(None, None, None, None, None, None, 1.0, conf=conf)
    assert (np.diff(a, axis=1) <= 0).all()
    assert (a >= 0).all() and (a <= 1).all()


def _position_only_round(V, gamma, B, seed):
    rng = np.random.default_rng(seed)
    U = np.repeat(rng.normal(0, 1.2, size=(1, gamma, V)).astype(np.float32), B, axis=0)
    tgt = np.repeat(rng.normal(0, 1.2, size=(1, gamma + 1, V)).astype(np.float32), B, axis=0)
    W1 = np.zeros((V, 3))
    W2 = rng.normal(0, 1.0, size=(3, V))
    x0 = np.zeros(B, dtype=np.int32)
    return U, W1, W2, x0, tgt


def test_analytical_survival_is_position_acceptance_product():
    V, gamma, B = 7, 3, 4
    U, W1, W2, x0, tgt = _position_only_round(V, gamma, B, seed=1)
    seeds = np.arange(B, dtype=np.uint64) + np.uint64(5)
    d = ref.markov_draft(U, W1, W2, x0, 0.9, seeds, rnd=4)
    c, a = ref.survival(U, W1, W2, x0, d["tokens"], tgt, 0.9)
    # with W1 = 0 every c*_k is 1 - TV(softmax(U_k/T), softmax(tgt_k/T))
    for k in range(gamma):
        pd = np.exp(U[0, k] / 0.9 - np.logaddexp.reduce(U[0, k] / 0.9))
        pt = np.exp(tgt[0, k] / 0.9 - np.logaddexp.reduce(tgt[0, k] / 0.9))
        assert abs(c[0, k] - (1 - 0.5 * np.abs(pd - pt).sum())) < 1e-6
    assert (np.diff(a, axis=1) <= 1e-15).all()
    np.testing.assert_allclose(a, np.cumprod(c, axis=1), rtol=1e-15)


@pytest.mark.slow
def test_survival_is_prefix_acceptance_probability_in_position_only_case():
    # W1 = 0 and targets that ignore the prefix: P(n >= k) = prod_{i<=k} c*_i and
    # the expected emitted length is 1 + sum_k a_k (the scheduler's tau per request)
    V, gamma, B, R = 6, 3, 100, 60
    U, W1, W2, x0, tgt = _position_only_round(V, gamma, B, seed=2)
    T = 1.0
    ge = np.zeros(gamma)
    total_len = 0
    for rnd in range(R):
        seeds = np.arange(B, dtype=np.uint64) * np.uint64(31) + np.uint64(rnd * 1000 + 1)
        d = ref.markov_draft(U, W1, W2, x0, T, seeds, rnd)
        v = ref.verify(U, W1, W2, x0, d["tokens"], tgt, T, seeds, rnd)
        for k in range(gamma):
            ge[k] += (v["accept_len"] >= k + 1).sum()
        total_len += int((v["accept_len"] + 1).sum())
    c, a = ref.survival(U, W1, W2, x0, d["tokens"], tgt, T)
    N = B * R
    for k in range(gamma):
        p = a[0, k]
        assert abs(ge[k] / N - p) < 5 * np.sqrt(p * (1 - p) / N) + 1e-12
    expected_len = 1 + a[0].sum()
    assert abs(total_len / N - expected_len) < 0.05


def test_greedy_survival_is_argmax_agreement_indicator():
    V, gamma, B = 5, 3, 1
    U = np.zeros((B, gamma, V), dtype=np.float32)
    W1, W2 = np.zeros((V, 2)), np.zeros((2, V))
    tgt = np.zeros((B, gamma + 1, V), dtype=np.float32)
    draft = np.array([[1, 2, 3]], dtype=np.int32)
    tgt[0, 0, 1] = 1.0
    tgt[0, 1, 4] = 1.0
    tgt[0, 2, 3] = 1.0
    c, a = ref.survival(U, W1, W2, np.zeros(B, np.int32), draft, tgt, 0.0)
    assert c[0].tolist() == [1.0, 0.0, 1.0]
    assert a[0].tolist() == [1.0, 0.0, 0.0]
