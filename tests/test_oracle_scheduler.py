"""Pins of the oracle's hardware-aware prefix scheduler (Algorithm 1 of the
DSpark technical review, "The Hardware-Aware Prefix Scheduler") and of
verification with scheduled lengths: the printed worked traces, Lemmas 1-2
against brute force over every length assignment, and the non-anticipation
counterexample of Eq. 9-10 as a law test through draft, scheduler and
verifier; and the asynchronous adaptation (capacity from an unconstrained
search on earlier survivals, admission of the current top-K), pinned by the
same printed curves, a jagged curve, brute force and a law test."""

import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax
from scipy.stats import chisquare

from conftest import golden_path
from oracle import dspark_ref as ref


def _examples():
    ex, cur = {}, None
    for line in open(golden_path("scheduler_worked_examples.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = ex.setdefault(line.strip("[]"), {"conf": []})
            continue
        key, _, rest = line.partition(" ")
        f = rest.split()
        if key == "conf":
            cur["conf"].append([float(x) for x in f])
        elif key == "sps":
            pairs = [x.split(":") for x in f]
            sps = np.full(max(int(n) for n, _ in pairs) + 1, np.nan)
            for n, v in pairs:
                sps[int(n)] = float(v)
            cur["sps"] = sps
        elif key == "order":
            cur["order"] = [tuple(int(y) for y in x.split(",")) for x in f]
        elif key == "lengths":
            cur["lengths"] = [int(x) for x in f]
        elif key == "best":
            cur["best"] = (float(f[0]), f[0])
        elif key == "trace":
            rows = []
            for x in f:
                rj, B, tau, theta = x.split(":")
                rows.append((tuple(int(y) for y in rj.split(",")), int(B), (float(tau), tau), (float(theta), theta)))
            cur["trace"] = rows
    return ex


def _unit(printed):
    """One unit of the last printed digit."""
    return 10.0 ** -(len(printed.split(".")[1]) if "." in printed else 0)


def _close(value, printed):
    return abs(value - printed[0]) <= _unit(printed[1]) + 1e-12


@pytest.mark.parametrize("name", ["two", "three", "eq9"])
def test_printed_worked_examples(name):
    e = _examples()[name]
    a = np.cumprod(np.array(e["conf"]), axis=1)
    lengths, best, _ = ref.schedule(a, e["sps"])
    assert lengths.tolist() == e["lengths"]
    assert _close(best, e["best"])
    # the full scan (no early stop) reproduces every printed row, in order
    trace = []
    ref.schedule(a, e["sps"], early_stop=False, trace=trace)
    if "order" in e:
        assert [(r, j) for r, j, _, _, _ in trace] == e["order"]
    for (rj, B, tau, theta), got in zip(e["trace"], trace):
        assert (got[0], got[1]) == rj and got[2] == B
        assert _close(got[3], tau) and _close(got[4], theta)


def test_early_stop_halts_at_the_first_non_improvement():
    e = _examples()["three"]
    a = np.cumprod(np.array(e["conf"]), axis=1)
    trace = []
    ref.schedule(a, e["sps"], trace=trace)
    # (1,1) improves, (1,2) does not: the scan ends after two candidates
    assert [(r, j) for r, j, _, _, _ in trace] == [(1, 1), (1, 2)]


def _brute_best_tau(a, m):
    """Largest tau over every prefix-consistent length assignment with
    sum(l) = m (exhaustive)."""
    R, gamma = a.shape
    best = -math.inf
    for ls in itertools.product(range(gamma + 1), repeat=R):
        if sum(ls) != m:
            continue
        best = max(best, R + sum(a[r, :l].sum() for r, l in enumerate(ls)))
    return best


def test_sorted_scan_reaches_the_best_tau_at_every_batch_size():
    # Lemmas 1-2: the top-m candidates are prefix-closed and maximise tau, so
    # the scan's tau at B = R + m is the best over all assignments of that size.
    rng = np.random.default_rng(3)
    for _ in range(40):
        R, gamma = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        a = np.cumprod(rng.random((R, gamma)), axis=1)
        sps = np.concatenate([[np.nan], rng.random(R * (gamma + 1))])
        trace = []
        lengths, _, _ = ref.schedule(a, sps, early_stop=False, trace=trace)
        for m, (_, _, B, tau, _) in enumerate(trace, start=1):
            assert B == R + m
            assert abs(tau - _brute_best_tau(a, m)) < 1e-12
        # Lemma 1: every admitted set is prefix-closed
        seen = [0] * R
        for r, j, _, _, _ in trace:
            assert j == seen[r - 1] + 1
            seen[r - 1] = j


def test_early_stop_is_the_global_optimum_on_unimodal_curves():
    rng = np.random.default_rng(4)
    checked = 0
    for _ in range(300):
        R, gamma = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        a = np.cumprod(rng.random((R, gamma)), axis=1)
        n = np.arange(R * (gamma + 1) + 1, dtype=np.float64)
        sps = 1.0 / (1.0 + (n / rng.uniform(1.0, 2.0 * R)) ** rng.uniform(1.0, 3.0))
        trace = []
        ref.schedule(a, sps, early_stop=False, trace=trace)
        curve = [R * sps[R]] + [t[4] for t in trace]
        peak = int(np.argmax(curve))
        if not (all(x < y for x, y in zip(curve[:peak], curve[1:peak + 1]))
                and all(x > y for x, y in zip(curve[peak:], curve[peak + 1:]))):
            continue  # not unimodal: the early stop makes no optimality claim
        lengths, best, _ = ref.schedule(a, sps)
        brute = max(
            (R + sum(a[r, :l].sum() for r, l in enumerate(ls))) * sps[R + sum(ls)]
            for ls in itertools.product(range(gamma + 1), repeat=R))
        assert abs(best - brute) < 1e-12
        assert abs((R + sum(a[r, :l].sum() for r, l in enumerate(lengths))) * sps[R + lengths.sum()] - best) < 1e-12
        checked += 1
    assert checked >= 100


def test_ties_go_to_the_lowest_request_then_position():
    a = np.array([[0.5, 0.5], [0.5, 0.25], [0.5, 0.5]])
    trace = []
    ref.schedule(a, np.ones(10), early_stop=False, trace=trace)
    assert [(r, j) for r, j, _, _, _ in trace] == [(1, 1), (1, 2), (2, 1), (3, 1), (3, 2), (2, 2)]
    # zero survival is never a candidate
    lengths, best, _ = ref.schedule(np.array([[0.9, 0.0], [0.0, 0.0]]), np.ones(7))
    assert lengths.tolist() == [1, 0] and best == 2.9


def test_scheduled_lengths_end_the_block_with_the_bonus_of_row_l_plus_one():
    V, gamma, B = 5, 4, 6
    rng = np.random.default_rng(8)
    U = rng.normal(0, 1, size=(B, gamma, V)).astype(np.float32)
    tgt = rng.normal(0, 1, size=(B, gamma + 1, V)).astype(np.float32)
    W1, W2 = rng.normal(0, 1, size=(V, 2)), rng.normal(0, 1, size=(2, V))
    x0 = np.zeros(B, dtype=np.int32)
    seeds = np.arange(B, dtype=np.uint64) + np.uint64(11)
    d = ref.markov_draft(U, W1, W2, x0, 1.0, seeds, 2)
    full = ref.verify(U, W1, W2, x0, d["tokens"], tgt, 1.0, seeds, 2)
    same = ref.verify(U, W1, W2, x0, d["tokens"], tgt, 1.0, seeds, 2, lengths=np.full(B, gamma))
    for key in ("accept_len", "out_tokens"):
        assert (full[key] == same[key]).all()
    zero = ref.verify(U, W1, W2, x0, d["tokens"], tgt, 1.0, seeds, 2, lengths=np.zeros(B, dtype=np.int32))
    assert (zero["accept_len"] == 0).all() and (zero["out_tokens"][:, 1:] == -1).all()
    assert np.isnan(zero["accept_prob"]).all()
    for b in range(B):
        # l = 0 is plain decoding: the stream-2 draw at position 1 from p_t^1
        y, _ = ref.inverse_cdf(sp_softmax(tgt[b, 0].astype(np.float64)), ref.philox.uniform(int(seeds[b]), 2, 1, 2))
        assert zero["out_tokens"][b, 0] == y
    greedy = ref.verify(U, W1, W2, x0, d["tokens"], tgt, 0.0, seeds, 2, lengths=np.zeros(B, dtype=np.int32))
    assert (greedy["out_tokens"][:, 0] == np.argmax(tgt[:, 0], axis=1)).all()


def _counterexample_round(B, early_stop, rnd):
    """Eq. 9-10: vocabulary {A, B}, p_d = (0.5, 0.5), p_t = (0.7, 0.3) at
    position 1, a_1 = 0.8; the confidence of position 2 depends on the drafted
    x_1 (0.9 after A, 0 after B).  Returns the first emitted token per request."""
    V, gamma = 2, 2
    U = np.zeros((B, gamma, V), dtype=np.float32)
    tgt = np.tile(np.log(np.array([0.7, 0.3])).astype(np.float32), (B, gamma + 1, 1))
    W1, W2 = np.zeros((V, 2)), np.zeros((2, V))
    x0 = np.zeros(B, dtype=np.int32)
    seeds = (np.arange(B, dtype=np.uint64) + np.uint64(rnd * B)) * np.uint64(40503) + np.uint64(7)
    d = ref.markov_draft(U, W1, W2, x0, 1.0, seeds, rnd)
    sps = np.array([np.nan, 1.0, 0.5, 0.45])
    lengths = np.empty(B, dtype=np.int32)
    for b in range(B):
        c2 = 0.9 if d["tokens"][b, 0] == 0 else 0.0
        lengths[b] = ref.schedule(np.array([[0.8, 0.8 * c2]]), sps, early_stop=early_stop)[0][0]
    v = ref.verify(U, W1, W2, x0, d["tokens"], tgt, 1.0, seeds, rnd, lengths=lengths)
    return v["out_tokens"][:, 0]


@pytest.mark.slow
def test_non_anticipating_scheduler_is_lossless_and_anticipating_one_is_not():
    n = 20000
    causal = _counterexample_round(n, True, 1)
    anticip = _counterexample_round(n, False, 1)
    se = math.sqrt(0.7 * 0.3 / n)
    assert abs((causal == 0).mean() - 0.7) < 5 * se          # Pr(Y = A) = p_t(A)
    assert abs((anticip == 0).mean() - 0.85) < 5 * math.sqrt(0.85 * 0.15 / n)  # Eq. 10


@pytest.mark.slow
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_fixed_scheduled_lengths_keep_the_round_lossless(T):
    # lengths fixed before drafting (non-anticipating): the first emitted
    # token follows p_t^1 and the second p_t^2(. | first) for every length mix
    V, gamma, r, B, R = 4, 3, 2, 160, 60
    rng = np.random.default_rng(6)
    U = np.repeat(rng.normal(0, 1.0, size=(1, gamma, V)).astype(np.float32), B, axis=0)
    W1, W2 = rng.normal(0, 1.0, size=(V, r)), rng.normal(0, 1.0, size=(r, V))
    G = rng.normal(0, 1.2, size=(gamma + 1, V, V)).astype(np.float32)
    anchor = 2
    x0 = np.full(B, anchor, dtype=np.int32)
    lengths = (np.arange(B) % (gamma + 1)).astype(np.int32)
    first, second = np.zeros(V), np.zeros((V, V))
    for rnd in range(R):
        seeds = (np.arange(B, dtype=np.uint64) + np.uint64(rnd * B)) * np.uint64(2246822519) + np.uint64(3)
        d = ref.markov_draft(U, W1, W2, x0, T, seeds, rnd)
        tgt = np.empty((B, gamma + 1, V), dtype=np.float32)
        for b in range(B):
            prev = anchor
            for k in range(gamma + 1):
                tgt[b, k] = G[k, prev]
                if k < gamma:
                    prev = d["tokens"][b, k]
        v = ref.verify(U, W1, W2, x0, d["tokens"], tgt, T, seeds, rnd, lengths=lengths)
        assert (v["accept_len"] <= lengths).all()
        for b in range(B):
            y = v["out_tokens"][b]
            first[y[0]] += 1
            if v["accept_len"][b] >= 1:
                second[y[0], y[1]] += 1
    law1 = sp_softmax(G[0, anchor].astype(np.float64) / T)
    assert chisquare(first, law1 * first.sum()).pvalue > 1e-4
    tested = 0
    for x in range(V):
        if second[x].sum() < 150:
            continue
        law2 = sp_softmax(G[1, x].astype(np.float64) / T)
        assert chisquare(second[x], law2 * second[x].sum()).pvalue > 1e-4
        tested += 1
    assert tested >= 2


# ----------------------------------------------------------------------------
# The asynchronous adaptation ("Adapting Algorithm 1 to Real Hardware: Two
# Conflicts", "The Asynchronous Fix, and Why It Stays Lossless"): capacity K
# from an unconstrained search on earlier survival products, admission of the
# current top-K candidates.
# ----------------------------------------------------------------------------

def test_capacity_on_the_printed_curves_is_their_global_maximum():
    ex = _examples()
    for name, K in (("two", 1), ("three", 1), ("eq9", 0)):
        e = ex[name]
        a = np.cumprod(np.array(e["conf"]), axis=1)
        k, theta = ref.schedule_capacity(a, e["sps"])
        assert k == K and _close(theta, e["best"])


def test_jagged_curve_traps_the_early_stop_but_not_the_capacity_search():
    # Conflict 1: a cliff right after B = R stops the causal scan at once;
    # the unconstrained search finds the maximum past it.
    a = np.array([[0.9, 0.8, 0.7]])
    sps = np.array([np.nan, 1.0, 0.5, 0.49, 0.48])
    assert ref.schedule(a, sps)[0].tolist() == [0]
    k, theta = ref.schedule_capacity(a, sps)
    assert k == 3 and abs(theta - 3.4 * 0.48) < 1e-12


def test_capacity_is_the_optimum_over_every_assignment_on_any_curve():
    rng = np.random.default_rng(12)
    for _ in range(60):
        R, gamma = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        a = np.cumprod(rng.random((R, gamma)), axis=1)
        sps = np.concatenate([[np.nan], rng.random(R * (gamma + 1))])   # jagged
        k, theta = ref.schedule_capacity(a, sps)
        brute = max((R + sum(a[r, :l].sum() for r, l in enumerate(ls))) * sps[R + sum(ls)]
                    for ls in itertools.product(range(gamma + 1), repeat=R))
        assert abs(theta - brute) < 1e-12
        lengths = ref.admit_top(a, k)
        assert lengths.sum() == k
        assert abs((R + sum(a[r, :l].sum() for r, l in enumerate(lengths))) * sps[R + k] - theta) < 1e-12


def test_top_k_admission_is_prefix_closed_and_bounded():
    rng = np.random.default_rng(13)
    a = np.cumprod(np.round(rng.uniform(0.2, 1.0, size=(9, 5)) * 4) / 4, axis=1)   # with ties
    order = []
    ref.schedule(a, np.ones(60), early_stop=False, trace=order)
    for K in range(0, 50):
        lengths = ref.admit_top(a, K)
        assert lengths.sum() == min(K, 45)
        # the admitted set is the first K candidates of Algorithm 1's order
        seen = [0] * 9
        for r, j, _, _, _ in order[:K]:
            seen[r - 1] = max(seen[r - 1], j)
        assert lengths.tolist() == seen
    assert ref.admit_top(np.array([[0.5, 0.0], [0.0, 0.0]]), 5).tolist() == [1, 0]


def _lagged_round(B, K, rnd):
    """Two requests per pair: request 2i is the Eq. 9-10 counterexample
    (p_d = (0.5, 0.5), p_t = (0.7, 0.3), c_2 = 0.9 after A and 0 after B),
    request 2i+1 has survivals (0.7, 0.35) fixed.  With capacity K fixed
    before the draft, the second admission goes to request 2i's position 2
    after A (0.72 > 0.7) and to request 2i+1 otherwise."""
    V, gamma = 2, 2
    U = np.zeros((B, gamma, V), dtype=np.float32)
    tgt = np.tile(np.log(np.array([0.7, 0.3])).astype(np.float32), (B, gamma + 1, 1))
    W1, W2 = np.zeros((V, 2)), np.zeros((2, V))
    x0 = np.zeros(B, dtype=np.int32)
    seeds = (np.arange(B, dtype=np.uint64) + np.uint64(rnd * B)) * np.uint64(69069) + np.uint64(5)
    d = ref.markov_draft(U, W1, W2, x0, 1.0, seeds, rnd)
    lengths = np.empty(B, dtype=np.int32)
    for p in range(0, B, 2):
        c2 = 0.9 if d["tokens"][p, 0] == 0 else 0.0
        a = np.array([[0.8, 0.8 * c2], [0.7, 0.35]])
        lengths[p:p + 2] = ref.admit_top(a, K)
    v = ref.verify(U, W1, W2, x0, d["tokens"], tgt, 1.0, seeds, rnd, lengths=lengths)
    return v["out_tokens"][:, 0], lengths


@pytest.mark.slow
def test_lagged_capacity_admission_is_lossless():
    n = 20000
    first, lengths = _lagged_round(n, 2, 3)
    assert set(np.unique(lengths[1::2])) == {0, 1}       # request 2i+1's admission varies with 2i's draft
    for part in (first[0::2], first[1::2]):
        m = len(part)
        assert abs((part == 0).mean() - 0.7) < 5 * math.sqrt(0.21 / m)
