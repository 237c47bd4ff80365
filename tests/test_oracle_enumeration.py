"""Exact laws of the oracle's own draft and verify code, by enumeration.

The oracle's random numbers are replaced by symbolic uniforms: each one is
resolved where the oracle uses it -- an inverse-CDF draw (the outcome v with
probability p(v)) or an accept / keep comparison ``u < a`` (true with
probability a) -- and every combination of outcomes is run through the
unmodified ``markov_draft`` and ``verify`` (or ``residual_sample``), each
path weighted by the product of the probabilities of its outcomes.  The
result is the exact output law of the oracle's code, with no sampling error,
and it is held to what the pages fix:

* [E] "Speculative decoding, from zero to DSpark", section 2: the emitted
  tokens follow the target exactly.  With a target table G[k][prev] standing
  in for the target model on the drafted prefix (position k + 1 sees the
  token drafted at k), the first emitted token has law p_t^1 and, given that
  the first m - 1 emitted tokens were accepted drafts s, the m-th has law
  p_t^m( . | s).  Checked to 1e-12 for every prefix, for V <= 8, gamma <= 3.
* the same section's residual rule: the proposal scheme the oracle uses
  before its exact fallback has exactly the law norm(max(0, p_t - p_d))
  for every proposal limit.
* [R] "The Sequential Correction" (Eq. 4): the block law of the draft is the
  product of the per-position softmaxes along the drafted prefix.
"""

import collections

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import dspark_ref as ref
from oracle import philox


class _Paths:
    """Depth-first enumeration of outcome paths: ``choose`` returns the index
    of the outcome taken at the next branching point of the current run."""

    def __init__(self, prefix):
        self.path = list(prefix)
        self.nalt = [None] * len(prefix)
        self.pos = 0
        self.weight = 1.0

    def choose(self, weights):
        alts = [(i, w) for i, w in enumerate(weights) if w > 0]
        if self.pos < len(self.path):
            k = self.path[self.pos]
            self.nalt[self.pos] = len(alts)
        else:
            k = 0
            self.path.append(0)
            self.nalt.append(len(alts))
        self.pos += 1
        idx, w = alts[k]
        self.weight *= w
        return idx


class _SymUniform:
    """A uniform whose value is decided where it is used."""

    def __init__(self, paths):
        self.paths = paths

    def __lt__(self, a):           # accept / keep test: u < a holds with probability a
        a = float(a)
        return self.paths.choose([a, 1.0 - a]) == 0

    def __sub__(self, other):      # boundary-distance bookkeeping only
        return 1.0

    def __rsub__(self, other):
        return 1.0


class _SymPhilox:
    STREAM_DRAFT = philox.STREAM_DRAFT
    STREAM_ACCEPT = philox.STREAM_ACCEPT
    STREAM_RESIDUAL = philox.STREAM_RESIDUAL
    STREAM_FALLBACK = philox.STREAM_FALLBACK

    def __init__(self, paths):
        self.paths = paths

    def uniform(self, *args, **kw):
        return _SymUniform(self.paths)

    def block(self, *args, **kw):
        return (0, 0, 0, 0)

    def to_uniform(self, word):
        return _SymUniform(self.paths)


def _enumerate(run):
    """{outcome: exact probability} of ``run(paths)`` over every outcome path.
    Inside ``run`` the oracle module draws symbolic uniforms."""
    real_philox, real_icdf = ref.philox, ref.inverse_cdf
    law = collections.defaultdict(float)
    stack = [[]]
    npaths = 0
    try:
        while stack:
            prefix = stack.pop()
            paths = _Paths(prefix)
            ref.philox = _SymPhilox(paths)

            def icdf(p, u, _paths=paths):
                if not isinstance(u, _SymUniform):
                    return real_icdf(p, u)
                return _paths.choose(list(np.asarray(p, dtype=np.float64))), np.inf

            ref.inverse_cdf = icdf
            out = run(paths)
            for depth in range(len(prefix), len(paths.path)):
                for alt in range(1, paths.nalt[depth]):
                    stack.append(paths.path[:depth] + [alt])
            law[out] += paths.weight
            npaths += 1
    finally:
        ref.philox, ref.inverse_cdf = real_philox, real_icdf
    return law, npaths


def _problem(V, gamma, r, seed):
    rng = np.random.default_rng(seed)
    U = rng.normal(0, 1.0, size=(1, gamma, V)).astype(np.float32)
    W1 = rng.normal(0, 0.8, size=(V, r))
    W2 = rng.normal(0, 0.8, size=(r, V))
    G = rng.normal(0, 1.2, size=(gamma + 1, V, V)).astype(np.float32)   # G[k][prev]: target logits
    return U, W1, W2, G


def _round_law(V, gamma, r, T, max_proposals, seed, lengths=None):
    U, W1, W2, G = _problem(V, gamma, r, seed)
    anchor = V // 2
    x0 = np.array([anchor], dtype=np.int32)
    seeds = np.array([12345], dtype=np.uint64)

    def run(paths):
        d = ref.markov_draft(U, W1, W2, x0, T, seeds, 7)
        tgt = np.empty((1, gamma + 1, V), dtype=np.float32)
        prev = anchor
        for k in range(gamma + 1):
            tgt[0, k] = G[k, prev]
            if k < gamma:
                prev = int(d["tokens"][0, k])
        v = ref.verify(U, W1, W2, x0, d["tokens"], tgt, T, seeds, 7, max_proposals=max_proposals,
                       lengths=lengths)
        n = int(v["accept_len"][0])
        return tuple(int(t) for t in v["out_tokens"][0, :n + 1])

    law, npaths = _enumerate(run)
    return law, npaths, G, anchor


def _assert_lossless(law, G, anchor, T, ell):
    V = G.shape[1]
    assert abs(sum(law.values()) - 1.0) < 1e-12
    checked = 0
    for m in range(1, ell + 2):
        mass = collections.defaultdict(lambda: np.zeros(V))
        for seq, p in law.items():
            if len(seq) >= m:
                mass[seq[:m - 1]][seq[m - 1]] += p
        for s, row in mass.items():
            prev = s[-1] if s else anchor
            want = sp_softmax(G[m - 1, prev].astype(np.float64) / T)
            np.testing.assert_allclose(row, row.sum() * want, rtol=0, atol=1e-12)
            checked += 1
    assert checked >= (1 if ell == 0 else 3)


@pytest.mark.parametrize("V,gamma,T,max_prop", [
    (4, 3, 1.0, 0), (4, 3, 0.7, 1), (6, 3, 1.0, 0), (5, 3, 0.7, 0), (8, 2, 1.0, 0), (8, 2, 0.5, 0)])
def test_round_law_is_the_target_law_exactly(V, gamma, T, max_prop):
    law, npaths, G, anchor = _round_law(V, gamma, 3, T, max_prop, seed=V * 10 + gamma)
    assert npaths > V ** gamma
    _assert_lossless(law, G, anchor, T, gamma)


@pytest.mark.parametrize("ell", [0, 1, 2])
def test_scheduled_length_round_law_is_the_target_law_exactly(ell):
    V, gamma, T = 5, 3, 1.0
    lengths = np.array([ell], dtype=np.int32)
    law, _, G, anchor = _round_law(V, gamma, 3, T, 0, seed=3, lengths=lengths)
    assert max(len(s) for s in law) == ell + 1
    _assert_lossless(law, G, anchor, T, ell)


def test_a_planted_wrong_residual_fails_the_exact_law():
    # the oracle's residual replaced by a draw from p_t (the rule [R] could be
    # misread as): the exact law check must reject it
    def wrong(pt, pd, seed, rnd, j, max_proposals, dists):
        u = ref.philox.uniform(seed, rnd, j, ref.philox.STREAM_FALLBACK)
        return ref.inverse_cdf(pt, u)[0]

    saved = ref.residual_sample
    ref.residual_sample = wrong
    try:
        law, _, G, anchor = _round_law(4, 2, 3, 1.0, 0, seed=11)
    finally:
        ref.residual_sample = saved
    with pytest.raises(AssertionError):
        _assert_lossless(law, G, anchor, 1.0, 2)


@pytest.mark.parametrize("max_prop", [0, 1, 2, 3])
def test_residual_proposal_scheme_has_the_residual_law_exactly(max_prop):
    rng = np.random.default_rng(21 + max_prop)
    V = 5
    pt = rng.dirichlet(np.ones(V))
    pd = rng.dirichlet(np.ones(V))
    law, npaths = _enumerate(lambda paths: ref.residual_sample(pt, pd, 1, 2, 3, max_prop, []))
    got = np.zeros(V)
    for v, p in law.items():
        got[v] += p
    np.testing.assert_allclose(got, ref.residual_law(pt, pd), rtol=0, atol=1e-13)
    assert npaths >= int((pt > pd).sum())


def test_residual_law_is_the_normalised_positive_part():
    pt = np.array([0.7, 0.3])
    pd = np.array([0.5, 0.5])
    np.testing.assert_allclose(ref.residual_law(pt, pd), [1.0, 0.0], rtol=0, atol=0)
    pt = np.array([0.1, 0.2, 0.3, 0.4])
    pd = np.array([0.4, 0.1, 0.1, 0.4])
    np.testing.assert_allclose(ref.residual_law(pt, pd), [0.0, 1 / 3, 2 / 3, 0.0], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(ref.residual_law(pt, pt), pt)     # no positive mass: p_t


def test_draft_block_law_is_the_product_of_position_softmaxes():
    V, gamma, T = 5, 3, 0.8
    U, W1, W2, _ = _problem(V, gamma, 2, seed=4)
    x0 = np.array([2], dtype=np.int32)
    law, _ = _enumerate(lambda paths: tuple(int(t) for t in ref.markov_draft(
        U, W1, W2, x0, T, np.array([1], dtype=np.uint64), 0)["tokens"][0]))
    assert len(law) == V ** gamma
    for blk, p in law.items():
        want, prev = 1.0, 2
        for k, x in enumerate(blk):
            l = (U[0, k].astype(np.float64) + W1[prev] @ W2) / T
            want *= sp_softmax(l)[x]
            prev = x
        assert abs(p - want) < 1e-14


# ---------------------------------------------------------------------------
# Drafts of the RNN head ([R] "Instantiation 2: The RNN Head", Eq. 6): the
# decode round of [R] "Putting It All Together" verifies either head's block.
# Verification given the RNN draft's operand rows E is lossless; given the
# Markov head's law in their place it is not.
# ---------------------------------------------------------------------------

def _rnn_problem(V, gamma, r, d, seed):
    U, W1, W2, G = _problem(V, gamma, r, seed)
    rng = np.random.default_rng(seed + 1000)
    Wp = rng.normal(0, 0.9, size=(3 * r, 2 * r + d))
    h = rng.normal(0, 1.0, size=(1, gamma, d))
    return U, W1, W2, Wp, h, G


def _rnn_round(V, gamma, T, seed, use_e=True, r=2, d=2):
    U, W1, W2, Wp, h, G = _rnn_problem(V, gamma, r, d, seed)
    anchor = V // 2
    x0 = np.array([anchor], dtype=np.int32)
    seeds = np.array([99], dtype=np.uint64)

    def run(paths):
        dr = ref.rnn_draft(U, W1, W2, Wp, h, x0, T, seeds, 5)
        tgt = np.empty((1, gamma + 1, V), dtype=np.float32)
        prev = anchor
        for k in range(gamma + 1):
            tgt[0, k] = G[k, prev]
            if k < gamma:
                prev = int(dr["tokens"][0, k])
        v = ref.verify(U, W1, W2, x0, dr["tokens"], tgt, T, seeds, 5, max_proposals=0,
                       E=dr["E"] if use_e else None)
        n = int(v["accept_len"][0])
        return tuple(int(t) for t in v["out_tokens"][0, :n + 1])

    law, _ = _enumerate(run)
    return law, (U, W1, W2, Wp, h, G, x0, anchor)


@pytest.mark.parametrize("V,gamma,T", [(4, 3, 1.0), (5, 2, 0.7), (6, 2, 1.3)])
def test_rnn_draft_round_law_is_the_target_law_exactly(V, gamma, T):
    law, prob = _rnn_round(V, gamma, T, seed=50 + V)
    G, anchor = prob[5], prob[7]
    _assert_lossless(law, G, anchor, T, gamma)


def test_rnn_draft_verified_with_the_markov_law_is_not_lossless():
    law, prob = _rnn_round(4, 2, 1.0, seed=54, use_e=False)
    with pytest.raises(AssertionError):
        _assert_lossless(law, prob[5], prob[7], 1.0, 2)


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_rnn_survival_is_the_exact_acceptance_of_each_prefix(T):
    # c*_k along a drafted prefix s = x_1..x_{k-1} equals the exact probability
    # that position k is accepted given that s was drafted and accepted: the
    # ratio of the round-law masses of "n >= k, prefix s" and "n >= k-1, prefix
    # s", read off the enumerated round
    V, gamma = 4, 3
    U, W1, W2, Wp, h, G, x0, anchor = _rnn_problem(V, gamma, 2, 2, 77)[:6] + (
        np.array([V // 2], dtype=np.int32), V // 2)
    seeds = np.array([99], dtype=np.uint64)

    def run(paths):
        dr = ref.rnn_draft(U, W1, W2, Wp, h, x0, T, seeds, 5)
        tgt = np.empty((1, gamma + 1, V), dtype=np.float32)
        prev = anchor
        for k in range(gamma + 1):
            tgt[0, k] = G[k, prev]
            if k < gamma:
                prev = int(dr["tokens"][0, k])
        v = ref.verify(U, W1, W2, x0, dr["tokens"], tgt, T, seeds, 5, max_proposals=0, E=dr["E"])
        n = int(v["accept_len"][0])
        return n, tuple(int(t) for t in v["out_tokens"][0, :n])

    law, _ = _enumerate(run)
    checked = 0
    for k in range(1, gamma + 1):
        tested = collections.defaultdict(float)
        passed = collections.defaultdict(float)
        for (n, acc), p in law.items():
            if n >= k - 1:
                tested[acc[:k - 1]] += p
            if n >= k:
                passed[acc[:k - 1]] += p
        for s, pm in tested.items():
            forced = np.array([list(s) + [0] * (gamma - len(s))], dtype=np.int32)
            dr = ref.rnn_draft(U, W1, W2, Wp, h, x0, T, seeds, 5, forced=forced)
            tgt = np.empty((1, gamma + 1, V), dtype=np.float32)
            prev = anchor
            for j in range(gamma + 1):
                tgt[0, j] = G[j, prev]
                if j < gamma:
                    prev = int(forced[0, j])
            c, _ = ref.survival(U, W1, W2, x0, forced, tgt, T, E=dr["E"])
            assert abs(passed[s] / pm - c[0, k - 1]) < 1e-12, (k, s)
            checked += 1
    assert checked == 1 + V + V * V
