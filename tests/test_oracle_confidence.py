"""Pins of the oracle's confidence head (Eq. 7 of the DSpark technical review,
"The Confidence Head") with per-position temperature scaling (STS, same
section): special cases that reduce to the logistic function, the role of the
previous token's Markov embedding, and the order preservation the page
states for temperature scaling."""

import numpy as np
from scipy.special import expit

from oracle import dspark_ref as ref


def _case(B=5, gamma=4, d=6, r=3, V=9, seed=0):
    rng = np.random.default_rng(seed)
    h = rng.normal(0, 1, size=(B, gamma, d)).astype(np.float32)
    w = rng.normal(0, 0.7, size=d + r).astype(np.float32)
    W1 = rng.normal(0, 1, size=(V, r))
    x0 = rng.integers(0, V, size=B).astype(np.int32)
    tok = rng.integers(0, V, size=(B, gamma)).astype(np.int32)
    return h, w, W1, x0, tok


def test_zero_weights_give_one_half():
    h, w, W1, x0, tok = _case()
    c = ref.confidence(h, np.zeros_like(w), W1, x0, tok)
    assert (c == 0.5).all()


def test_is_the_logistic_of_the_concatenated_dot_product():
    h, w, W1, x0, tok = _case(seed=1)
    d = h.shape[2]
    c = ref.confidence(h, w, W1, x0, tok)
    for b in range(h.shape[0]):
        prev = [x0[b]] + tok[b, :-1].tolist()
        for k in range(h.shape[1]):
            feat = np.concatenate([h[b, k].astype(np.float64), W1[prev[k]]])
            assert abs(c[b, k] - expit(feat @ w.astype(np.float64))) < 1e-15
    # the hidden part alone (Markov weights zero) and the embedding part alone
    w_h = w.copy(); w_h[d:] = 0
    assert np.allclose(ref.confidence(h, w_h, W1, x0, tok), expit(h.astype(np.float64) @ w_h[:d].astype(np.float64)),
                       rtol=0, atol=1e-15)


def test_previous_token_is_the_anchor_then_the_drafted_prefix():
    h, w, W1, x0, tok = _case(seed=2)
    c = ref.confidence(h, w, W1, x0, tok)
    x0b = (x0 + 1) % W1.shape[0]
    c2 = ref.confidence(h, w, W1, x0b, tok)
    assert (c2[:, 0] != c[:, 0]).all() and (c2[:, 1:] == c[:, 1:]).all()
    tokb = tok.copy(); tokb[:, 1] = (tokb[:, 1] + 1) % W1.shape[0]
    c3 = ref.confidence(h, w, W1, x0, tokb)
    assert (c3[:, 2] != c[:, 2]).all()
    assert (np.delete(c3, 2, axis=1) == np.delete(c, 2, axis=1)).all()
    # the last drafted token feeds no position
    tokc = tok.copy(); tokc[:, -1] = (tokc[:, -1] + 1) % W1.shape[0]
    assert (ref.confidence(h, w, W1, x0, tokc) == c).all()


def test_temperature_scaling_is_order_preserving_and_pulls_to_one_half():
    h, w, W1, x0, tok = _case(B=40, seed=3)
    c = ref.confidence(h, w, W1, x0, tok)
    sts = np.array([0.5, 1.0, 2.0, 7.0])
    cs = ref.confidence(h, w, W1, x0, tok, sts=sts)
    assert (cs[:, 1] == c[:, 1]).all()                     # t = 1 is the raw score
    for k in range(4):                                     # same ranking of requests at every position
        assert (np.argsort(c[:, k], kind="stable") == np.argsort(cs[:, k], kind="stable")).all()
    assert (np.abs(cs[:, 2:] - 0.5) <= np.abs(c[:, 2:] - 0.5) + 1e-15).all()   # t > 1 flattens
    assert (np.abs(cs[:, 0] - 0.5) >= np.abs(c[:, 0] - 0.5) - 1e-15).all()     # t < 1 sharpens
    # sigma(z / t) = sigma(z)^(1/t) / (sigma(z)^(1/t) + (1 - sigma(z))^(1/t))
    p = c[:, 3] ** (1 / 7.0)
    q = (1 - c[:, 3]) ** (1 / 7.0)
    assert np.allclose(cs[:, 3], p / (p + q), rtol=1e-12, atol=0)
