"""The law of the library's residual draws against the plain residual law.

[E] "Speculative decoding, from zero to DSpark", section 2: after the first
rejection the replacement token is drawn from norm(max(0, p_t - p_d)).  Every
request of these batches has the same draft row and the same target row at
position 1 (only the Philox keys differ), so every request that rejects at
position 1 draws its correction from one law, which ``oracle.residual_law``
writes out directly (no proposal scheme, no random numbers).  The corrections
the GPU emits are binned and compared with that law by a chi-square test.

The rows span many 256-column target tiles (V = 6000, the probable tokens
spread over the whole vocabulary), so proposals land in many tiles; in the
second case the two rows are so close that the residual mass is about 2 %
and a fifth of the rejecting requests exhaust their 64 proposals and take the
exact inverse CDF fallback.
"""

import sys

import numpy as np
import pytest
from scipy.stats import chisquare

import oracle
from parity import seeds_tensor

torch = pytest.importorskip("torch")
dsp = pytest.importorskip("draft_sampling_verification_bias_amd")

pytestmark = pytest.mark.gpu


def _rows(V, r, noise, seed):
    rng = np.random.default_rng(seed)
    u = rng.normal(0, 1.0, size=V).astype(np.float32)
    hot = rng.choice(V, size=48, replace=False)
    u[hot] += 5.0
    W1 = (rng.normal(0, 0.05, size=(V, r))).astype(np.float32)
    W2 = (rng.normal(0, 0.05, size=(r, V))).astype(np.float32)
    x0 = int(rng.integers(0, V))
    t = u.astype(np.float64) + W1[x0].astype(np.float64) @ W2.astype(np.float64)
    t[hot] += rng.normal(0, noise, size=hot.size)
    return u, W1, W2, x0, t.astype(np.float32)


@pytest.mark.parametrize("noise,B,rounds", [(0.8, 4096, 6), (0.1, 16384, 8)])
def test_corrections_follow_the_residual_law(noise, B, rounds):
    V, r, gamma, T = 6000, 64, 1, 1.0
    u, W1, W2, x0, t = _rows(V, r, noise, seed=int(noise * 1000))
    print("residual law: V=%d B=%d rounds=%d target noise %g" % (V, B, rounds, noise), flush=True)
    dev = "cuda:0"
    U = torch.from_numpy(np.tile(u, (B, gamma, 1))).to(dev)
    tgt = torch.from_numpy(np.tile(t, (B, gamma + 1, 1))).to(dev)
    dW1, dW2 = torch.from_numpy(W1).to(dev), torch.from_numpy(W2).to(dev)
    dx0 = torch.full((B,), x0, dtype=torch.int32, device=dev)
    corrections = []
    for rnd in range(rounds):
        seeds = seeds_tensor(np.arange(B, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15) + np.uint64(rnd + 1))
        tok, prob, _ = dsp.markov_draft(U, dW1, dW2, dx0, T, seeds, rnd)
        alen, otok, _ = dsp.verify(U, dW1, dW2, dx0, tok, prob, tgt, T, seeds, rnd)
        torch.cuda.synchronize()
        a, o = alen.cpu().numpy(), otok.cpu().numpy()
        assert ((a == 0) | (a == 1)).all()
        corrections.append(o[a == 0, 0])
    y = np.concatenate(corrections)
    # the law, from the oracle's plain float64 softmaxes of the same rows
    pd, _ = oracle.softmax(oracle.draft_logits(u, W1.astype(np.float64), W2.astype(np.float64), x0, T))
    pt, _ = oracle.softmax(oracle.target_logits(t, T))
    law = oracle.residual_law(pt, pd)
    mass = float(np.maximum(0.0, pt - pd).sum())
    n = y.size
    print("residual law: mass %.4f, %d corrections" % (mass, n), flush=True)
    sys.stdout.flush()
    assert n >= 1500
    assert (law[y] > 0).all(), "a correction outside the support of the residual"
    counts = np.bincount(y, minlength=V).astype(np.float64)
    expect = law * n
    big = expect >= 5.0
    obs = np.append(counts[big], counts[~big].sum())
    exp = np.append(expect[big], expect[~big].sum())
    if exp[-1] < 5.0:  # pool the small tail into the last big bin
        obs[-2] += obs[-1]
        exp[-2] += exp[-1]
        obs, exp = obs[:-1], exp[:-1]
    assert big.sum() >= 8
    p = chisquare(obs, exp).pvalue
    print("residual law: %d bins, chi-square p = %.4f" % (obs.size, p), flush=True)
    assert p > 1e-4
