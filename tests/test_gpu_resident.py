"""GPU parity of the device-resident draft loop: dspark_markov_draft given the
vocabulary-major W2T copy runs all gamma positions of [R] "The Sequential
Correction" (Eq. 4, Markov head Eq. 5) in one cooperative launch with W2 held
in registers.  Every case checks, through the library's event timer, that the
resident kernel is what ran (one launch, no per-position tile passes), then
compares tokens, draft_prob and draft_lse with the float64 oracle to the
parity bar.

Cases: vocabularies with most waves' column ranges empty (V = 8192) and with
every range full (V = 153600), ragged last row groups, two selections per
workgroup (B > 256), greedy, invalid anchors,
determinism, and the full-size workloads whose draft the benchmark times --
every request of V=151936 B=256 T=0.7 and B=32, and every request of the
greedy B=512 workload.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads
from oracle_pool import OraclePool
from parity import Dev, compare_draft, f64_weights

torch = pytest.importorskip("torch")
dsp = pytest.importorskip("draft_sampling_verification_bias_amd")

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    dsp.load()
    yield
    torch.cuda.synchronize()


def resident_draft(d, wl, W2T, rnd=None, x0=None):
    """The draft with W2T, asserting that the resident kernel ran."""
    dsp.profile_enable(True)
    out = dsp.markov_draft(d.U, d.W1, d.W2, d.x0 if x0 is None else x0, wl.T, d.seeds,
                           wl.rnd if rnd is None else rnd, W2T=W2T)
    torch.cuda.synchronize()
    prof = dsp.profile_read()
    dsp.profile_enable(False)
    assert prof.get("draft_resident", (0, 0.0))[0] == 1, prof
    assert "tile_pass_sample" not in prof and "tile_pass_greedy" not in prof, prof
    return [t.cpu().numpy() for t in out]


SMALL = [
    ("v151936_b256_t07", dict(B=16, V=8192, gamma=4)),      # most column ranges empty
    ("v151936_b32", dict(B=40, V=40960, gamma=3)),           # ragged last group of 16 rows
    ("v151936_b32", dict(B=7, V=153600, gamma=2)),           # five 16-column sub-blocks in every range
    ("v151936_b256_t07", dict(B=300, V=16384, gamma=2)),     # two selections per workgroup
    ("greedy_v151936_b512", dict(B=24, V=16384, gamma=3)),
    ("greedy_v151936_b512", dict(B=300, V=8192, gamma=2)),
    ("v262144_b128", dict(B=33, V=65536, gamma=3, T=0.5)),
    # halves of 64 and 36 requests on disjoint selector waves, E rows issued
    # late and early over five positions
    ("v151936_b256_t07", dict(B=100, V=24576, gamma=5)),
    ("greedy_v151936_b512", dict(B=128, V=16384, gamma=4)),  # two halves of exactly 64
    ("v151936_b32", dict(B=129, V=8192, gamma=3)),            # first half of 80: every wave on both halves
]


@pytest.mark.parametrize("name,kw", SMALL)
def test_resident_draft_matches_the_oracle(name, kw):
    wl = workloads.make(name, **kw)
    say("[resident %s %s]" % (name, kw))
    d = Dev(wl)
    W2T = dsp.transpose_w2(d.W2)
    tok, prob, lse = resident_draft(d, wl, W2T)
    W1f, W2f = f64_weights(wl)
    ref = oracle.markov_draft(wl.U, W1f, W2f, wl.x0, wl.T, wl.seeds, wl.rnd)
    n, ex, whole = compare_draft(ref, tok, prob, lse, range(wl.B), wl.T)
    say("[resident] %d positions equal, %d exempt" % (n, ex))
    assert ex <= 1 and len(whole) >= wl.B - 1


def test_resident_draft_invalid_anchors_and_determinism():
    wl = workloads.make("v151936_b256_t07", B=20, V=16384, gamma=3)
    d = Dev(wl)
    W2T = dsp.transpose_w2(d.W2)
    x0 = wl.x0.copy()
    x0[3], x0[11] = wl.V, -1
    dx0 = torch.from_numpy(x0).cuda()
    tok, prob, lse = resident_draft(d, wl, W2T, x0=dx0)
    assert (tok[[3, 11]] == -1).all() and np.isnan(prob[[3, 11]]).all() and np.isnan(lse[[3, 11]]).all()
    W1f, W2f = f64_weights(wl)
    reqs = [b for b in range(wl.B) if b not in (3, 11)]
    ref = oracle.markov_draft(wl.U, W1f, W2f, x0, wl.T, wl.seeds, wl.rnd, requests=reqs)
    n, ex, _ = compare_draft(ref, tok, prob, lse, reqs, wl.T)
    assert n > 0 and ex == 0
    tok2, prob2, lse2 = resident_draft(d, wl, W2T, x0=dx0)
    np.testing.assert_array_equal(tok2, tok)
    np.testing.assert_array_equal(prob2[~np.isnan(prob2)], prob[~np.isnan(prob)])
    np.testing.assert_array_equal(lse2[~np.isnan(lse2)], lse[~np.isnan(lse)])


def test_resident_and_per_position_drafts_agree():
    # the same draws from both schedules of the loop (their float32 sums are
    # ordered differently, so a draw within rounding of a boundary may differ)
    wl = workloads.make("v151936_b32", B=64, V=32768, gamma=5)
    d = Dev(wl)
    W2T = dsp.transpose_w2(d.W2)
    tok, prob, lse = resident_draft(d, wl, W2T)
    t2, p2, l2 = (t.cpu().numpy() for t in dsp.markov_draft(d.U, d.W1, d.W2, d.x0, wl.T, d.seeds, wl.rnd))
    same = (tok == t2).all(axis=1)
    assert same.sum() >= wl.B - 1
    np.testing.assert_allclose(prob[same], p2[same], rtol=2e-5)
    np.testing.assert_allclose(lse[same], l2[same], rtol=1e-5, atol=2e-6)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["v151936_b256_t07", "v151936_b32", "greedy_v151936_b512"])
def test_resident_draft_full_size_every_request(name):
    wl = workloads.make(name)
    say("[resident full %s] B=%d V=%d gamma=%d T=%g" % (name, wl.B, wl.V, wl.gamma, wl.T))
    d = Dev(wl)
    W2T = dsp.transpose_w2(d.W2)
    tok, prob, lse = resident_draft(d, wl, W2T)
    del d
    torch.cuda.empty_cache()
    with OraclePool(wl) as pool:
        ref = pool.draft(range(wl.B))
    n, ex, whole = compare_draft(ref, tok, prob, lse, range(wl.B), wl.T)
    say("[resident full %s] %d positions equal, %d exempt, %d whole requests" % (name, n, ex, len(whole)))
    assert ex <= 1
    assert len(whole) >= wl.B - 1
