"""GPU parity of dspark_rnn_draft (block sampling with the RNN head of DSpark,
"Instantiation 2: The RNN Head", Eq. 6) against the float64 oracle, through
the C ABI -- and of the verification and survival products of its drafts
(dspark_verify / dspark_survival given the draft's operand rows e_k, the
decode round of "Putting It All Together" feeding either head's block to the
target) against oracle.verify / oracle.survival with the oracle's own e_k.

The oracle runs the cell in float64 with e_k unrounded; the library runs the
cell in float32 (the precision of its inputs Wp and hp) and feeds e_k to the
bf16 tile pass as two bf16 parts, so the draft logits agree to the tolerances
of ``parity.py`` and e_k itself within E_ATOL.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import Dev, compare_draft, compare_survival, compare_verify, f64_weights

torch = pytest.importorskip("torch")
dsp = pytest.importorskip("draft_sampling_verification_bias_amd")

pytestmark = pytest.mark.gpu

# e_k = tanh(o): float32 dot products of 2r terms of size ~1 / sqrt(2r), the
# state carried over gamma steps through gates below 1, float32 tanh; each
# part is a few 1e-8 at r <= 512
E_ATOL = 1e-6


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


def run_rnn(wl, reqs, label, seed=0, check_verify=True):
    say("[%s] rnn draft B=%d V=%d r=%d gamma=%d T=%g" % (label, wl.B, wl.V, wl.r, wl.gamma, wl.T))
    assert wl.wdtype == "bf16"
    Wp, hp = workloads.rnn_inputs(wl.B, wl.gamma, wl.r, seed=seed)
    d = Dev(wl)
    dWp, dhp = torch.from_numpy(Wp).cuda(), torch.from_numpy(hp).cuda()
    tok, prob, lse, e = dsp.rnn_draft(d.U, d.W1, d.W2, dWp, dhp, d.x0, wl.T, d.seeds, wl.rnd, with_e=True)
    torch.cuda.synchronize()
    tok_h, prob_h, lse_h, e_h = (t.cpu().numpy() for t in (tok, prob, lse, e))
    W1f, W2f = f64_weights(wl)
    ref = oracle.rnn_draft(wl.U, W1f, W2f, Wp.astype(np.float64), None, wl.x0, wl.T, wl.seeds, wl.rnd,
                           requests=reqs, hp=hp.astype(np.float64))
    n, ex, whole = compare_draft(ref, tok_h, prob_h, lse_h, reqs, wl.T)
    say("[%s] draft: %d positions equal, %d exempt draws" % (label, n, ex))
    assert n > 0
    for b in whole:
        err = np.abs(e_h[b] - ref["E"][b]).max()
        assert err <= E_ATOL, "e_k of request %d: max |gpu - oracle| = %.3g" % (b, err)
    if check_verify and whole:
        vreq = sorted(whole)
        vref = oracle.verify(wl.U, W1f, W2f, wl.x0, tok_h, wl.tgt, wl.T, wl.seeds, wl.rnd, requests=vreq,
                             E=ref["E"])
        variants = [None] + ([dsp.transpose_w2(d.W2)] if wl.T > 0 else [])
        for W2T in variants:
            alen, otok, aprob = dsp.verify(d.U, d.W1, d.W2, d.x0, tok, prob, d.tgt, wl.T, d.seeds, wl.rnd, E=e,
                                           W2T=W2T)
            torch.cuda.synchronize()
            nv, exv = compare_verify(vref, alen.cpu().numpy(), otok.cpu().numpy(), aprob.cpu().numpy(), vreq, wl.T)
            say("[%s] verify of the rnn draft%s: %d requests equal, %d exempt; mean accepted %.3f"
                % (label, " with W2T" if W2T is not None else "", nv, exv, alen.cpu().numpy()[vreq].mean()))
            assert nv > 0 and exv <= 1
        cst, surv = dsp.survival(d.U, d.W1, d.W2, d.x0, tok, lse, d.tgt, wl.T, E=e)
        torch.cuda.synchronize()
        rc, ra = oracle.survival(wl.U, W1f, W2f, wl.x0, tok_h, wl.tgt, wl.T, requests=vreq, E=ref["E"])
        compare_survival(rc, ra, cst.cpu().numpy(), surv.cpu().numpy(), vreq)
        say("[%s] survival of the rnn draft: %d requests equal" % (label, len(vreq)))
    return tok_h, e_h, ref


SMALL = [
    ("v151936_b32", dict(V=4099, B=37, gamma=5, r=64)),
    ("v151936_b256_t07", dict(V=3001, B=40, r=256)),
    ("greedy_v151936_b512", dict(V=5003, B=70, r=32)),
    # r = 512: two load passes of the cell's 16-column chunks
    ("v151936_b32", dict(V=130, B=3, gamma=2, r=512)),
    ("v151936_b32", dict(V=5, B=2, gamma=3, r=16)),
    # r = 48: three chunks, the rest of the cell's load pass repeats the last
    ("v151936_b32", dict(V=777, B=11, gamma=3, r=48)),
    # many full tiles and a ragged one under the generic tile kernel, several
    # row groups, a ragged request group of the cell
    ("v151936_b256_t07", dict(V=65540, B=203, gamma=2)),
    ("greedy_v151936_b512", dict(V=20000, B=131, gamma=3)),
    # rows of more than 2048 tiles: the block-wide selection
    ("v151936_b32", dict(V=264000, B=9, gamma=2)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=["%s-%s" % (n, "-".join("%s%s" % i for i in kw.items())) for n, kw in SMALL])
def test_small_rnn_parity(name, kw):
    wl = workloads.make(name, **kw)
    run_rnn(wl, list(range(wl.B)), name)


def test_full_size_sampled_rnn_parity():
    """V = 151936, B = 256, gamma = 7, r = 256, T = 0.7; the oracle on a
    sample of requests."""
    wl = workloads.make("v151936_b256_t07")
    run_rnn(wl, [0, 97, 255], "v151936_b256_t07")
    torch.cuda.empty_cache()


def test_full_size_sampled_rnn_parity_greedy():
    """V = 151936, B = 512, gamma = 7, r = 256, T = 0 (argmax summaries on
    the eight-wave two-part ring tile kernel, two row groups)."""
    wl = workloads.make("greedy_v151936_b512")
    run_rnn(wl, [0, 300, 511], "greedy_v151936_b512", seed=1)
    torch.cuda.empty_cache()


def test_full_size_sampled_rnn_parity_v262144():
    """V = 262144 (2048 tiles, the wave-level selection's largest rows),
    B = 128, gamma = 7, r = 256, T = 1."""
    wl = workloads.make("v262144_b128")
    run_rnn(wl, [0, 64, 127], "v262144_b128", seed=2)
    torch.cuda.empty_cache()


def test_invalid_anchor_is_reported_per_request():
    wl = workloads.make("v151936_b32", V=1001, B=6, gamma=3, r=32)
    wl.x0[1] = -1
    wl.x0[4] = wl.V
    Wp, hp = workloads.rnn_inputs(wl.B, wl.gamma, wl.r)
    d = Dev(wl)
    tok, prob, lse, _ = dsp.rnn_draft(d.U, d.W1, d.W2, torch.from_numpy(Wp).cuda(), torch.from_numpy(hp).cuda(),
                                      d.x0, wl.T, d.seeds, wl.rnd)
    torch.cuda.synchronize()
    tok_h, prob_h = tok.cpu().numpy(), prob.cpu().numpy()
    for b in (1, 4):
        assert (tok_h[b] == -1).all() and np.isnan(prob_h[b]).all()
    good = [0, 2, 3, 5]
    W1f, W2f = f64_weights(wl)
    ref = oracle.rnn_draft(wl.U, W1f, W2f, Wp.astype(np.float64), None, wl.x0, wl.T, wl.seeds, wl.rnd,
                           requests=good, hp=hp.astype(np.float64))
    n, _, _ = compare_draft(ref, tok_h, prob_h, lse.cpu().numpy(), good, wl.T)
    assert n > 0


def test_rnn_draft_is_deterministic_and_differs_from_markov():
    wl = workloads.make("v151936_b256_t07", V=3001, B=16, r=64)
    Wp, hp = workloads.rnn_inputs(wl.B, wl.gamma, wl.r, seed=3)
    d = Dev(wl)
    dWp, dhp = torch.from_numpy(Wp).cuda(), torch.from_numpy(hp).cuda()
    a = [t.cpu().numpy() for t in dsp.rnn_draft(d.U, d.W1, d.W2, dWp, dhp, d.x0, wl.T, d.seeds, 5, with_e=True)]
    b = [t.cpu().numpy() for t in dsp.rnn_draft(d.U, d.W1, d.W2, dWp, dhp, d.x0, wl.T, d.seeds, 5, with_e=True)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)
    m = dsp.markov_draft(d.U, d.W1, d.W2, d.x0, wl.T, d.seeds, 5)
    assert not np.array_equal(m[1].cpu().numpy(), a[1])



@pytest.mark.parametrize("name,kw", [
    ("v151936_b256_t07", dict(V=20000, B=200, gamma=3)),   # the eight-wave two-part ring
    ("greedy_v151936_b512", dict(V=20000, B=70, gamma=3)),  # the four-wave two-part ring, greedy
])
def test_rnn_draft_verified_at_scheduled_lengths(name, kw):
    """An RNN-head draft verified with its e_k rows at fixed scheduled
    lengths l_b (every length 0..gamma) against oracle.verify with the same
    lengths and the oracle's own e_k."""
    wl = workloads.make(name, **kw)
    Wp, hp = workloads.rnn_inputs(wl.B, wl.gamma, wl.r, seed=4)
    d = Dev(wl)
    tok, prob, lse, e = dsp.rnn_draft(d.U, d.W1, d.W2, torch.from_numpy(Wp).cuda(), torch.from_numpy(hp).cuda(),
                                      d.x0, wl.T, d.seeds, wl.rnd, with_e=True)
    torch.cuda.synchronize()
    tok_h = tok.cpu().numpy()
    W1f, W2f = f64_weights(wl)
    reqs = list(range(wl.B))
    ref = oracle.rnn_draft(wl.U, W1f, W2f, Wp.astype(np.float64), None, wl.x0, wl.T, wl.seeds, wl.rnd,
                           requests=reqs, hp=hp.astype(np.float64))
    n, ex, whole = compare_draft(ref, tok_h, prob.cpu().numpy(), lse.cpu().numpy(), reqs, wl.T)
    assert n > 0 and whole
    lengths = (np.arange(wl.B) % (wl.gamma + 1)).astype(np.int32)
    lens_d = torch.from_numpy(lengths).cuda()
    W2T = dsp.transpose_w2(d.W2) if wl.T > 0 else None
    alen, otok, aprob = dsp.verify(d.U, d.W1, d.W2, d.x0, tok, prob, d.tgt, wl.T, d.seeds, wl.rnd, E=e,
                                   W2T=W2T, lengths=lens_d)
    torch.cuda.synchronize()
    vreq = sorted(whole)
    vref = oracle.verify(wl.U, W1f, W2f, wl.x0, tok_h, wl.tgt, wl.T, wl.seeds, wl.rnd, requests=vreq,
                         lengths=lengths, E=ref["E"])
    alen_h = alen.cpu().numpy()
    nv, exv = compare_verify(vref, alen_h, otok.cpu().numpy(), aprob.cpu().numpy(), vreq, wl.T)
    say("[%s] rnn draft at scheduled lengths: %d requests equal, %d exempt; mean accepted %.3f"
        % (name, nv, exv, alen_h[vreq].mean()))
    assert nv > 0 and exv <= 1
    assert (alen_h[vreq] <= lengths[vreq]).all()
