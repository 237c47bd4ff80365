"""GPU parity of the confidence head (dspark_confidence, Eq. 7 with
per-position temperature scaling) against the float64 oracle, and of the
whole scheduling round built on it: draft, confidence, survival products,
prefix scheduler and verification at the scheduled lengths, all through the
C ABI.  Confidences within 1e-5 relative; lengths exact; verification with
the tolerances of ``parity.py``."""

import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import PROB_ATOL, PROB_RTOL, Dev, compare_draft, compare_verify, f64_weights

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


def _weights(wl):
    if wl.wdtype == "bf16":
        return torch.from_numpy(wl.W1.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(wl.W1).cuda()


def _compare(c_gpu, c_ref, label):
    bad = np.abs(c_gpu - c_ref) > PROB_RTOL * np.abs(c_ref) + PROB_ATOL
    assert not bad.any(), "[%s] confidence differs at %s: gpu %r oracle %r" % (
        label, np.argwhere(bad)[:5].tolist(), c_gpu[bad][:5], c_ref[bad][:5])


@pytest.mark.parametrize("name,kw,d,use_sts", [
    ("tiny_v1000_b4", {}, 1000, False),
    ("v151936_b32", dict(V=4099, B=9, gamma=3, r=48), 17, True),      # d % 4 != 0: scalar loads
    ("v151936_b256_t07", dict(V=3001, B=40, r=64), 4096, True),
    ("v151936_b256_t07", {}, 4096, True),                              # full size, B = 256, r = 256
])
def test_confidence_parity(name, kw, d, use_sts):
    wl = workloads.make(name, **kw)
    h, w, sts = workloads.confidence_inputs(wl.B, wl.gamma, d, wl.r, seed=d)
    rng = np.random.default_rng(d)
    tokens = rng.integers(0, wl.V, size=(wl.B, wl.gamma)).astype(np.int32)
    W1f, _ = f64_weights(wl)
    conf = dsp.confidence(torch.from_numpy(h).cuda(), torch.from_numpy(w).cuda(), _weights(wl),
                          torch.from_numpy(wl.x0.astype(np.int32)).cuda(), torch.from_numpy(tokens).cuda(),
                          sts=torch.from_numpy(sts).cuda() if use_sts else None)
    torch.cuda.synchronize()
    ref = oracle.confidence(h, w, W1f, wl.x0, tokens, sts=sts if use_sts else None)
    _compare(conf.cpu().numpy(), ref, name)
    say("[%s d=%d] %d confidences equal, range %.3f..%.3f" % (name, d, ref.size, ref.min(), ref.max()))


def test_confidence_marks_invalid_previous_tokens_nan():
    B, gamma, d, r, V = 3, 3, 32, 16, 50
    h, w, _ = workloads.confidence_inputs(B, gamma, d, r)
    W1 = torch.randn(V, r, device="cuda")
    x0 = torch.tensor([0, -1, 3], dtype=torch.int32, device="cuda")
    tok = torch.tensor([[1, 2, 3], [1, 2, 3], [4, V, 5]], dtype=torch.int32, device="cuda")
    c = dsp.confidence(torch.from_numpy(h).cuda(), torch.from_numpy(w).cuda(), W1, x0, tok).cpu().numpy()
    assert np.isfinite(c[0]).all()
    assert np.isnan(c[1, 0]) and np.isfinite(c[1, 1:]).all()
    assert np.isfinite(c[2, :2]).all() and np.isnan(c[2, 2])


def test_confidence_scheduled_round_full_size():
    """v151936_b256_t07: draft, confidence head (d = 4096, STS), survival
    products of the confidences, prefix scheduler, verification at the
    scheduled lengths.  The oracle recomputes the confidences and the schedule
    of every request and the verification of a sample."""
    wl = workloads.make("v151936_b256_t07")
    d = 4096
    dv = Dev(wl)
    tok, prob, lse = dsp.markov_draft(dv.U, dv.W1, dv.W2, dv.x0, wl.T, dv.seeds, wl.rnd)
    h, w, sts = workloads.confidence_inputs(wl.B, wl.gamma, d, wl.r, seed=1)
    conf = dsp.confidence(torch.from_numpy(h).cuda(), torch.from_numpy(w).cuda(), dv.W1, dv.x0, tok,
                          sts=torch.from_numpy(sts).cuda())
    _, surv = dsp.survival(None, None, None, None, None, None, None, wl.T, conf=conf)
    sps = workloads.sps_curve(wl.B * (wl.gamma + 1), 4.0 * wl.B, 2.0)
    lengths, theta = dsp.schedule(surv, torch.from_numpy(sps).cuda())
    W2T = dsp.transpose_w2(dv.W2)
    alen, otok, aprob = dsp.verify(dv.U, dv.W1, dv.W2, dv.x0, tok, prob, dv.tgt, wl.T, dv.seeds, wl.rnd, W2T=W2T,
                                   lengths=lengths)
    torch.cuda.synchronize()
    tok_h = tok.cpu().numpy()
    W1f, W2f = f64_weights(wl)
    # the draft of a sample of requests
    rng = np.random.default_rng(9)
    reqs = sorted(set([0, wl.B - 1] + rng.choice(wl.B, size=4, replace=False).tolist()))
    ref_d = oracle.markov_draft(wl.U, W1f, W2f, wl.x0, wl.T, wl.seeds, wl.rnd, requests=reqs)
    n, ex, whole = compare_draft(ref_d, tok_h, prob.cpu().numpy(), lse.cpu().numpy(), reqs, wl.T)
    # confidences and survival products of every request from the GPU's drafted tokens
    c_ref = oracle.confidence(h, w, W1f, wl.x0, tok_h, sts=sts)
    _compare(conf.cpu().numpy(), c_ref, "scheduled round")
    _, a_ref = oracle.survival(None, None, None, None, None, None, wl.T, conf=c_ref)
    surv_h = surv.cpu().numpy()
    assert np.all(np.abs(surv_h - a_ref) <= PROB_RTOL * np.abs(a_ref) + PROB_ATOL)
    # the schedule from the GPU's survival products
    ref_len, ref_theta, margin = oracle.schedule(surv_h.astype(np.float64), sps)
    assert margin > 1e-9 * abs(ref_theta)
    lengths_h = lengths.cpu().numpy()
    assert (lengths_h == ref_len).all()
    # verification at those lengths on the sample
    vreq = sorted(whole)
    vref = oracle.verify(wl.U, W1f, W2f, wl.x0, tok_h, wl.tgt, wl.T, wl.seeds, wl.rnd, requests=vreq,
                         lengths=lengths_h)
    nv, exv = compare_verify(vref, alen.cpu().numpy(), otok.cpu().numpy(), aprob.cpu().numpy(), vreq, wl.T)
    say("[scheduled round] mean length %.2f, %d verified requests equal, %d exempt" % (lengths_h.mean(), nv, exv))
    assert nv > 0
    del dv, W2T
    torch.cuda.empty_cache()
