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


# ---------------------------------------------------------------------------
# The confidence head fused into the draft: dspark_markov_draft's optional
# confidence output, computed by the selection that draws x_{k-1} ("The
# Confidence Head", Eq. 7 and the draft loop of "Putting It All Together").
# The oracle drafts its own tokens and evaluates Eq. 7 on them; the requests
# whose whole block matches are compared.
# ---------------------------------------------------------------------------
FUSED = [
    ("tiny_v1000_b4", {}, 1000, False),                                # float32 weights
    ("v151936_b32", dict(V=4099, B=9, gamma=3, r=48), 17, True),       # d % 4 != 0: scalar loads
    ("v151936_b256_t07", dict(V=3001, B=40, r=64), 4096, True),
    ("greedy_v151936_b512", dict(V=5003, B=70, r=32), 64, True),       # greedy: the block-wide selection
    ("v151936_b32", dict(V=264000, B=9, gamma=2), 256, True),          # > 2048 tiles: block-wide sampling
    ("v151936_b256_t07", dict(B=300, V=20000, gamma=3), 4096, True),   # the ring tile pass, r = 256
    ("v151936_b256_t07", {}, 4096, True),                              # full size
]


@pytest.mark.parametrize("name,kw,d,use_sts", FUSED,
                         ids=["%s-d%d-%s" % (n, d, "-".join("%s%s" % i for i in kw.items())) for n, kw, d, _ in FUSED])
def test_draft_confidence_output_matches_the_oracle(name, kw, d, use_sts):
    from oracle_pool import OraclePool
    wl = workloads.make(name, **kw)
    say("[fused conf %s %s d=%d]" % (name, kw, d))
    h, w, sts = workloads.confidence_inputs(wl.B, wl.gamma, d, wl.r, seed=d + 1)
    dv = Dev(wl)
    head = (torch.from_numpy(h).cuda(), torch.from_numpy(w).cuda(), torch.from_numpy(sts).cuda() if use_sts else None)
    tok, prob, lse, conf = dsp.markov_draft(dv.U, dv.W1, dv.W2, dv.x0, wl.T, dv.seeds, wl.rnd, conf_head=head)
    t2, p2, l2 = dsp.markov_draft(dv.U, dv.W1, dv.W2, dv.x0, wl.T, dv.seeds, wl.rnd)
    torch.cuda.synchronize()
    # the confidence output leaves the draft itself unchanged
    assert torch.equal(tok, t2) and torch.equal(prob, p2) and torch.equal(lse, l2)
    tok_h, prob_h, lse_h, conf_h = (t.cpu().numpy() for t in (tok, prob, lse, conf))
    del dv, head, tok, prob, lse, conf, t2, p2, l2
    torch.cuda.empty_cache()
    W1f, W2f = f64_weights(wl)
    if wl.B * wl.V * wl.gamma > 1 << 26:
        with OraclePool(wl) as pool:
            ref = pool.draft(range(wl.B))
    else:
        ref = oracle.markov_draft(wl.U, W1f, W2f, wl.x0, wl.T, wl.seeds, wl.rnd)
    n, ex, whole = compare_draft(ref, tok_h, prob_h, lse_h, range(wl.B), wl.T)
    assert ex <= 1 and len(whole) >= wl.B - 1
    reqs = sorted(whole)
    c_ref = oracle.confidence(h, w, W1f, wl.x0, ref["tokens"], sts=sts if use_sts else None, requests=reqs)
    _compare(conf_h[reqs], c_ref[reqs], name)
    say("[fused conf %s] %d confidences equal, range %.3f..%.3f" % (name, len(reqs) * wl.gamma,
                                                                     np.nanmin(c_ref), np.nanmax(c_ref)))


def test_draft_confidence_output_invalid_anchor_and_resident_fallback():
    # an invalid anchor makes the whole block -1 and every confidence of that
    # request NaN; with W2T given, the draft that also returns confidences
    # runs the per-position launches (same draws, same confidences)
    wl = workloads.make("v151936_b256_t07", B=20, V=16384, gamma=3)
    d = 256
    h, w, sts = workloads.confidence_inputs(wl.B, wl.gamma, d, wl.r, seed=4)
    x0 = wl.x0.copy()
    x0[5], x0[13] = -1, wl.V
    dv = Dev(wl)
    dx0 = torch.from_numpy(x0.astype(np.int32)).cuda()
    head = (torch.from_numpy(h).cuda(), torch.from_numpy(w).cuda(), torch.from_numpy(sts).cuda())
    W2T = dsp.transpose_w2(dv.W2)
    dsp.profile_enable(True)
    tok, prob, lse, conf = dsp.markov_draft(dv.U, dv.W1, dv.W2, dx0, wl.T, dv.seeds, wl.rnd, conf_head=head, W2T=W2T)
    torch.cuda.synchronize()
    prof = dsp.profile_read()
    dsp.profile_enable(False)
    assert "draft_resident" not in prof and prof.get("draft_select", (0, 0.0))[0] == wl.gamma, prof
    tok_h, conf_h = tok.cpu().numpy(), conf.cpu().numpy()
    assert (tok_h[[5, 13]] == -1).all() and np.isnan(conf_h[[5, 13]]).all()
    good = [b for b in range(wl.B) if b not in (5, 13)]
    W1f, W2f = f64_weights(wl)
    ref = oracle.markov_draft(wl.U, W1f, W2f, x0, wl.T, wl.seeds, wl.rnd, requests=good)
    _, ex, whole = compare_draft(ref, tok_h, prob.cpu().numpy(), lse.cpu().numpy(), good, wl.T)
    reqs = sorted(whole)
    assert len(reqs) >= len(good) - 1
    c_ref = oracle.confidence(h, w, W1f, x0, ref["tokens"], sts=sts, requests=reqs)
    _compare(conf_h[reqs], c_ref[reqs], "invalid anchors")
