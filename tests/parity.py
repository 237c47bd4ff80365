"""Helpers of the GPU parity tests: device copies of a workload, the oracle
run on the same bytes, and the element-by-element comparisons with the
tolerances of the path:

* probabilities (draft_prob, accept_prob, c_star, survival):
  |gpu - oracle| <= 1e-5 * |oracle| + 1e-30;
* log-normalisers (draft_lse): |gpu - oracle| <= 4e-6 * |oracle| + 1e-6
  (float32 storage of a value near 20 alone is 1e-6);
* tokens, accepted lengths: exact, except where the oracle's uniform lies
  within 1e-6 (EXEMPT_RADIUS) of a decision boundary; at T = 0 exact always.
  After a mismatch at position k the rest of that request is conditioned on a
  different prefix and is not compared.
"""

import numpy as np
import torch

import oracle
from oracle import EXEMPT_RADIUS

PROB_RTOL = 1e-5
PROB_ATOL = 1e-30
LSE_RTOL = 4e-6
LSE_ATOL = 1e-6


class Dev:
    """Device copies of one workload (float32 logits, bf16 or float32 weights)."""

    def __init__(self, wl, device="cuda"):
        self.wl = wl
        self.U = torch.from_numpy(wl.U).to(device)
        self.tgt = torch.from_numpy(wl.tgt).to(device)
        if wl.wdtype == "bf16":
            self.W1 = torch.from_numpy(wl.W1.view(np.int16)).to(device).view(torch.bfloat16)
            self.W2 = torch.from_numpy(wl.W2.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            self.W1 = torch.from_numpy(wl.W1).to(device)
            self.W2 = torch.from_numpy(wl.W2).to(device)
        self.x0 = torch.from_numpy(wl.x0.astype(np.int32)).to(device)
        self.seeds = torch.from_numpy(wl.seeds.view(np.int64)).to(device).view(torch.uint64) \
            if hasattr(torch, "uint64") else None


def seeds_tensor(seeds, device="cuda"):
    return torch.from_numpy(np.asarray(seeds, dtype=np.uint64).view(np.int64)).to(device).view(torch.uint64)


def f64_weights(wl):
    return oracle.weights_as_f64(wl.W1, wl.wdtype), oracle.weights_as_f64(wl.W2, wl.wdtype)


def close(gpu, ref, rtol, atol):
    return abs(float(gpu) - float(ref)) <= rtol * abs(float(ref)) + atol


def compare_draft(ref, tok, prob, lse, reqs, T):
    """Compare the GPU draft with the oracle's on requests ``reqs``.
    Returns (compared positions, exempt mismatches, set of requests whose whole
    block matched)."""
    compared, exempt, whole = 0, 0, set()
    for b in reqs:
        ok_all = True
        for k in range(tok.shape[1]):
            rt = int(ref["tokens"][b, k])
            if int(tok[b, k]) != rt:
                d = ref["dist"][b, k]
                assert T > 0 and d < EXEMPT_RADIUS, (
                    "draft token mismatch at request %d position %d: gpu %d oracle %d (boundary distance %.3g)"
                    % (b, k + 1, int(tok[b, k]), rt, d))
                exempt += 1
                ok_all = False
                break
            compared += 1
            assert close(prob[b, k], ref["prob"][b, k], PROB_RTOL, PROB_ATOL), (
                "draft_prob request %d position %d: gpu %.9g oracle %.9g" % (b, k + 1, prob[b, k], ref["prob"][b, k]))
            assert close(lse[b, k], ref["lse"][b, k], LSE_RTOL, LSE_ATOL), (
                "draft_lse request %d position %d: gpu %.9g oracle %.9g" % (b, k + 1, lse[b, k], ref["lse"][b, k]))
        if ok_all:
            whole.add(b)
    return compared, exempt, whole


def compare_verify(ref, alen, otok, aprob, reqs, T):
    """Compare the GPU verify outputs with the oracle's on ``reqs``.
    Returns (compared requests, exempt requests)."""
    compared, exempt = 0, 0
    gamma = otok.shape[1] - 1
    for b in reqs:
        same = int(alen[b]) == int(ref["accept_len"][b]) and np.array_equal(otok[b], ref["out_tokens"][b])
        if not same:
            d = ref["min_dist"][b]
            assert T > 0 and d < EXEMPT_RADIUS, (
                "verify mismatch at request %d: gpu n=%d tokens %s, oracle n=%d tokens %s (min boundary distance %.3g)"
                % (b, int(alen[b]), list(otok[b]), int(ref["accept_len"][b]), list(ref["out_tokens"][b]), d))
            exempt += 1
            continue
        compared += 1
        if aprob is not None:
            for k in range(gamma):
                r, g = ref["accept_prob"][b, k], aprob[b, k]
                if np.isnan(r):
                    assert np.isnan(g), "accept_prob request %d position %d should be NaN, got %r" % (b, k + 1, g)
                else:
                    assert close(g, r, PROB_RTOL, PROB_ATOL), (
                        "accept_prob request %d position %d: gpu %.9g oracle %.9g" % (b, k + 1, g, r))
    return compared, exempt


def compare_survival(ref_c, ref_a, cst, surv, reqs):
    for b in reqs:
        for k in range(surv.shape[1]):
            if ref_c is not None and cst is not None:
                assert close(cst[b, k], ref_c[b, k], PROB_RTOL, PROB_ATOL), (
                    "c_star request %d position %d: gpu %.9g oracle %.9g" % (b, k + 1, cst[b, k], ref_c[b, k]))
            assert close(surv[b, k], ref_a[b, k], PROB_RTOL, PROB_ATOL), (
                "survival request %d position %d: gpu %.9g oracle %.9g" % (b, k + 1, surv[b, k], ref_a[b, k]))
