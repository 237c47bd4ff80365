"""Plain float64 reference of DSpark's per-round token path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything in ``oracle/``.  It shares no code, header, table or helper
with the HIP library; the two meet only on the seeded inputs of ``workloads``.

Every function follows one passage of the pages (cited by page title and the
section / equation it sits in) and is written for a reader to check by eye:
one request at a time, one position at a time, whole-vocabulary numpy vectors,
float64 throughout.

Sources (page titles):
  [R]  "DSpark: Confidence-Scheduled Speculative Decoding with Semi-Autoregressive
       Generation" technical review (zhongzhuzhou.org), sections "Speculative
       Decoding: Draft, Then Verify", "The Sequential Correction" (Eq. 4),
       "Instantiation 1: The Markov Head" (Eq. 5), "The Confidence Head" (Eq. 8),
       "Deriving the Acceptance-Rate Identity" (Eq. 8a-8c), "The Hardware-Aware
       Prefix Scheduler" (survival products), "Common Questions Answered"
       (greedy decoding), "Putting It All Together" (decode-round pseudocode).
  [E]  "Speculative decoding, from zero to DSpark" (bittide.aicompass.dev),
       section 2 "The loop, and why it's lossless" (residual rule, bonus token).
  [Z]  robotworld.top review (Chinese), section on the confidence head (the
       accept rate clamped to [0, 1]).

Readings where the pages are silent (each listed in the design doc):
  * temperature T divides the summed logits, draft and target alike; T = 0 is
    the argmax limit with the lowest index winning ties;
  * a categorical draw is the inverse CDF: the first v (ascending vocabulary
    order, sequential float64 cumulative sum) with C(v) > u; if rounding leaves
    no such v, the last v with p(v) > 0;
  * the residual norm(max(0, p_t - p_d)) is drawn by rejection against p_t
    (propose v ~ p_t, keep it with probability max(0, 1 - p_d(v)/p_t(v))), at
    most ``max_proposals`` times, then by the inverse CDF of the residual
    itself; both routes have exactly the residual law;
  * the survival products use the analytical acceptance c*_k for every block
    position along the drafted prefix, or given confidences when supplied.
"""

import math

import numpy as np

from . import philox

EXEMPT_RADIUS = 1e-6   # draws closer than this to a decision boundary may differ on the GPU


# ----------------------------------------------------------------------------
# Inputs
# ----------------------------------------------------------------------------

def weights_as_f64(w, wdtype):
    """The exact float64 values of a weight array stored as bf16 bit patterns
    (uint16) or as float32."""
    if wdtype == "bf16":
        bits = np.asarray(w, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if wdtype == "f32":
        return np.asarray(w, dtype=np.float32).astype(np.float64)
    raise ValueError("unknown weight dtype %r" % (wdtype,))


# ----------------------------------------------------------------------------
# Distributions
# ----------------------------------------------------------------------------

def markov_bias(W1, W2, prev):
    """Eq. 5 of [R] ("Instantiation 1: The Markov Head"): the bigram bias row
    B(prev, .) = W1[prev] W2, a length-V vector."""
    return W1[prev] @ W2


def draft_logits(U_row, W1, W2, prev, T):
    """Logits of one draft position, Eq. 4 of [R]: base logits U_k plus the
    Markov bias of the previous token, divided by the temperature (T > 0) or
    left unscaled for the argmax limit (T = 0)."""
    l = np.asarray(U_row, dtype=np.float64) + markov_bias(W1, W2, prev)
    return l / T if T > 0 else l


def position_logits(U, W1, W2, E, b, k, prev, T):
    """Draft logits of block position k (1-based) of request b, as the draft
    produced them: the Markov head's (Eq. 5 of [R], from the previous token
    ``prev``) when E is None, otherwise the RNN head's of [R] "Instantiation
    2: The RNN Head" (Eq. 6), U_k + e_k W2 with e_k = E[b][k-1] the operand
    row the RNN draft used."""
    if E is None:
        return draft_logits(U[b, k - 1], W1, W2, prev, T)
    l = np.asarray(U[b, k - 1], dtype=np.float64) + np.asarray(E[b, k - 1], dtype=np.float64) @ W2
    return l / T if T > 0 else l


def target_logits(tgt_row, T):
    """Target logits of one position, divided by the temperature when T > 0."""
    l = np.asarray(tgt_row, dtype=np.float64)
    return l / T if T > 0 else l


def softmax(l):
    """Exact per-position softmax (the normalised exponential of Eq. 4 of [R]).
    Returns (p, log-normaliser).  -inf logits get probability 0."""
    m = np.max(l)
    e = np.exp(l - m)
    z = e.sum()
    return e / z, m + math.log(z)


def first_argmax(l):
    """argmax with the lowest index winning ties (np.argmax returns the first)."""
    return int(np.argmax(l))


def inverse_cdf(p, u):
    """Categorical draw by inverse CDF: the first v with C(v) > u, where
    C(v) = p(0) + ... + p(v) is summed sequentially in ascending order.
    Returns (v, distance of u to the nearer edge of v's CDF interval)."""
    C = np.cumsum(p)
    v = int(np.searchsorted(C, u, side="right"))
    if v >= len(p):
        v = int(np.flatnonzero(p > 0)[-1])
    lo = C[v - 1] if v > 0 else 0.0
    return v, min(abs(u - lo), abs(C[v] - u))


# ----------------------------------------------------------------------------
# Draft: semi-autoregressive Markov-head sampling
# ----------------------------------------------------------------------------

def markov_draft(U, W1, W2, x0, T, seeds, rnd, requests=None):
    """Sample the gamma block positions of every request left to right
    ([R] "The Sequential Correction", Eq. 4; Markov bias Eq. 5; the decode-round
    pseudocode steps 3-5).  Position k uses the token drawn at k-1, the anchor
    x0 at k = 1.

    U: [B][gamma][V] float32 base logits; W1 [V][r], W2 [r][V] float64 values;
    x0: [B] anchors; seeds: [B] uint64 request keys; rnd: round counter.
    Returns dict with tokens [B][gamma] int32, prob [B][gamma] (p_d^k(x_k)),
    lse [B][gamma] (log-normaliser of the draft logits; 0 at T = 0) and dist
    [B][gamma] (distance of each uniform to its CDF edge; top-2 logit gap at
    T = 0).  Only rows in ``requests`` (default: all) are computed.
    """
    B, gamma, V = U.shape
    reqs = range(B) if requests is None else requests
    tokens = np.full((B, gamma), -1, dtype=np.int32)
    prob = np.full((B, gamma), np.nan)
    lse = np.full((B, gamma), np.nan)
    dist = np.full((B, gamma), np.inf)
    for b in reqs:
        prev = int(x0[b])
        for k in range(1, gamma + 1):
            l = draft_logits(U[b, k - 1], W1, W2, prev, T)
            if T == 0:
                x = first_argmax(l)
                top2 = np.partition(l, -2)[-2:]
                tokens[b, k - 1], prob[b, k - 1], lse[b, k - 1] = x, 1.0, 0.0
                dist[b, k - 1] = top2[1] - top2[0]
            else:
                p, z = softmax(l)
                u = philox.uniform(int(seeds[b]), rnd, k, philox.STREAM_DRAFT)
                x, d = inverse_cdf(p, u)
                tokens[b, k - 1], prob[b, k - 1], lse[b, k - 1] = x, p[x], z
                dist[b, k - 1] = d
            prev = x
    return dict(tokens=tokens, prob=prob, lse=lse, dist=dist)


# ----------------------------------------------------------------------------
# Verify: lossless rejection sampling
# ----------------------------------------------------------------------------

def residual_law(pt, pd):
    """The resampling law at the first rejection, written out as [E] section 2
    states it: norm(max(0, p_t - p_d)), the positive part of the difference
    divided by its total.  When the difference has no positive mass (which a
    rejection rules out in exact arithmetic) the law is p_t."""
    res = np.maximum(0.0, np.asarray(pt, dtype=np.float64) - np.asarray(pd, dtype=np.float64))
    mass = res.sum()
    return res / mass if mass > 0 else np.asarray(pt, dtype=np.float64)


def residual_sample(pt, pd, seed, rnd, j, max_proposals, dists):
    """Draw from norm(max(0, p_t - p_d)), the resampling law at the first
    rejection ([E] section 2).

    Rejection against p_t: proposal i takes words 0 and 1 of the stream-2
    block (rnd, j, 2, i); v ~ p_t by inverse CDF, kept iff
    u_acc < max(0, 1 - p_d(v)/p_t(v)).  One round keeps v with probability
    max(0, p_t(v) - p_d(v)), so a kept v follows the residual law.  After
    ``max_proposals`` misses the residual itself is drawn by inverse CDF with
    stream 3; if it has no mass (possible only by rounding) p_t is used.
    Appends every boundary distance to ``dists``.
    """
    for i in range(max_proposals):
        w = philox.block(seed, rnd, j, philox.STREAM_RESIDUAL, i)
        u_prop, u_acc = philox.to_uniform(w[0]), philox.to_uniform(w[1])
        v, d = inverse_cdf(pt, u_prop)
        dists.append(d)
        keep = max(0.0, 1.0 - pd[v] / pt[v])
        dists.append(abs(u_acc - keep))
        if u_acc < keep:
            return v
    res = np.maximum(0.0, pt - pd)
    mass = res.sum()
    u = philox.uniform(seed, rnd, j, philox.STREAM_FALLBACK)
    v, d = inverse_cdf(res / mass if mass > 0 else pt, u)
    dists.append(d)
    return v


def verify(U, W1, W2, x0, draft_tokens, tgt, T, seeds, rnd, max_proposals=64,
           requests=None, lengths=None, E=None):
    """Rejection-sampling verification of every request's drafted block
    ([R] "Speculative Decoding: Draft, Then Verify" step 3; [E] section 2).

    Left to right, x_k is accepted with probability
    alpha_k = min(1, p_t^k(x_k) / p_d^k(x_k)) (accept iff u < alpha_k, u from
    stream 1).  The first rejection at j emits a residual draw and stops; if
    all gamma positions pass, a bonus token is drawn from the target row
    gamma+1 (stream 2, index 0).  At T = 0 acceptance is the exact match
    x_k == argmax tgt_k and the correction / bonus is the target argmax
    ([R] "Common Questions Answered", greedy decoding).

    tgt: [B][gamma+1][V].  p_d^k is recomputed here from U, W1, W2 and the
    drafted prefix.  Returns dict: accept_len [B] (n), out_tokens [B][gamma+1]
    (x_1..x_n, y, -1...), accept_prob [B][gamma] (alpha_k of tested positions,
    NaN after), min_dist [B] (smallest boundary distance of all draws of the
    request; inf at T = 0).

    ``lengths`` ([B], optional): the scheduled verification lengths l_b of
    [R] "The Hardware-Aware Prefix Scheduler" (Algorithm 1).  Only x_1..x_l
    are offered to the target; if all of them pass, the bonus token comes
    from the target row l+1 (stream 2 at position l+1, index 0), so l = 0
    emits one token drawn from p_t^1 (plain decoding) and l = gamma is the
    full block.

    ``E`` ([B][gamma][r], optional): the operand rows e_k of an RNN draft
    ([R] "Instantiation 2: The RNN Head", Eq. 6; ``rnn_draft`` returns them).
    p_d^k is then softmax((U_k + e_k W2) / T), the law the RNN head drew x_k
    from, in place of the Markov head's (the decode round of [R] "Putting It
    All Together" feeds either head's draft to verification).
    """
    B, gamma, V = U.shape
    reqs = range(B) if requests is None else requests
    accept_len = np.full(B, -1, dtype=np.int32)
    out_tokens = np.full((B, gamma + 1), -1, dtype=np.int32)
    accept_prob = np.full((B, gamma), np.nan)
    min_dist = np.full(B, np.inf)
    for b in reqs:
        seed = int(seeds[b])
        prev = int(x0[b])
        dists = []
        emitted = []
        ell = gamma if lengths is None else int(lengths[b])
        n = ell
        for k in range(1, ell + 1):
            x = int(draft_tokens[b, k - 1])
            lt = target_logits(tgt[b, k - 1], T)
            if T == 0:
                y = first_argmax(lt)
                accept_prob[b, k - 1] = 1.0 if y == x else 0.0
                if y == x:
                    emitted.append(x)
                    prev = x
                    continue
                emitted.append(y)
                n = k - 1
                break
            pd, _ = softmax(position_logits(U, W1, W2, E, b, k, prev, T))
            pt, _ = softmax(lt)
            alpha = min(1.0, pt[x] / pd[x])
            accept_prob[b, k - 1] = alpha
            u = philox.uniform(seed, rnd, k, philox.STREAM_ACCEPT)
            dists.append(abs(u - alpha))
            if u < alpha:
                emitted.append(x)
                prev = x
                continue
            emitted.append(residual_sample(pt, pd, seed, rnd, k, max_proposals, dists))
            n = k - 1
            break
        if n == ell:
            lt = target_logits(tgt[b, ell], T)
            if T == 0:
                emitted.append(first_argmax(lt))
            else:
                pt, _ = softmax(lt)
                u = philox.uniform(seed, rnd, ell + 1, philox.STREAM_RESIDUAL)
                y, d = inverse_cdf(pt, u)
                dists.append(d)
                emitted.append(y)
        accept_len[b] = n
        out_tokens[b, :len(emitted)] = emitted
        min_dist[b] = min(dists) if dists else np.inf
    return dict(accept_len=accept_len, out_tokens=out_tokens,
                accept_prob=accept_prob, min_dist=min_dist)


# ----------------------------------------------------------------------------
# Survival products
# ----------------------------------------------------------------------------

def acceptance_rate(pd, pt):
    """Analytical acceptance of one position, Eq. 8a of [R]:
    sum_v min(p_d(v), p_t(v)), clamped to [0, 1] as the accept-rate label is in
    [Z]."""
    return min(1.0, max(0.0, float(np.minimum(pd, pt).sum())))


def survival(U, W1, W2, x0, draft_tokens, tgt, T, conf=None, requests=None, E=None):
    """Prefix survival a_{b,k} = prod_{i<=k} c_{b,i} ([R] "The Hardware-Aware
    Prefix Scheduler", step 1 of Algorithm 1).

    With ``conf`` ([B][gamma]) the products are taken of the given
    confidences.  Otherwise c_{b,k} is the analytical acceptance c*_k of Eq. 8
    at every block position along the drafted prefix (all gamma positions,
    also those after a rejection); at T = 0 it is the indicator
    x_k == argmax tgt_k.  With ``E`` (the operand rows of an RNN draft, as in
    ``verify``) p_d^k is the RNN head's law.  Returns (c_star [B][gamma] or
    None, survival).
    """
    if conf is not None:
        conf = np.asarray(conf, dtype=np.float64)
        return None, np.cumprod(conf, axis=1)
    B, gamma, V = U.shape
    reqs = range(B) if requests is None else requests
    c = np.full((B, gamma), np.nan)
    for b in reqs:
        prev = int(x0[b])
        for k in range(1, gamma + 1):
            x = int(draft_tokens[b, k - 1])
            lt = target_logits(tgt[b, k - 1], T)
            if T == 0:
                c[b, k - 1] = 1.0 if first_argmax(lt) == x else 0.0
            else:
                pd, _ = softmax(position_logits(U, W1, W2, E, b, k, prev, T))
                pt, _ = softmax(lt)
                c[b, k - 1] = acceptance_rate(pd, pt)
            prev = x
    return c, np.cumprod(c, axis=1)


# ----------------------------------------------------------------------------
# Hardware-aware prefix scheduler
# ----------------------------------------------------------------------------

def schedule(a, sps, early_stop=True, trace=None):
    """Algorithm 1 of [R] "The Hardware-Aware Prefix Scheduler": per-request
    verification lengths that maximise Theta = tau * SPS(B).

    a: [R][gamma] prefix survival probabilities a_{r,j} (non-increasing in j);
    sps: SPS(n) for n = 0, 1, ... (at least R (gamma + 1) + 1 entries), the
    profiled throughput at n verified tokens.  Every (r, j) with a_{r,j} > 0
    is a candidate; candidates are taken in descending a, ties to the lowest
    request id ([R] "Common Questions Answered"), then the lowest position.
    Starting from l = 0, B = R, tau = R, each candidate sets l_r = j and adds
    one token to B and a_{r,j} to tau; Theta = tau * SPS(B) is kept as the
    new best while it improves, and the scan stops at the first candidate
    that does not improve it (the non-anticipating early stop of "The
    Non-Anticipating Property").  ``early_stop=False`` scans every candidate
    and keeps the global best: the anticipating variant the pages show to be
    lossy, here only as a test of that claim.

    Returns (lengths [R] int, Theta_best, margin): margin is the smallest
    |Theta - Theta_best| over the comparisons made (a decision closer than
    rounding may differ on the GPU).  With a list ``trace``, every admitted
    candidate appends (r, j, B, tau, Theta), r and j 1-based as on the pages.
    """
    a = np.asarray(a, dtype=np.float64)
    R, gamma = a.shape
    pool = [(a[r, j], r, j + 1) for r in range(R) for j in range(gamma) if a[r, j] > 0]
    pool.sort(key=lambda e: (-e[0], e[1], e[2]))
    cur = [0] * R
    size = R
    tau = float(R)
    best = tau * float(sps[size])
    best_len = list(cur)
    margin = math.inf
    for val, r, j in pool:
        cur[r] = j
        size += 1
        tau += val
        theta = tau * float(sps[size])
        if trace is not None:
            trace.append((r + 1, j, size, tau, theta))
        margin = min(margin, abs(theta - best))
        if theta > best:
            best = theta
            best_len = list(cur)
        elif early_stop:
            break
    return np.array(best_len, dtype=np.int32), best, margin


# ----------------------------------------------------------------------------
# Confidence head
# ----------------------------------------------------------------------------

def confidence(h, w, W1, x0, draft_tokens, sts=None, requests=None):
    """Per-position confidence of Eq. 7 of [R] ("The Confidence Head"):
    c_k = sigma(w . [h_k ; W1[x_{k-1}]]), with x_0 the anchor, followed by the
    per-position temperature of Sequential Temperature Scaling (the same
    section): the logit is divided by the calibrated temperature of position k
    (temperature scaling of a sigmoid), c_k = sigma(z_k / t_k).

    h: [B][gamma][d] hidden states; w: [d + r] head weights (hidden part
    first); W1: [V][r] float64 Markov embedding; sts: [gamma] temperatures
    (None: 1).  Returns c [B][gamma] in float64 (NaN for requests not in
    ``requests``).
    """
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, gamma, d = h.shape
    reqs = range(B) if requests is None else requests
    c = np.full((B, gamma), np.nan)
    for b in reqs:
        prev = int(x0[b])
        for k in range(1, gamma + 1):
            z = float(w[:d] @ h[b, k - 1]) + float(w[d:] @ W1[prev])
            t = 1.0 if sts is None else float(sts[k - 1])
            c[b, k - 1] = 1.0 / (1.0 + math.exp(-z / t))
            prev = int(draft_tokens[b, k - 1])
    return c


def schedule_capacity(a, sps):
    """The capacity K of the asynchronous adaptation in [R] "The Asynchronous
    Fix, and Why It Stays Lossless": the unconstrained search over the whole
    sorted scan of Algorithm 1 (no early stop, so a jagged SPS curve cannot
    trap it), run on survival products from two steps earlier.  K is the
    number of draft-token admissions at the first maximum of Theta (0: none).
    Returns (K, Theta at K)."""
    a = np.asarray(a, dtype=np.float64)
    lengths, best, _ = schedule(a, sps, early_stop=False)
    return int(lengths.sum()), best


def admit_top(a, K):
    """The live half of the asynchronous adaptation (same section): the
    current candidates, in Algorithm 1's order (descending a_{r,j}, ties to
    the lowest request, then position, a > 0 only), fill the K admissions
    decided earlier.  Returns the per-request lengths (largest admitted
    position)."""
    a = np.asarray(a, dtype=np.float64)
    R, gamma = a.shape
    pool = [(a[r, j], r, j + 1) for r in range(R) for j in range(gamma) if a[r, j] > 0]
    pool.sort(key=lambda e: (-e[0], e[1], e[2]))
    lengths = np.zeros(R, dtype=np.int32)
    for _, r, j in pool[:max(0, int(K))]:
        lengths[r] = max(lengths[r], j)
    return lengths


# ----------------------------------------------------------------------------
# RNN head (the second sequential block)
# ----------------------------------------------------------------------------

def round_to_bf16(x):
    """Nearest bfloat16 value (8 significant bits, ties to even) of float64
    values, returned as float64.  Applied once to the float64 value itself
    (no intermediate float32)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0) / 256.0, e)   # numpy rounds halves to even


def rnn_draft(U, W1, W2, Wp, h, x0, T, seeds, rnd, bf16_operand=False, forced=None, requests=None, hp=None):
    """Block sampling with the RNN head of [R] "Instantiation 2: The RNN Head"
    (Eq. 6) in place of the Markov bias: per request, s_0 = 0 and for
    k = 1..gamma
        z_k = [s_{k-1} ; W1[x_{k-1}] ; h_k]          (x_0 = the anchor)
        (g, c, o) = Wp z_k                           (Wp: [3r][2r + d], rows
                                                      gate, candidate, output)
        s_k = sigma(g) s_{k-1} + (1 - sigma(g)) tanh(c)
        e_k = tanh(o);  bias_k = e_k W2;  p_d^k = softmax((U_k + bias_k) / T)
    then x_k is drawn as in markov_draft (same stream-0 uniforms), or taken
    from ``forced`` [B][gamma] when given (for evaluating block laws).

    ``hp`` ([B][gamma][3r], optional) is the hidden part W_p[:, 2r:] h_k given
    precomputed (it depends on no drafted token, so the parallel stage can
    produce it); ``Wp`` then needs only its first 2r columns and ``h`` is not
    read.  Everything is float64; e_k enters the projection unrounded.  With
    ``bf16_operand`` it is first rounded to bf16, as a model that keeps its
    activations in bf16 would (an alternative reading, kept as an option).  Returns dict with tokens, prob, lse, dist as
    markov_draft and E [B][gamma][r], the operand rows e_k used.
    """
    U = np.asarray(U)
    B, gamma, V = U.shape
    r = W1.shape[1]
    reqs = range(B) if requests is None else requests
    tokens = np.full((B, gamma), -1, dtype=np.int32)
    prob = np.full((B, gamma), np.nan)
    lse = np.full((B, gamma), np.nan)
    dist = np.full((B, gamma), np.inf)
    E = np.full((B, gamma, r), np.nan)
    for b in reqs:
        prev = int(x0[b])
        state = np.zeros(r)
        for k in range(1, gamma + 1):
            if hp is None:
                z = np.concatenate([state, W1[prev], np.asarray(h[b, k - 1], dtype=np.float64)])
                proj = Wp @ z
            else:
                z = np.concatenate([state, W1[prev]])
                proj = np.asarray(Wp, dtype=np.float64)[:, :2 * r] @ z + np.asarray(hp[b, k - 1], dtype=np.float64)
            g, c, o = proj[:r], proj[r:2 * r], proj[2 * r:]
            gate = 1.0 / (1.0 + np.exp(-g))
            e = np.tanh(o)
            if bf16_operand:
                e = round_to_bf16(e)
            E[b, k - 1] = e
            l = np.asarray(U[b, k - 1], dtype=np.float64) + e @ W2
            if T > 0:
                l = l / T
            state = gate * state + (1.0 - gate) * np.tanh(c)
            if T == 0:
                x = first_argmax(l) if forced is None else int(forced[b, k - 1])
                top2 = np.partition(l, -2)[-2:]
                tokens[b, k - 1], prob[b, k - 1], lse[b, k - 1] = x, 1.0, 0.0
                dist[b, k - 1] = top2[1] - top2[0]
            else:
                p, zl = softmax(l)
                if forced is None:
                    u = philox.uniform(int(seeds[b]), rnd, k, philox.STREAM_DRAFT)
                    x, d = inverse_cdf(p, u)
                else:
                    x, d = int(forced[b, k - 1]), np.inf
                tokens[b, k - 1], prob[b, k - 1], lse[b, k - 1] = x, p[x], zl
                dist[b, k - 1] = d
            prev = x
    return dict(tokens=tokens, prob=prob, lse=lse, dist=dist, E=E)
