"""Seeded synthetic inputs for the DSpark per-round token path.

This module is the only code shared by the float64 oracle's tests and the HIP
path's tests and benchmark.  It draws data and nothing else: no softmax, no
sampling, no acceptance test.  The one product it forms is the target logits'
"bias" term of the workload recipes (see ``_target_bias``), a data recipe
computed with a numpy matmul.

The five workloads follow the synthetic shapes of the pages' settings: a
Qwen3-scale vocabulary of 151936 and a 262144 vocabulary, Markov rank 256,
block of 7 draft positions, batch from 32 to 512 requests.  No dataset is
used; every array comes from ``numpy.random.default_rng(1000 + index)``,
drawn in a fixed order: U, W1, W2, x0, boosts, target noise, bonus base row.

Readings of the recipes (listed in the design doc):
  * N(0, s) is a normal with standard deviation s;
  * bf16 weights are float32 normals rounded to bf16 (nearest, ties to even)
    and are handed out as uint16 bit patterns;
  * "k tokens boosted +c" adds c at k distinct random ids of each (b, k) row;
  * the target's bias term is the Markov bias along a generator-chosen prefix
    g (g_0 = anchor, g_k = argmax of U_k), standing in for the drafted prefix
    the target would see;
  * the greedy workload's boosted token is set 2 above the row maximum, so it
    is the draft argmax; the target copies it with probability 0.8;
  * per-request Philox keys are word 0 of Philox4x64-10 under key
    (master, 1) at counter (b, 0, 0, 0), drawn with numpy's own Philox.
"""

import dataclasses

import numpy as np

# name -> recipe.  Index order is the order of the workload list.
WORKLOADS = {
    "tiny_v1000_b4": dict(index=0, V=1000, r=16, gamma=4, B=4, T=1.0, wdtype="f32",
                          w_std=0.1, u_std=2.0, boosts=0, boost=0.0,
                          tgt="u_noise", noise=0.5),
    "v151936_b32": dict(index=1, V=151936, r=256, gamma=7, B=32, T=1.0, wdtype="bf16",
                        w_std=0.02, u_std=3.0, boosts=3, boost=8.0,
                        tgt="u_bias_noise", noise=1.0),
    "v151936_b256_t07": dict(index=2, V=151936, r=256, gamma=7, B=256, T=0.7,
                             wdtype="bf16", w_std=0.02, u_std=3.0, boosts=3,
                             boost=8.0, tgt="u_bias_noise", noise=1.0),
    "greedy_v151936_b512": dict(index=3, V=151936, r=256, gamma=7, B=512, T=0.0,
                                wdtype="bf16", w_std=0.02, u_std=3.0, boosts=1,
                                boost=None, tgt="greedy_agree", noise=1.0,
                                agree=0.8),
    "v262144_b128": dict(index=4, V=262144, r=256, gamma=7, B=128, T=1.0, wdtype="bf16",
                         w_std=0.02, u_std=3.0, boosts=5, boost=6.0,
                         tgt="u_bias_noise", noise=1.5),
}

NAMES = list(WORKLOADS)


@dataclasses.dataclass
class Workload:
    name: str
    V: int
    r: int
    gamma: int
    B: int
    T: float
    wdtype: str          # "bf16" (W as uint16 bit patterns) or "f32"
    U: np.ndarray        # [B][gamma][V] float32 base logits
    W1: np.ndarray       # [V][r]
    W2: np.ndarray       # [r][V]
    x0: np.ndarray       # [B] int32 anchors
    tgt: np.ndarray      # [B][gamma+1][V] float32 target logits
    seeds: np.ndarray    # [B] uint64 per-request Philox keys
    rnd: int             # round counter used for the draws

    @property
    def nbytes(self):
        return sum(a.nbytes for a in (self.U, self.W1, self.W2, self.x0, self.tgt, self.seeds))


def f32_to_bf16_bits(x):
    """Round float32 to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def request_seeds(master, B):
    """Per-request keys: word 0 of Philox4x64-10, key (master, 1), counter (b,0,0,0).
    numpy's Philox bumps its counter before producing a block, so it starts one
    below the wanted counter (with borrow through all four words)."""
    out = np.empty(B, dtype=np.uint64)
    for b in range(B):
        c = (b - 1) % (1 << 256)
        ctr = np.array([(c >> (64 * i)) & ((1 << 64) - 1) for i in range(4)], dtype=np.uint64)
        g = np.random.Philox(counter=ctr, key=np.array([master, 1], dtype=np.uint64))
        out[b] = g.random_raw(1)[0]
    return out


def _normal(rng, shape, std):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _distinct_ids(rng, rows, k, V):
    """k distinct ids in [0, V) for each of ``rows`` rows."""
    ids = rng.integers(0, V, size=(rows, k))
    for i in range(rows):
        while len(set(ids[i].tolist())) < k:
            ids[i] = rng.integers(0, V, size=k)
    return ids


def _target_bias(W1f, W2f, prefix):
    """Data recipe of the target logits' bias term: row prefix of W1 times W2,
    float32 numpy matmul (prefix: [n] token ids)."""
    return W1f[prefix] @ W2f


def make(name, *, B=None, V=None, gamma=None, r=None, T=None, w_std=None,
         master_seed=0, rnd=1):
    """Build one workload.  Keyword overrides shrink or reshape the recipe (for
    the oracle-sized parity cases) without changing its draw order."""
    spec = dict(WORKLOADS[name])
    for key, val in (("B", B), ("V", V), ("gamma", gamma), ("r", r), ("T", T), ("w_std", w_std)):
        if val is not None:
            spec[key] = val
    Bn, Vn, G, R = spec["B"], spec["V"], spec["gamma"], spec["r"]
    rng = np.random.default_rng(1000 + spec["index"])

    U = _normal(rng, (Bn, G, Vn), spec["u_std"])
    W1f = _normal(rng, (Vn, R), spec["w_std"])
    W2f = _normal(rng, (R, Vn), spec["w_std"])
    if spec["wdtype"] == "bf16":
        W1, W2 = f32_to_bf16_bits(W1f), f32_to_bf16_bits(W2f)
        W1f, W2f = bf16_bits_to_f32(W1), bf16_bits_to_f32(W2)
    else:
        W1, W2 = W1f, W2f
    x0 = rng.integers(0, Vn, size=Bn).astype(np.int32)

    rows = U.reshape(Bn * G, Vn)
    if spec["boosts"]:
        ids = _distinct_ids(rng, Bn * G, spec["boosts"], Vn)
        ridx = np.arange(Bn * G)[:, None]
        if spec["boost"] is None:
            # greedy recipe: the boosted token sits 2 above the row maximum
            rows[ridx[:, 0], ids[:, 0]] = rows.max(axis=1) + np.float32(2.0)
        else:
            rows[ridx, ids] += np.float32(spec["boost"])
    else:
        ids = None

    tgt = np.empty((Bn, G + 1, Vn), dtype=np.float32)
    tgt[:, :G, :] = U
    tgt[:, :G, :] += _normal(rng, (Bn, G, Vn), spec["noise"])
    bonus = _normal(rng, (Bn, Vn), spec["u_std"])
    bonus += _normal(rng, (Bn, Vn), spec["noise"])
    tgt[:, G, :] = bonus

    if spec["tgt"] == "u_bias_noise":
        prefix = np.empty((Bn, G + 1), dtype=np.int64)
        prefix[:, 0] = x0
        prefix[:, 1:] = U.argmax(axis=2)
        for b in range(Bn):
            tgt[b] += _target_bias(W1f, W2f, prefix[b])
    elif spec["tgt"] == "greedy_agree":
        agree = rng.random(size=Bn * G) < spec["agree"]
        other = rng.integers(0, Vn - 1, size=Bn * G)
        drafted = ids[:, 0]
        pick = np.where(agree, drafted, other + (other >= drafted))
        bi, ki = np.divmod(np.arange(Bn * G), G)
        tgt[bi, ki, pick] = tgt[:, :G, :].max(axis=2).reshape(-1) + np.float32(1.0)

    return Workload(name=name, V=Vn, r=R, gamma=G, B=Bn, T=float(spec["T"]),
                    wdtype=spec["wdtype"], U=U, W1=W1, W2=W2, x0=x0, tgt=tgt,
                    seeds=request_seeds(master_seed, Bn), rnd=int(rnd))


def sps_curve(n_max, half, power, ripple=0.0, seed=0):
    """A synthetic profiled throughput table SPS(n), n = 0..n_max, standing in
    for the engine's measured steps-per-second curve over verified tokens:
    1 / (1 + (n / half)^power), optionally times (1 + ripple * noise) with
    noise uniform in [-1, 1] (a jagged curve).  float64."""
    n = np.arange(n_max + 1, dtype=np.float64)
    s = 1.0 / (1.0 + (n / float(half)) ** float(power))
    if ripple:
        s *= 1.0 + ripple * np.random.default_rng(seed).uniform(-1.0, 1.0, size=n.shape)
    return s


def confidence_inputs(B, gamma, d, r, seed=0, spread=1.5):
    """Synthetic inputs of the confidence head: hidden states h ~ N(0, 1)
    [B][gamma][d], head weights w [d + r] ~ N(0, spread / sqrt(d)) (so the
    hidden part of the logit has standard deviation about `spread`) and
    per-position temperatures rising from 0.8 to 1.6 over the block.
    float32."""
    rng = np.random.default_rng(5000 + seed)
    h = _normal(rng, (B, gamma, d), 1.0)
    w = _normal(rng, (d + r,), spread / np.sqrt(d))
    sts = np.linspace(0.8, 1.6, gamma).astype(np.float32)
    return h, w, sts


def rnn_inputs(B, gamma, r, seed=0, gain=1.5, hp_std=0.5):
    """Synthetic inputs of the RNN head: the cell projection's state and token
    columns Wp [3r][2r] ~ N(0, gain / sqrt(2r)) and its hidden-state part hp
    [B][gamma][3r] ~ N(0, hp_std), the share a random hidden state of the
    target would contribute.  float32."""
    rng = np.random.default_rng(5000 + seed)
    Wp = _normal(rng, (3 * r, 2 * r), gain / np.sqrt(2.0 * r))
    hp = _normal(rng, (B, gamma, 3 * r), hp_std)
    return Wp, hp
