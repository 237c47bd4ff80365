"""The float64 oracle over many requests at once, for the full-size parity
cases: worker processes (spawned, never forked from a process that holds a
GPU context), one BLAS thread each, reading the workload's arrays from
memory-mapped .npy files in /dev/shm instead of receiving copies.

Only test code uses this module; it calls nothing but ``oracle``.
"""

import multiprocessing
import os
import shutil
import tempfile

import numpy as np

_W = {}


def _init(folder, T, rnd, wdtype):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass
    import oracle
    ld = lambda n: np.load(os.path.join(folder, n + ".npy"), mmap_mode="r")
    _W.update(U=ld("U"), tgt=ld("tgt"), x0=ld("x0"), seeds=ld("seeds"), T=T, rnd=rnd)
    _W["W1"] = oracle.weights_as_f64(ld("W1"), wdtype)
    _W["W2"] = oracle.weights_as_f64(ld("W2"), wdtype)


def _draft(b):
    import oracle
    w = _W
    r = oracle.markov_draft(w["U"], w["W1"], w["W2"], w["x0"], w["T"], w["seeds"], w["rnd"], requests=[b])
    return b, {k: v[b].copy() for k, v in r.items()}


def _verify(task):
    import oracle
    b, tokens = task
    w = _W
    B, gamma = w["U"].shape[:2]
    tok = np.full((B, gamma), -1, dtype=np.int32)
    tok[b] = tokens
    r = oracle.verify(w["U"], w["W1"], w["W2"], w["x0"], tok, w["tgt"], w["T"], w["seeds"], w["rnd"], requests=[b])
    return b, {k: v[b].copy() for k, v in r.items()}


def _survival(task):
    import oracle
    b, tokens = task
    w = _W
    B, gamma = w["U"].shape[:2]
    tok = np.full((B, gamma), -1, dtype=np.int32)
    tok[b] = tokens
    c, a = oracle.survival(w["U"], w["W1"], w["W2"], w["x0"], tok, w["tgt"], w["T"], requests=[b])
    return b, {"c_star": c[b].copy(), "survival": a[b].copy()}


class OraclePool:
    """with OraclePool(wl) as pool: pool.draft(reqs), pool.verify(reqs, tokens),
    pool.survival(reqs, tokens)."""

    def __init__(self, wl, workers=None):
        self.wl = wl
        self.workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
        base = "/dev/shm" if os.path.isdir("/dev/shm") else None
        self.folder = tempfile.mkdtemp(prefix="dspark_oracle_", dir=base)
        for name in ("U", "tgt", "x0", "seeds", "W1", "W2"):
            np.save(os.path.join(self.folder, name + ".npy"), np.ascontiguousarray(getattr(wl, name)))
        ctx = multiprocessing.get_context("spawn")
        self.pool = ctx.Pool(self.workers, initializer=_init, initargs=(self.folder, wl.T, wl.rnd, wl.wdtype))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def close(self):
        if self.pool is not None:
            self.pool.terminate()
            self.pool.join()
            self.pool = None
        if self.folder and os.path.isdir(self.folder):
            shutil.rmtree(self.folder, ignore_errors=True)
            self.folder = None

    def _merge(self, results, shapes):
        out = {k: np.full(shape, fill, dtype=dt) for k, (shape, fill, dt) in shapes.items()}
        for b, r in results:
            for k in out:
                out[k][b] = r[k]
        return out

    def draft(self, reqs):
        B, gamma = self.wl.B, self.wl.gamma
        res = self.pool.map(_draft, list(reqs), chunksize=1)
        return self._merge(res, {"tokens": ((B, gamma), -1, np.int32), "prob": ((B, gamma), np.nan, np.float64),
                                 "lse": ((B, gamma), np.nan, np.float64), "dist": ((B, gamma), np.inf, np.float64)})

    def verify(self, reqs, tokens):
        B, gamma = self.wl.B, self.wl.gamma
        res = self.pool.map(_verify, [(b, np.asarray(tokens[b], dtype=np.int32)) for b in reqs], chunksize=1)
        return self._merge(res, {"accept_len": ((B,), -1, np.int32), "out_tokens": ((B, gamma + 1), -1, np.int32),
                                 "accept_prob": ((B, gamma), np.nan, np.float64),
                                 "min_dist": ((B,), np.inf, np.float64)})

    def survival(self, reqs, tokens):
        """(c_star, survival) of the analytical mode, [B][gamma] each (NaN
        outside ``reqs``)."""
        B, gamma = self.wl.B, self.wl.gamma
        res = self.pool.map(_survival, [(b, np.asarray(tokens[b], dtype=np.int32)) for b in reqs], chunksize=1)
        out = self._merge(res, {"c_star": ((B, gamma), np.nan, np.float64),
                                "survival": ((B, gamma), np.nan, np.float64)})
        return out["c_star"], out["survival"]
