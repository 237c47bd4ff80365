"""Python binding of libdspark: DSpark's per-round token path on MI355X.

Thin ctypes marshalling over the C ABI declared in ``include/dspark.h``:
every step of the path runs in the library's HIP kernels; this module only
checks tensor metadata, passes device pointers and the current HIP stream,
and raises on a non-zero status.  PyTorch provides device memory and streams.

Functions (same names as the C entry points, without the ``dspark_`` prefix):
  markov_bias, markov_draft, verify, survival, workspace_size, version.
"""

import ctypes
import os

import torch

__all__ = [
    "DsparkError", "OP_DRAFT", "OP_VERIFY", "OP_SURVIVAL", "OP_RNN_DRAFT", "MAX_RESIDUAL_PROPOSALS",
    "SCHEDULE_EARLY_STOP", "SCHEDULE_CAPACITY", "SCHEDULE_TOP_K",
    "library_path", "load", "version", "workspace_size", "markov_bias",
    "markov_draft", "markov_draft_noalloc", "static_scratch_bytes", "rnn_draft", "verify", "transpose_w2", "survival", "confidence", "schedule", "profile_enable",
    "profile_read",
]

OP_DRAFT, OP_VERIFY, OP_SURVIVAL, OP_RNN_DRAFT = 0, 1, 2, 3
SCHEDULE_EARLY_STOP, SCHEDULE_CAPACITY, SCHEDULE_TOP_K = 0, 1, 2
_F32, _BF16 = 0, 1
MAX_RESIDUAL_PROPOSALS = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class DsparkError(RuntimeError):
    def __init__(self, func, status, message):
        super().__init__("%s failed: %s (status %d)" % (func, message, status))
        self.status = status


def library_path():
    return os.path.join(_HERE, "libdspark.so")


def load():
    """Load libdspark.so (built in-tree by ``python -m draft_sampling_verification_bias_amd.build``)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError("libdspark.so is not built (%s); run "
                           "`python -m draft_sampling_verification_bias_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, I, F, U64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint64, ctypes.c_size_t
    lib.dspark_version.restype = I
    lib.dspark_version.argtypes = []
    lib.dspark_status_string.restype = ctypes.c_char_p
    lib.dspark_status_string.argtypes = [I]
    lib.dspark_workspace_size.restype = SZ
    lib.dspark_workspace_size.argtypes = [I, I, I, I, I]
    lib.dspark_markov_bias.restype = I
    lib.dspark_markov_bias.argtypes = [P, P, I, P, I, I, I, P, P]
    lib.dspark_markov_draft.restype = I
    lib.dspark_markov_draft.argtypes = [P, P, P, P, I, P, I, I, I, I, F, P, U64, P, P, P, P, P, P, I, P, P, SZ, P]
    lib.dspark_markov_draft_noalloc.restype = I
    lib.dspark_markov_draft_noalloc.argtypes = [P, P, P, P, I, P, I, I, I, I, F, P, U64, P, P, P, P, P, P, I, P, P]
    lib.dspark_static_scratch_bytes.restype = SZ
    lib.dspark_static_scratch_bytes.argtypes = []
    lib.dspark_rnn_draft.restype = I
    lib.dspark_rnn_draft.argtypes = [P, P, P, I, P, P, P, I, I, I, I, F, P, U64, P, P, P, P, P, SZ, P]
    lib.dspark_verify.restype = I
    lib.dspark_verify.argtypes = [P, P, P, P, I, P, P, P, P, P, P, I, I, I, I, F, P, U64, P, P, P, P, SZ, P]
    lib.dspark_confidence.restype = I
    lib.dspark_confidence.argtypes = [P, P, P, I, P, P, P, I, I, I, I, I, P, P]
    lib.dspark_schedule.restype = I
    lib.dspark_schedule.argtypes = [P, P, I, I, I, I, P, P, P, P, P]
    lib.dspark_transpose_w2.restype = I
    lib.dspark_transpose_w2.argtypes = [P, I, I, I, P, P]
    lib.dspark_survival.restype = I
    lib.dspark_survival.argtypes = [P, P, P, I, P, P, P, P, P, P, I, I, I, I, F, P, P, P, SZ, P]
    lib.dspark_profile_enable.restype = I
    lib.dspark_profile_enable.argtypes = [I]
    lib.dspark_profile_kinds.restype = I
    lib.dspark_profile_kinds.argtypes = []
    lib.dspark_profile_get.restype = I
    lib.dspark_profile_get.argtypes = [I, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_longlong),
                                       ctypes.POINTER(ctypes.c_double)]
    _LIB = lib
    return lib


def version():
    return load().dspark_version()


def workspace_size(op, B, gamma, V, r):
    return int(load().dspark_workspace_size(op, B, gamma, V, r))


def profile_enable(on=True):
    """Start (clearing earlier records) or stop per-kernel HIP-event timing."""
    _check("dspark_profile_enable", load().dspark_profile_enable(1 if on else 0))


def profile_read():
    """{kernel name: (launches, total milliseconds)} of the recorded launches."""
    lib = load()
    out = {}
    for kind in range(lib.dspark_profile_kinds()):
        name, n, ms = ctypes.c_char_p(), ctypes.c_longlong(), ctypes.c_double()
        _check("dspark_profile_get", lib.dspark_profile_get(kind, ctypes.byref(name), ctypes.byref(n),
                                                            ctypes.byref(ms)))
        if n.value:
            out[name.value.decode()] = (int(n.value), float(ms.value))
    return out


def _check(func, status):
    if status != 0:
        msg = load().dspark_status_string(status).decode()
        raise DsparkError(func, status, msg)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t


def _wdtype(W1, W2):
    if W1.dtype != W2.dtype:
        raise ValueError("W1 and W2 must share a dtype")
    if W1.dtype == torch.bfloat16:
        return _BF16
    if W1.dtype == torch.float32:
        return _F32
    raise ValueError("weights must be bfloat16 or float32, got %s" % W1.dtype)


def _stream(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(op, B, gamma, V, r, workspace, device):
    need = workspace_size(op, B, gamma, V, r)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    _dev(workspace, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def markov_bias(W1, W2, tokens, out=None, stream=None):
    """out[i] = W1[tokens[i]] @ W2 (float32 [n][V])."""
    V, r = W1.shape
    _dev(W1, "W1")
    _dev(W2, "W2", W1.dtype, (r, V))
    _dev(tokens, "tokens", torch.int32)
    n = tokens.numel()
    if out is None:
        out = torch.empty((n, V), dtype=torch.float32, device=W1.device)
    _dev(out, "out", torch.float32, (n, V))
    st = load().dspark_markov_bias(_p(W1), _p(W2), _wdtype(W1, W2), _p(tokens), n, V, r, _p(out),
                                   _stream(stream, W1.device))
    _check("dspark_markov_bias", st)
    return out


def _draft_outputs(U, W1, W2, x0, seeds, out, conf_head, W2T):
    """Checks the draft's arguments; returns (B, gamma, V, r, outputs, conf args)."""
    B, gamma, V = U.shape
    r = W1.shape[1]
    dev = U.device
    _dev(U, "U", torch.float32)
    _dev(W1, "W1", None, (V, r))
    _dev(W2, "W2", W1.dtype, (r, V))
    _dev(x0, "x0", torch.int32, (B,))
    if seeds is not None:
        _dev(seeds, "seeds", torch.uint64, (B,))
    if W2T is not None:
        _dev(W2T, "W2T", W2.dtype, (V, r))
    n = 3 if conf_head is None else 4
    if out is None:
        out = tuple(torch.empty((B, gamma), dtype=torch.int32 if i == 0 else torch.float32, device=dev)
                    for i in range(n))
    if len(out) != n:
        raise ValueError("out needs %d tensors" % n)
    for t, name, dt in zip(out, ("draft_tokens", "draft_prob", "draft_lse", "conf"),
                           (torch.int32, torch.float32, torch.float32, torch.float32)):
        _dev(t, name, dt, (B, gamma))
    cargs = (None, None, None, 0, None)
    if conf_head is not None:
        h, w, sts = conf_head
        d = h.shape[2]
        _dev(h, "conf h", torch.float32, (B, gamma, d))
        _dev(w, "conf w", torch.float32, (d + r,))
        if sts is not None:
            _dev(sts, "sts", torch.float32, (gamma,))
        cargs = (_p(h), _p(w), _p(sts), d, _p(out[3]))
    return B, gamma, V, r, out, cargs


def markov_draft(U, W1, W2, x0, temperature, seeds, rnd, out=None, workspace=None, stream=None, W2T=None,
                 conf_head=None):
    """Draft gamma tokens per request.  Returns (draft_tokens, draft_prob,
    draft_lse), and the confidences as a fourth tensor when ``conf_head`` =
    (h [B][gamma][d], w [d + r], sts [gamma] or None) is given (the
    confidence head, computed inside the draft's selections).
    W2T: optional transposed copy of W2 (transpose_w2), which lets the library
    run all positions in one device-resident launch."""
    B, gamma, V, r, out, cargs = _draft_outputs(U, W1, W2, x0, seeds, out, conf_head, W2T)
    dev = U.device
    ws, nbytes = _workspace(OP_DRAFT, B, gamma, V, r, workspace, dev)
    st = load().dspark_markov_draft(_p(U), _p(W1), _p(W2), _p(W2T), _wdtype(W1, W2), _p(x0), B, gamma, V, r,
                                    float(temperature), _p(seeds), int(rnd), _p(out[0]), _p(out[1]), _p(out[2]),
                                    *cargs, _p(ws), nbytes, _stream(stream, dev))
    _check("dspark_markov_draft", st)
    return out


def markov_draft_noalloc(U, W1, W2, x0, temperature, seeds, rnd, out=None, stream=None, W2T=None,
                         conf_head=None):
    """markov_draft with the library's static scratch array instead of a
    workspace (dspark_markov_draft_noalloc).  Returns what markov_draft
    returns; pass ``out`` to allocate nothing here either."""
    B, gamma, V, r, out, cargs = _draft_outputs(U, W1, W2, x0, seeds, out, conf_head, W2T)
    st = load().dspark_markov_draft_noalloc(_p(U), _p(W1), _p(W2), _p(W2T), _wdtype(W1, W2), _p(x0), B, gamma, V, r,
                                            float(temperature), _p(seeds), int(rnd), _p(out[0]), _p(out[1]),
                                            _p(out[2]), *cargs, _stream(stream, U.device))
    _check("dspark_markov_draft_noalloc", st)
    return out


def static_scratch_bytes():
    return int(load().dspark_static_scratch_bytes())


def rnn_draft(U, W1, W2, Wp, hp, x0, temperature, seeds, rnd, out=None, with_e=False, workspace=None,
              stream=None):
    """Draft gamma tokens per request with the RNN head (bf16 W1, W2; float32
    Wp [3r][2r] and hp [B][gamma][3r]).  Returns (draft_tokens, draft_prob,
    draft_lse, e or None)."""
    B, gamma, V = U.shape
    r = W1.shape[1]
    dev = U.device
    _dev(U, "U", torch.float32)
    _dev(W1, "W1", torch.bfloat16, (V, r))
    _dev(W2, "W2", torch.bfloat16, (r, V))
    _dev(Wp, "Wp", torch.float32, (3 * r, 2 * r))
    _dev(hp, "hp", torch.float32, (B, gamma, 3 * r))
    _dev(x0, "x0", torch.int32, (B,))
    if seeds is not None:
        _dev(seeds, "seeds", torch.uint64, (B,))
    if out is None:
        out = (torch.empty((B, gamma), dtype=torch.int32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev),
               torch.empty((B, gamma, r), dtype=torch.float32, device=dev) if with_e else None)
    tok, prob, lse, e = out
    _dev(tok, "draft_tokens", torch.int32, (B, gamma))
    _dev(prob, "draft_prob", torch.float32, (B, gamma))
    _dev(lse, "draft_lse", torch.float32, (B, gamma))
    if e is not None:
        _dev(e, "e", torch.float32, (B, gamma, r))
    ws, nbytes = _workspace(OP_RNN_DRAFT, B, gamma, V, r, workspace, dev)
    st = load().dspark_rnn_draft(_p(U), _p(W1), _p(W2), _wdtype(W1, W2), _p(Wp), _p(hp), _p(x0), B, gamma, V, r,
                                 float(temperature), _p(seeds), int(rnd), _p(tok), _p(prob), _p(lse), _p(e),
                                 _p(ws), nbytes, _stream(stream, dev))
    _check("dspark_rnn_draft", st)
    return tok, prob, lse, e


def verify(U, W1, W2, x0, draft_tokens, draft_prob, target, temperature, seeds, rnd, out=None,
           with_accept_prob=True, workspace=None, stream=None, W2T=None, lengths=None, E=None):
    """Rejection-sampling verification.  Returns (accept_len, out_tokens, accept_prob or None).
    W2T: optional transposed copy of W2 from transpose_w2.  lengths: optional
    int32 [B] scheduled verification lengths (from schedule).  E: the
    float32 [B][gamma][r] operand rows of an RNN draft (rnn_draft with_e=True)
    when the tokens come from the RNN head."""
    B, g1, V = target.shape
    gamma = g1 - 1
    dev = target.device
    _dev(target, "target", torch.float32)
    r = W1.shape[1] if W1 is not None else 16
    if U is not None:
        _dev(U, "U", torch.float32, (B, gamma, V))
    if W1 is not None:
        _dev(W1, "W1", None, (V, r))
        _dev(W2, "W2", W1.dtype, (r, V))
    wd = _wdtype(W1, W2) if W1 is not None else _BF16
    if W2T is not None:
        _dev(W2T, "W2T", W2.dtype, (V, r))
    _dev(x0, "x0", torch.int32, (B,))
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, gamma))
    if draft_prob is not None:
        _dev(draft_prob, "draft_prob", torch.float32, (B, gamma))
    if seeds is not None:
        _dev(seeds, "seeds", torch.uint64, (B,))
    if lengths is not None:
        _dev(lengths, "lengths", torch.int32, (B,))
    if E is not None:
        _dev(E, "E", torch.float32, (B, gamma, r))
    if out is None:
        out = (torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B, gamma + 1), dtype=torch.int32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev) if with_accept_prob else None)
    alen, otok, aprob = out
    _dev(alen, "accept_len", torch.int32, (B,))
    _dev(otok, "out_tokens", torch.int32, (B, gamma + 1))
    if aprob is not None:
        _dev(aprob, "accept_prob", torch.float32, (B, gamma))
    ws, nbytes = _workspace(OP_VERIFY, B, gamma, V, r, workspace, dev)
    st = load().dspark_verify(_p(U), _p(W1), _p(W2), _p(W2T), wd, _p(x0), _p(draft_tokens), _p(draft_prob), _p(E),
                              _p(target), _p(lengths), B, gamma, V, r, float(temperature), _p(seeds), int(rnd), _p(alen),
                              _p(otok), _p(aprob), _p(ws), nbytes, _stream(stream, dev))
    _check("dspark_verify", st)
    return alen, otok, aprob


def confidence(h, w, W1, x0, draft_tokens, sts=None, out=None, stream=None):
    """Confidence head: h float32 [B][gamma][d], w float32 [d + r], W1 [V][r],
    sts optional float32 [gamma].  Returns conf float32 [B][gamma]."""
    B, gamma, d = h.shape
    V, r = W1.shape
    dev = h.device
    _dev(h, "h", torch.float32)
    _dev(w, "w", torch.float32, (d + r,))
    _dev(W1, "W1", None)
    wd = _wdtype(W1, W1)
    _dev(x0, "x0", torch.int32, (B,))
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, gamma))
    if sts is not None:
        _dev(sts, "sts", torch.float32, (gamma,))
    if out is None:
        out = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    _dev(out, "conf", torch.float32, (B, gamma))
    st = load().dspark_confidence(_p(h), _p(w), _p(W1), wd, _p(x0), _p(draft_tokens), _p(sts), B, gamma, d, V, r,
                                  _p(out), _stream(stream, dev))
    _check("dspark_confidence", st)
    return out


def schedule(survival, sps, out=None, with_theta=True, stream=None, mode=None, capacity=None, capacity_out=None):
    """Hardware-aware prefix scheduler: survival float32 [B][gamma], sps
    float64 [n >= B (gamma + 1) + 1] (sps[n] = SPS(n)).  mode: SCHEDULE_EARLY_STOP
    (default), SCHEDULE_CAPACITY (writes capacity_out, int32 [1], when given) or
    SCHEDULE_TOP_K (capacity: int32 [1] device tensor).  Returns (lengths int32
    [B], theta float64 [1] or None)."""
    B, gamma = survival.shape
    dev = survival.device
    mode = SCHEDULE_EARLY_STOP if mode is None else int(mode)
    _dev(survival, "survival", torch.float32)
    _dev(sps, "sps", torch.float64)
    if sps.dim() != 1:
        raise ValueError("sps must be one-dimensional")
    if capacity is not None:
        _dev(capacity, "capacity", torch.int32, (1,))
    if capacity_out is not None:
        _dev(capacity_out, "capacity_out", torch.int32, (1,))
    if out is None:
        out = (torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((1,), dtype=torch.float64, device=dev) if with_theta else None)
    lengths, theta = out
    _dev(lengths, "lengths", torch.int32, (B,))
    if theta is not None:
        _dev(theta, "theta", torch.float64, (1,))
    st = load().dspark_schedule(_p(survival), _p(sps), int(sps.shape[0]), B, gamma, mode, _p(capacity),
                                _p(capacity_out), _p(lengths), _p(theta), _stream(stream, dev))
    _check("dspark_schedule", st)
    return lengths, theta


def transpose_w2(W2, out=None, stream=None):
    """W2 [r][V] -> a new (or the given) [V][r] tensor of the same dtype."""
    r, V = W2.shape
    dev = W2.device
    _dev(W2, "W2", None)
    wd = _wdtype(W2, W2)
    if out is None:
        out = torch.empty((V, r), dtype=W2.dtype, device=dev)
    _dev(out, "W2T", W2.dtype, (V, r))
    st = load().dspark_transpose_w2(_p(W2), wd, r, V, _p(out), _stream(stream, dev))
    _check("dspark_transpose_w2", st)
    return out


def survival(U, W1, W2, x0, draft_tokens, draft_lse, target, temperature, conf=None, out=None,
             with_c_star=True, workspace=None, stream=None, E=None):
    """Prefix survival products.  Returns (c_star or None, survival).  E: the
    operand rows of an RNN draft, as for verify."""
    if conf is not None:
        B, gamma = conf.shape
        dev = conf.device
        _dev(conf, "conf", torch.float32)
        surv = out[1] if out is not None else torch.empty((B, gamma), dtype=torch.float32, device=dev)
        _dev(surv, "survival", torch.float32, (B, gamma))
        st = load().dspark_survival(None, None, None, _BF16, None, None, None, None, None, _p(conf), B, gamma, 2, 16,
                                    0.0, None, _p(surv), None, 0, _stream(stream, dev))
        _check("dspark_survival", st)
        return None, surv
    B, g1, V = target.shape
    gamma = g1 - 1
    dev = target.device
    _dev(target, "target", torch.float32)
    r = W1.shape[1] if W1 is not None else 16
    if U is not None:
        _dev(U, "U", torch.float32, (B, gamma, V))
    if W1 is not None:
        _dev(W1, "W1", None, (V, r))
        _dev(W2, "W2", W1.dtype, (r, V))
    wd = _wdtype(W1, W2) if W1 is not None else _BF16
    _dev(x0, "x0", torch.int32, (B,))
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, gamma))
    if draft_lse is not None:
        _dev(draft_lse, "draft_lse", torch.float32, (B, gamma))
    if E is not None:
        _dev(E, "E", torch.float32, (B, gamma, r))
    if out is None:
        out = (torch.empty((B, gamma), dtype=torch.float32, device=dev) if with_c_star else None,
               torch.empty((B, gamma), dtype=torch.float32, device=dev))
    cst, surv = out
    if cst is not None:
        _dev(cst, "c_star", torch.float32, (B, gamma))
    _dev(surv, "survival", torch.float32, (B, gamma))
    ws, nbytes = _workspace(OP_SURVIVAL, B, gamma, V, r, workspace, dev)
    st = load().dspark_survival(_p(U), _p(W1), _p(W2), wd, _p(x0), _p(draft_tokens), _p(draft_lse), _p(E),
                                _p(target), None, B, gamma, V, r, float(temperature), _p(cst), _p(surv), _p(ws), nbytes,
                                _stream(stream, dev))
    _check("dspark_survival", st)
    return cst, surv
