"""C-ABI checks that need no GPU: the library loads, exports every entry point
that include/dspark.h declares, and rejects bad arguments on the host with the
documented status codes before any HIP call is made."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

dsp = pytest.importorskip("draft_sampling_verification_bias_amd")

HEADER = os.path.join(ROOT, "include", "dspark.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, SCRATCH = 0, -1, -2, -3, -4, -5
FAKE = 0x100000          # non-null, 16-byte aligned, never dereferenced (validation fails first)
MISALIGNED = 0x100004
FAKE2 = 0x200000         # a second distinct fake pointer


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsp.library_path()):
        pytest.fail("libdspark.so is not built: run python -m draft_sampling_verification_bias_amd.build")
    return dsp.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dspark_markov_draft", "dspark_verify", "dspark_survival", "dspark_markov_bias", "dspark_schedule",
              "dspark_confidence", "dspark_rnn_draft", "dspark_markov_draft_noalloc", "dspark_static_scratch_bytes",
              "dspark_workspace_size", "dspark_status_string", "dspark_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.dspark_version() >= 100
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, SCRATCH):
        s = lib.dspark_status_string(code)
        assert s and len(s) > 1
    assert lib.dspark_status_string(123) == b"unknown status"


@pytest.mark.parametrize("op", [dsp.OP_DRAFT, dsp.OP_VERIFY, dsp.OP_SURVIVAL, dsp.OP_RNN_DRAFT])
def test_workspace_size(lib, op):
    small = dsp.workspace_size(op, 4, 4, 1000, 16)
    big = dsp.workspace_size(op, 256, 7, 151936, 256)
    assert 0 < small < big
    # out-of-range sizes give 0
    for args in ((0, 4, 1000, 16), (4, 0, 1000, 16), (4, 33, 1000, 16), (4, 4, 1, 16),
                 (4, 4, 1000, 8), (4, 4, 1000, 24), (4, 4, 1000, 528), (65537, 4, 1000, 16)):
        assert dsp.workspace_size(op, *args) == 0
    assert dsp.workspace_size(7, 4, 4, 1000, 16) == 0


def _draft(lib, **kw):
    a = dict(U=FAKE, W1=FAKE, W2=FAKE, W2T=None, wd=1, x0=FAKE, B=4, gamma=4, V=1000, r=16, T=1.0, seeds=FAKE,
             rnd=0, tok=FAKE, prob=FAKE, lse=FAKE, ch=None, cw=None, csts=None, cd=0, conf=None, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return lib.dspark_markov_draft(a["U"], a["W1"], a["W2"], a["W2T"], a["wd"], a["x0"], a["B"], a["gamma"], a["V"],
                                   a["r"], a["T"], a["seeds"], a["rnd"], a["tok"], a["prob"], a["lse"],
                                   a["ch"], a["cw"], a["csts"], a["cd"], a["conf"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), INVALID), (dict(gamma=0), INVALID), (dict(gamma=33), INVALID), (dict(V=1), INVALID),
    (dict(r=8), INVALID), (dict(r=40), INVALID), (dict(T=-1.0), INVALID), (dict(T=float("nan")), INVALID),
    (dict(T=float("inf")), INVALID), (dict(U=None), INVALID), (dict(W2=None), INVALID),
    (dict(tok=None), INVALID), (dict(seeds=None), INVALID), (dict(U=MISALIGNED), INVALID),
    (dict(ws=None), INVALID), (dict(wd=5), UNSUPPORTED), (dict(wsb=16), WORKSPACE),
    (dict(W2T=MISALIGNED), INVALID), (dict(W2T=FAKE), INVALID),  # W2T may not alias W2
    # the confidence head: its inputs are checked only when its output is asked for
    (dict(conf=FAKE, ch=None, cw=FAKE, cd=64), INVALID),
    (dict(conf=FAKE, ch=FAKE, cw=MISALIGNED, cd=64), INVALID), (dict(conf=FAKE, ch=FAKE, cw=FAKE, cd=0), INVALID),
    (dict(conf=FAKE, ch=FAKE, cw=FAKE, cd=(1 << 20) + 1), INVALID),
    (dict(conf=MISALIGNED - 2, ch=FAKE, cw=FAKE, cd=64), INVALID),
    (dict(conf=FAKE, ch=FAKE, cw=FAKE, csts=MISALIGNED - 2, cd=64), INVALID),
])
def test_draft_rejects_bad_arguments(lib, kw, status):
    assert _draft(lib, **kw) == status


def _draft_noalloc(lib, **kw):
    a = dict(U=FAKE, W1=FAKE, W2=FAKE, W2T=None, wd=1, x0=FAKE, B=4, gamma=4, V=1000, r=16, T=1.0, seeds=FAKE,
             rnd=0, tok=FAKE, prob=FAKE, lse=FAKE, ch=None, cw=None, csts=None, cd=0, conf=None)
    a.update(kw)
    return lib.dspark_markov_draft_noalloc(a["U"], a["W1"], a["W2"], a["W2T"], a["wd"], a["x0"], a["B"], a["gamma"],
                                           a["V"], a["r"], a["T"], a["seeds"], a["rnd"], a["tok"], a["prob"],
                                           a["lse"], a["ch"], a["cw"], a["csts"], a["cd"], a["conf"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), INVALID), (dict(gamma=33), INVALID), (dict(V=1), INVALID), (dict(r=40), INVALID),
    (dict(T=-1.0), INVALID), (dict(U=None), INVALID), (dict(seeds=None), INVALID), (dict(U=MISALIGNED), INVALID),
    (dict(wd=5), UNSUPPORTED), (dict(conf=FAKE, ch=FAKE, cw=MISALIGNED, cd=64), INVALID),
    # sizes whose draft workspace exceeds the static array: rejected on the host
    (dict(B=4096, V=151936, r=256, gamma=7), SCRATCH), (dict(B=65536, V=16000, r=16), SCRATCH),
])
def test_draft_noalloc_rejects_bad_arguments_and_sizes_beyond_its_scratch(lib, kw, status):
    assert _draft_noalloc(lib, **kw) == status


def test_static_scratch_holds_the_timed_workloads(lib):
    cap = lib.dspark_static_scratch_bytes()
    assert cap == 32 << 20
    for B, gamma, V in ((256, 7, 151936), (512, 7, 151936), (128, 7, 262144), (32, 7, 151936)):
        assert 0 < dsp.workspace_size(dsp.OP_DRAFT, B, gamma, V, 256) <= cap
    assert dsp.workspace_size(dsp.OP_DRAFT, 4096, 7, 151936, 256) > cap


def _rnn_draft(lib, **kw):
    a = dict(U=FAKE, W1=FAKE, W2=FAKE, wd=1, Wp=FAKE, hp=FAKE, x0=FAKE, B=4, gamma=4, V=1000, r=16, T=1.0,
             seeds=FAKE, rnd=0, tok=FAKE, prob=FAKE, lse=FAKE, e=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.dspark_rnn_draft(a["U"], a["W1"], a["W2"], a["wd"], a["Wp"], a["hp"], a["x0"], a["B"], a["gamma"],
                                a["V"], a["r"], a["T"], a["seeds"], a["rnd"], a["tok"], a["prob"], a["lse"], a["e"],
                                a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), INVALID), (dict(gamma=33), INVALID), (dict(r=40), INVALID), (dict(T=-1.0), INVALID),
    (dict(Wp=None), INVALID), (dict(hp=None), INVALID), (dict(Wp=MISALIGNED), INVALID),
    (dict(hp=MISALIGNED - 2), INVALID), (dict(e=MISALIGNED - 2), INVALID), (dict(seeds=None), INVALID),
    (dict(wd=0), UNSUPPORTED), (dict(wd=5), UNSUPPORTED), (dict(wsb=16), WORKSPACE),
])
def test_rnn_draft_rejects_bad_arguments(lib, kw, status):
    assert _rnn_draft(lib, **kw) == status


def test_rnn_draft_workspace_holds_the_state_and_operands():
    B, gamma, V, r = 256, 7, 151936, 256
    need = dsp.workspace_size(dsp.OP_RNN_DRAFT, B, gamma, V, r)
    # tile summaries and look-ahead uniforms, float32 state (two buffers),
    # bf16 operand rows of 2r values
    ntiles = (V + 127) // 128
    assert need >= B * ntiles * 8 + 2 * B * 8 + 2 * B * r * 4 + B * gamma * 2 * r * 2


def test_draft_workspace_holds_either_schedule_of_the_loop():
    B, gamma, V, r = 256, 7, 151936, 256
    need = dsp.workspace_size(dsp.OP_DRAFT, B, gamma, V, r)
    # per-position launches: summaries, uniforms, ring operands
    assert need >= B * ((V + 127) // 128) * 8 + 2 * B * 8 + B * 512
    # the resident loop: range summaries (2048 per row), E rows, flags
    assert need >= B * 2048 * 8 + B * 512 + 257 * 4


def _verify(lib, **kw):
    a = dict(U=FAKE, W1=FAKE, W2=FAKE, W2T=None, wd=1, x0=FAKE, dt=FAKE, dp=FAKE, E=None, tgt=FAKE, lens=None, B=4,
             gamma=4, V=1000, r=16, T=1.0, seeds=FAKE, rnd=0, alen=FAKE, otok=FAKE, aprob=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.dspark_verify(a["U"], a["W1"], a["W2"], a["W2T"], a["wd"], a["x0"], a["dt"], a["dp"], a["E"], a["tgt"],
                             a["lens"], a["B"], a["gamma"], a["V"], a["r"], a["T"], a["seeds"], a["rnd"], a["alen"],
                             a["otok"], a["aprob"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=70000), INVALID), (dict(tgt=None), INVALID), (dict(alen=None), INVALID),
    (dict(dp=None), INVALID), (dict(tgt=MISALIGNED), INVALID), (dict(wd=9), UNSUPPORTED),
    (dict(wsb=0), WORKSPACE), (dict(T=-0.5), INVALID), (dict(W2T=MISALIGNED), INVALID),
    (dict(lens=MISALIGNED - 2), INVALID), (dict(E=MISALIGNED - 2), INVALID),
])
def test_verify_rejects_bad_arguments(lib, kw, status):
    assert _verify(lib, **kw) == status


def test_survival_rejects_bad_arguments(lib):
    s = lib.dspark_survival
    # confidence mode: bad sizes, missing output
    assert s(None, None, None, 1, None, None, None, None, None, FAKE, 0, 4, 2, 16, 0.0, None, FAKE, None, 0,
             None) == INVALID
    assert s(None, None, None, 1, None, None, None, None, None, FAKE, 4, 4, 2, 16, 0.0, None, None, None, 0,
             None) == INVALID
    # analytical mode: missing target, bad dtype, small workspace, misaligned draft rows
    assert s(FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, None, None, 4, 4, 1000, 16, 1.0, None, FAKE, FAKE, 1 << 30,
             None) == INVALID
    assert s(FAKE, FAKE, FAKE, 3, FAKE, FAKE, FAKE, None, FAKE, None, 4, 4, 1000, 16, 1.0, None, FAKE, FAKE, 1 << 30,
             None) == UNSUPPORTED
    assert s(FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, None, 4, 4, 1000, 16, 1.0, None, FAKE, FAKE, 8,
             None) == WORKSPACE
    assert s(FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, MISALIGNED - 2, FAKE, None, 4, 4, 1000, 16, 1.0, None, FAKE, FAKE,
             1 << 30, None) == INVALID


def test_transpose_w2_rejects_bad_arguments(lib):
    f = lib.dspark_transpose_w2
    assert f(FAKE, 1, 8, 1000, FAKE2, None) == INVALID          # r below 16
    assert f(FAKE, 1, 24, 1000, FAKE2, None) == INVALID         # r not a multiple of 16
    assert f(FAKE, 1, 16, 1, FAKE2, None) == INVALID            # V below 2
    assert f(None, 1, 16, 1000, FAKE2, None) == INVALID
    assert f(FAKE, 1, 16, 1000, MISALIGNED, None) == INVALID
    assert f(FAKE, 1, 16, 1000, FAKE, None) == INVALID          # in place
    assert f(FAKE, 4, 16, 1000, FAKE2, None) == UNSUPPORTED


def test_markov_bias_rejects_bad_arguments(lib):
    f = lib.dspark_markov_bias
    assert f(FAKE, FAKE, 1, FAKE, 0, 1000, 16, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 1, FAKE, 4, 1000, 17, FAKE, None) == INVALID
    assert f(FAKE, None, 1, FAKE, 4, 1000, 16, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 2, FAKE, 4, 1000, 16, FAKE, None) == UNSUPPORTED


def test_schedule_rejects_bad_arguments(lib):
    f = lib.dspark_schedule
    # (survival, sps, sps_len, B, gamma, mode, capacity_in, capacity_out, lengths, theta, stream)
    assert f(FAKE, FAKE, 20, 4, 4, 0, None, None, FAKE, None, None) == INVALID   # sps shorter than B (gamma + 1) + 1
    assert f(FAKE, FAKE, 1 << 20, 0, 4, 0, None, None, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, 1 << 20, 4, 33, 0, None, None, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, 1 << 20, 4097, 4, 0, None, None, FAKE, None, None) == INVALID  # more than 16384 candidates
    assert f(None, FAKE, 1 << 20, 4, 4, 0, None, None, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, 1 << 20, 4, 4, 0, None, None, None, None, None) == INVALID
    assert f(FAKE, MISALIGNED, 1 << 20, 4, 4, 0, None, None, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, 1 << 20, 4, 4, 3, None, None, FAKE, None, None) == INVALID     # unknown mode
    assert f(FAKE, FAKE, 1 << 20, 4, 4, 2, None, None, FAKE, None, None) == INVALID     # top-K without a capacity
    assert f(FAKE, FAKE, 1 << 20, 4, 4, 1, None, MISALIGNED - 2, FAKE, None, None) == INVALID


def test_confidence_rejects_bad_arguments(lib):
    f = lib.dspark_confidence
    # (h, w, W1, wdtype, x0, tokens, sts, B, gamma, d, V, r, conf, stream)
    ok = [FAKE, FAKE, FAKE, 1, FAKE, FAKE, None, 4, 4, 64, 1000, 16, FAKE, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a9=0) == INVALID            # d = 0
    assert call(a7=0) == INVALID            # B = 0
    assert call(a11=24) == INVALID          # r not a multiple of 16
    assert call(a0=None) == INVALID
    assert call(a1=MISALIGNED) == INVALID   # w not 16-byte aligned
    assert call(a6=MISALIGNED - 2) == INVALID
    assert call(a12=None) == INVALID
    assert call(a3=7) == UNSUPPORTED
