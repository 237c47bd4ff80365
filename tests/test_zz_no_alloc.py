"""The allocation-free draft (dspark_markov_draft_noalloc, scratch in a static
device array) against the workspace draft (dspark_markov_draft) through the
C ABI: two calls in a row, the second with a smaller input, each compared
with the workspace entry point on the same inputs to the parity bar (tokens
exact, probabilities to 1e-5 relative)."""

import numpy as np
import pytest
import torch

dsp = pytest.importorskip("draft_sampling_verification_bias_amd")

pytestmark = pytest.mark.gpu


def _inputs(B, gamma, V, r, seed, wdtype=torch.bfloat16):
    g = torch.Generator(device="cpu").manual_seed(seed)
    U = (torch.randn((B, gamma, V), generator=g) * 3.0).float()
    hot = torch.randint(0, V, (B, gamma, 3), generator=g)
    U.scatter_add_(2, hot, torch.full(hot.shape, 8.0))
    W1 = (torch.randn((V, r), generator=g) * 0.02).to(wdtype)
    W2 = (torch.randn((r, V), generator=g) * 0.02).to(wdtype)
    x0 = torch.randint(0, V, (B,), generator=g, dtype=torch.int32)
    seeds = torch.randint(0, 2 ** 62, (B,), generator=g, dtype=torch.int64)
    dev = "cuda:0"
    return (U.to(dev), W1.to(dev), W2.to(dev), x0.to(dev), seeds.to(dev).view(torch.uint64))


def _compare(case, B, gamma, V, r, T, seed, wdtype=torch.bfloat16):
    print("no-alloc case %s: B=%d gamma=%d V=%d r=%d T=%g" % (case, B, gamma, V, r, T), flush=True)
    U, W1, W2, x0, seeds = _inputs(B, gamma, V, r, seed, wdtype)
    ref = dsp.markov_draft(U, W1, W2, x0, T, seeds, 11)
    got = dsp.markov_draft_noalloc(U, W1, W2, x0, T, seeds, 11)
    torch.cuda.synchronize()
    rt, rp, rl = (t.cpu().numpy() for t in ref)
    gt, gp, gl = (t.cpu().numpy() for t in got)
    assert (rt >= 0).all() and (rt < V).all()
    np.testing.assert_array_equal(gt, rt)
    np.testing.assert_allclose(gp, rp, rtol=1e-5, atol=1e-30)
    np.testing.assert_allclose(gl, rl, rtol=1e-5, atol=1e-6)


def test_noalloc_draft_matches_the_workspace_draft_on_two_calls():
    # first call: the 256-row ring tile pass, a ragged last tile, sampling
    _compare("large", 256, 7, 20000, 256, 0.7, seed=1)
    # second call, smaller: the generic tile pass and selection on the same
    # static array (its earlier contents must not leak into the result)
    _compare("small", 37, 4, 4099, 64, 1.0, seed=2)


def test_noalloc_draft_greedy_and_float32_weights():
    _compare("greedy", 64, 5, 8192, 256, 0.0, seed=3)
    _compare("f32", 9, 3, 1000, 16, 1.0, seed=4, wdtype=torch.float32)


def test_noalloc_draft_rejects_sizes_beyond_its_scratch():
    assert dsp.static_scratch_bytes() == 32 << 20
    U, W1, W2, x0, seeds = _inputs(4, 2, 256, 16, seed=5)
    # a workspace need above the array is refused on the host, before any launch
    lib = dsp.load()
    st = lib.dspark_markov_draft_noalloc(U.data_ptr(), W1.data_ptr(), W2.data_ptr(), None, 1, x0.data_ptr(), 4096, 7,
                                         151936, 256, 1.0, seeds.data_ptr(), 0, x0.data_ptr(), U.data_ptr(),
                                         U.data_ptr(), None, None, None, 0, None, None)
    assert st == -5


def test_noalloc_draft_confidence_output():
    # the fused confidence head through the allocation-free entry point: the
    # same confidences as the workspace draft's
    B, gamma, V, r, d = 48, 5, 8192, 256, 512
    U, W1, W2, x0, seeds = _inputs(B, gamma, V, r, seed=6)
    g = torch.Generator(device="cpu").manual_seed(7)
    head = (torch.randn((B, gamma, d), generator=g).cuda(), (torch.randn((d + r,), generator=g) * 0.05).cuda(),
            torch.linspace(0.8, 1.6, gamma).cuda())
    ref = dsp.markov_draft(U, W1, W2, x0, 1.0, seeds, 12, conf_head=head)
    got = dsp.markov_draft_noalloc(U, W1, W2, x0, 1.0, seeds, 12, conf_head=head)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got[0].cpu().numpy(), ref[0].cpu().numpy())
    rc, gc = ref[3].cpu().numpy(), got[3].cpu().numpy()
    assert np.isfinite(rc).all()
    np.testing.assert_allclose(gc, rc, rtol=1e-6, atol=0)
