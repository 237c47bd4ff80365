"""Pin of the oracle's weight decoding: the float64 value of every bf16 bit
pattern equals torch's own bfloat16 -> float64 conversion (all 65536
patterns: signed zeros, subnormals, infinities, NaNs), and float32 weights
are widened exactly.  Every parity case reads its Markov weights through this
decoding, so a wrong shift or byte order here would move every oracle value."""

import numpy as np
import pytest
import torch

from oracle import dspark_ref as ref


@pytest.mark.filterwarnings("ignore:invalid value encountered in cast:RuntimeWarning")
def test_every_bf16_bit_pattern_decodes_as_torch_does():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = ref.weights_as_f64(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))   # -0.0 stays negative
    assert got[0x3F80] == 1.0 and got[0xC000] == -2.0 and got[0x0001] == 2.0 ** -133


def test_bf16_rounded_weights_round_trip():
    # weights as the workloads store them: float32 normals rounded to bf16 by torch
    x = np.random.default_rng(3).normal(0, 0.02, size=50000).astype(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ref.weights_as_f64(bits, "bf16"), t.to(torch.float64).numpy())


def test_float32_weights_widen_exactly():
    x = np.random.default_rng(4).normal(0, 0.1, size=4096).astype(np.float32)
    x[:4] = [0.0, -0.0, np.float32(1e-45), np.float32(3.4e38)]
    got = ref.weights_as_f64(x, "f32")
    np.testing.assert_array_equal(got, torch.from_numpy(x).to(torch.float64).numpy())
    assert got.dtype == np.float64
