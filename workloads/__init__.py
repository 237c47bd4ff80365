"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the
benchmark.  Holds data recipes only."""

from .gen import (NAMES, WORKLOADS, Workload, bf16_bits_to_f32, f32_to_bf16_bits, make, request_seeds, rnn_inputs,  # noqa: F401
                  confidence_inputs, sps_curve)
