"""Seeded synthetic workloads for the verification step (no verification arithmetic)."""
from .gen import (WORKLOADS, HEADLINE, Workload, make_inputs, f32_to_bf16_bits, bf16_bits_to_f32,  # noqa: F401
                  pack_ragged, ragged_lengths)
