"""Seeded synthetic workloads shared by the oracle's tests and the HIP path's
tests and benchmark.  No attention arithmetic lives here."""
from .synth import (D_LATENT, D_QK, D_ROPE, SM_SCALE, WORKLOADS, Workload,
                    bf16_bits_to_f32, bf16_bits_to_f64, custom, f32_to_bf16_bits)

__all__ = ["D_LATENT", "D_QK", "D_ROPE", "SM_SCALE", "WORKLOADS", "Workload",
           "bf16_bits_to_f32", "bf16_bits_to_f64", "custom", "f32_to_bf16_bits"]
