"""Seeded synthetic workloads shared by the oracle and the GPU path.

Shapes and value recipe only: nothing here computes attention, states,
masks or their composition.
"""
from .configs import WORKLOADS, Workload, get  # noqa: F401
from .inputs import (InputStream, bf16_bits_to_f32, bf16_bits_to_f64,  # noqa: F401
                     pos_encoding, step_inputs, step_masters, to_bf16_bits,
                     token_coords)
