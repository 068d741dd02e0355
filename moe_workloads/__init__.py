"""Seeded synthetic workloads for the DeepSeekMoE layer.

This module only draws numbers: configuration records and seeded random
tensors (activations, expert affinity vectors, routing biases, expert
weights).  It contains none of the layer's arithmetic, so both the GPU
path's tests/benchmark and the CPU oracle's tests can take their inputs
from it without sharing any of the method.
"""

from .configs import CONFIGS, PARITY_CONFIGS, MoEConfig, get_config  # noqa: F401
from .generate import (  # noqa: F401
    MoEInputs,
    make_inputs,
    make_expert_weights,
    seed_for,
    to_numpy_f32,
)
