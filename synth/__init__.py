"""Seeded synthetic inputs for the per-layer KronQ solver.

This package only draws random numbers and rounds them to the storage types
(fp32, bf16). It holds no step of the quantization method, so both the
float64 oracle and the GPU path can take their inputs from it without sharing
any of the method's arithmetic.
"""
from .configs import (  # noqa: F401
    CONFIGS, LayerSpec, C5_SUBLAYERS, C5_INPUTS, C5_LAYERS, C5_TOKENS, c5_specs, scaled,
    layer_inputs, gen_W, gen_X, gen_X_chunks, gen_HG, gen_G, gen_omega, gen_signs, gen_X_drift,
    bf16_round, bf16_to_f32, f32_to_bf16_bits, widen, rng,
)
