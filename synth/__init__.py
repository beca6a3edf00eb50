"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's timing leg.

This package holds no arithmetic of the calibration method (no Hessians, no scale
search, no weight quantization).  It only draws tensors with fixed seeds and the
shapes/distributions of the workloads, converts them to the storage dtype, and (for
the activation-aware workload) produces the quantized activation input ``X_q`` by the
input recipe documented in ``synth.configs.activation_fake_quant``.
"""
from .configs import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make,
    rng_for,
)
