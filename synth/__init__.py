"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's timing leg.

This package holds no arithmetic of the calibration method (no Hessians, no scale
search, no weight or activation quantization).  It only draws tensors with fixed seeds
and the shapes/distributions of the workloads and converts them to the storage dtype.
The activation-aware workload's X_q (the input quantizer's fake-quant of X) is made by
the oracle in the tests and by the library in the benchmark, never here.
"""
from .configs import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make,
    rng_for,
)
