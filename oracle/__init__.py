"""CPU oracle for local-Hessian-weighted NVFP4 weight-scale calibration (test infrastructure).

Plain, slow, float64 NumPy.  Only the tests, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import it; the product path (the HIP library and its
Python binding) never does, and shares no code with it.

Pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``.  Parity unpinned: none of
the functions below lacks a pin; see the module docstring of ``oracle.lh_oracle`` for which pin
covers which function.
"""
from .lh_oracle import (  # noqa: F401
    E2M1_GRID,
    absmax,
    candidate_losses,
    accumulate,
    accumulate_act_aware,
    activation_fake_quant,
    candidate_scales,
    dequantize,
    e2m1_index,
    e4m3_ladder,
    e4m3_nearest,
    exempt_mask,
    fake_quant,
    global_scale,
    multiplier_allowed,
    multiplier_codes,
    pack_nibbles,
    sweep,
    sweep_blocks,
    sweep_blocks_diag,
    sweep_diag,
)
