"""Seeded synthetic inputs for QUOKA's per-chunk hot path.

This package only draws random numbers and lays them out. It holds none of
the method's arithmetic (no cosines, scores, selections or attention), so the
oracle and the HIP library can both take their inputs from it.
"""
from .generate import (  # noqa: F401
    CONFIGS, Workload, make_config, make_case, round_to_bf16, bf16_bits,
)
