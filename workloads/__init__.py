"""Seeded synthetic inputs shared by the oracle tests and the HIP path.

This package holds input generators only: it contains none of the attention,
selection or sampling arithmetic, so both sides of every parity check can use
it without sharing method code.
"""
from .synth import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits,
    bf16_round,
    gen_config,
    gen_exact,
    exact_keys,
    exact_family_block,
    gen_micro,
    gen_fourier_heads,
)
