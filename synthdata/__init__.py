"""Seeded synthetic inputs for the dynamic-chunking layer.

This package holds only input generation: random streams, the random
stand-ins for the networks around the chunk layer (byte embedding, causal
conv, q/k projections, stage projections, the global map) and bf16 rounding
of those inputs.  It holds none of the chunking method's own arithmetic, so
the CPU oracle and the HIP path can both consume its outputs without sharing
any code of the method.
"""
from .generators import (  # noqa: F401
    bf16_round, bf16_bits, from_bf16_bits, Ragged,
    gen_c0, gen_c0_dr_tiny, gen_c1, gen_c2, gen_c2_stage2_inputs, gen_c2_backproj,
    gen_c3, gen_c4, gen_c4_global, cluster_rows, event_bytes, CONFIG_SEED,
)
