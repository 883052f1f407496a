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
    gen_hnet_tiny, gen_coding_rate_tiny, gen_event_streams, gen_hnet_two_stage, gen_stage2_inputs, gen_stage2_backproj,
    gen_coding_rate_fp32, gen_byteflow_layer, gen_global_standin, gen_cosine_qk, cluster_rows, event_bytes, SEED_HNET_TINY, SEED_EVENT_STREAMS, SEED_HNET_TWO_STAGE,
    SEED_CODING_RATE_FP32, SEED_BYTEFLOW_LAYER,
)
