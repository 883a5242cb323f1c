"""Seeded synthetic inputs for sparse latent attention.

This package only draws random numbers and lays them out.  It holds none of the
attention arithmetic, so both the CPU oracle and the HIP path can consume its
output without sharing any of the method's code.
"""
from .generators import (  # noqa: F401
    AppendConfig,
    append_inputs,
    rotary_angles,
    CONFIGS,
    DEFAULT_SEED,
    DecodeConfig,
    PrefillConfig,
    bf16_round_bits,
    decode_batch_row,
    decode_inputs,
    decode_query_set,
    fp8_wkv_b_inputs,
    prefill_inputs,
    prefill_query_rows,
    projection_inputs,
    weights,
)
