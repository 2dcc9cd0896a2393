"""Seeded synthetic inputs for the GDN token mixer.

This package only draws random tensors. It holds none of the mixer's arithmetic, so both the
fp64 oracle (``oracle/``) and the HIP library (``linear_attention_token_amd``) can consume the
same tensors without sharing any code of the method.
"""
from .gen import (  # noqa: F401
    PrefillInputs,
    DecodeInputs,
    prefill_inputs,
    decode_inputs,
    ProjectionInputs,
    projection_inputs,
    IndexerInputs,
    indexer_inputs,
    loguniform_lengths,
    config_tiny,
    config_layer,
    config_long,
    config_varlen,
    config_decode,
    CONV_WIDTH,
)
