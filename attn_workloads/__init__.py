"""Seeded synthetic workloads for the tiled attention forward.

This package only draws inputs: shapes, random values rounded to the storage
dtype, block tables and per-sequence key lengths. It holds none of the
attention arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path
(``attention_forward_tiled_amd``) can consume the same inputs without sharing
any code with each other.
"""
from .configs import (  # noqa: F401
    PrefillCase,
    DecodeCase,
    CONFIGS,
    config,
)
from .generate import (  # noqa: F401
    PrefillInputs,
    DecodeInputs,
    make_prefill_inputs,
    make_decode_inputs,
    round_to_bits,
    bits_to_f64,
    bits_to_f32,
    NAN_BITS,
)
