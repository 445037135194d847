"""Seeded synthetic inputs for the wide-row bf16 top-k.

This package only draws and lays out input rows (bf16 bit patterns in a
row-strided uint16 matrix).  It performs no ranking, selection or
classification of values, so both the CPU oracle and the HIP library can be
fed from it without sharing any of the method's arithmetic.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    FAMILIES,
    Config,
    config,
    f32_to_bf16_bits,
    bf16_to_f16_bits,
    bf16_to_f32_bits,
    family_rows,
    head_inputs,
    make_config_input,
    poison_padding,
    sha256_of,
)
