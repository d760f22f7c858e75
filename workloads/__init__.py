"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This package holds shapes and random draws only: none of the attention
method's arithmetic lives here, so both the HIP path and the fp64 oracle can
consume the same inputs without sharing any code of the method.
"""
from .configs import CONFIGS, SwinConfig, get_config  # noqa: F401
from .generate import (BLOCK_BIAS_SCALE, ModuleParams, Inputs, BlockExtras, make_inputs,  # noqa: F401
                       make_block_extras, round_bf16, bf16_bits_to_f64)
