"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This package holds shapes and random draws only: none of the attention
method's arithmetic lives here, so both the HIP path and the fp64 oracle can
consume the same inputs without sharing any code of the method.
"""
from .configs import CONFIGS, SwinConfig, get_config  # noqa: F401
from .generate import (ModuleParams, Inputs, BlockExtras, make_inputs, make_block_extras,  # noqa: F401
                       round_bf16, bf16_bits_to_f64)
