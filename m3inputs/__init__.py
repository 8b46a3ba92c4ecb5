"""Seeded synthetic inputs for the Mamba-3 scan and decode step.

This package is the only code that both the CPU oracle and the HIP path
consume.  It draws random tensors with the shapes and value laws of the
workloads and rounds them to the storage dtype; it holds none of the
recurrence's arithmetic (no decay, no rotation, no state update).
"""
from .configs import CONFIGS, Config, config_by_name  # noqa: F401
from .gen import (  # noqa: F401
    bf16_round,
    bf16_bits,
    bits_to_f32,
    make_block_inputs,
    make_cotangents,
    make_scan_inputs,
    make_decode_inputs,
    make_small_case,
)
