"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package draws random numbers and nothing else: it holds none of the
W4A16 arithmetic (no packing, no dequantisation, no contraction, no output
rounding). Both the CPU oracle and the HIP path receive exactly these arrays.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Inputs,
    make_inputs,
    make_config,
    make_workspace,
)
