"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This package holds no arithmetic of the method: it only fixes shapes, seeds and
draw order, and encodes normally distributed draws as bf16 bit patterns (or
keeps them as fp32).  Both sides receive exactly the same bits.
"""
from .configs import CONFIGS, Config, config_by_index  # noqa: F401
from .gen import (  # noqa: F401
    f32_to_bf16_bits,
    make_attention_inputs,
    make_update_inputs,
    draw,
)
