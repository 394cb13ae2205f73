"""Seeded synthetic inputs for the group-quantized routed-expert MoE layer.

This package is shared by the CPU oracle (``oracle/``) and by the GPU path's
tests and benchmark.  It holds shapes, seeds and random draws only: none of
the layer's arithmetic (no dequantisation, routing, SwiGLU or combine) lives
here.  Random ``uint32`` words stand for packed quantised values directly,
because i.i.d. uniform words are exactly i.i.d. uniform 4- or 8-bit fields.
"""

from .configs import CONFIGS, GDN_CONFIGS, MoEConfig, get_config  # noqa: F401
from .generate import (  # noqa: F401
    bf16_bits_from_f32,
    expert_arrays,
    gdn_inputs,
    router_arrays,
    shared_arrays,
    token_x,
    tokens_x,
)
