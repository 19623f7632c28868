"""Seeded synthetic inputs for the routed-MoE layer.

This module only draws and stores inputs (activations, router weights, router
bias, expert weights in their storage formats).  It holds none of the layer's
arithmetic: the quantizer here *defines* the low-bit synthetic weights as
(code, scale) pairs, and each side decodes them with its own code.
"""
from .configs import CONFIGS, MoEConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    LayerInputs, make_layer, make_x, make_router, make_experts, quantize_pack,
    expert_view_to_numpy, tensor_to_numpy_storage,
)
