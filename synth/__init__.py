"""Seeded synthetic inputs for the Qwen3/Qwen3-VL decoder-layer prefill.

This module is shared by the oracle-side tests and the GPU-side tests and
bench. It holds no part of the layer's arithmetic: it only draws seeded
normal variates, rounds them to the storage precision, and lays out the
three-axis position table a workload prescribes. Every array it returns is
a host numpy array.
"""

from .configs import CONFIGS, LayerConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    NORM_NAMES,
    PROJ_NAMES,
    WEIGHT_NAMES,
    make_deepstack,
    make_deepstack_layers,
    make_layer_weights,
    make_model_weights,
    make_positions,
    make_quant_layer_weights,
    make_tokens,
    make_x,
    round_to_bf16,
)
