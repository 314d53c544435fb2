"""Seeded synthetic inputs for the DFlash draft-attention layer step.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the layer's arithmetic. Both the oracle-side tests and the HIP
side (tests, bench) take their inputs from here.
"""
from .configs import (  # noqa: F401
    CONFIGS,
    Case,
    LayerConfig,
    Weights,
    make_case,
    round_bf16,
)
from .ctxkv import (  # noqa: F401
    CTXKV_CONFIGS,
    CtxKVCase,
    CtxKVConfig,
    CtxKVWeights,
    MXKVWeights,
    MXLayerWeights,
    make_ctxkv_case,
    make_fc_inputs,
    make_mxfp8_kv_weights,
    make_mxfp8_layer_weights,
)
from .decoder import QWEN3_8B_INTERMEDIATE, MLPWeights, make_mlp_weights  # noqa: F401
