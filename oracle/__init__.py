"""Float64 CPU oracle of the DFlash draft-attention layer step, of the
multi-layer context K/V precompute (bf16 and MXFP8) and of the draft decoder
layer.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product (the HIP library and its Python binding) never imports it
and shares no code with it.
"""
from .ref_fp64 import (  # noqa: F401
    OracleCache,
    attention,
    crop,
    layer_step,
    linear,
    rms_norm,
    rope,
    rope_inv_freq,
    window_keep,
)
from .context_kv import combine_hidden_states, context_kv_precompute  # noqa: F401
from .decoder import decoder_layer_step, draft_forward, mlp, silu  # noqa: F401
from .mxfp8 import (  # noqa: F401
    context_kv_precompute_mxfp8,
    e4m3_encode,
    e4m3_value,
    e8m0_value,
    layer_step_mxfp8,
    mx_dequantize,
    mx_quantize,
    mxfp8_linear,
    round_bf16,
)
