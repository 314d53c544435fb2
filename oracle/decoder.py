"""Plain float64 CPU oracle of one DFlash draft decoder layer.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
library and its binding never do, and nothing here is shared with them.

The layer is the NeMo page "draft_qwen3" ``Qwen3DFlashDecoderLayer``: the
block's noise stream passes ``input_layernorm``, the non-causal attention
(``layer_step``: the context rows enter only its K/V), a residual add,
``post_attention_layernorm``, ``mlp = Qwen3MLP`` and a second residual add. The
MLP is the gated one the vLLM page "qwen3_dflash" loads as ``gate_up_proj``
(``gate_proj`` and ``up_proj`` stacked) followed by ``down_proj``:
``down(silu(gate(m)) * up(m))``, ``silu(g) = g / (1 + e^-g)``. The pages
print the parts but not the body; this is the pre-norm residual order those
parts name, the order ``DFlashQwen3Model.forward`` threads the residual in.

Each step uses the primitives of ``ref_fp64`` (float64 matmul, RMSNorm, the
layer step); its pins live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import numpy as np

from .ref_fp64 import OracleCache, _f64, layer_step, linear, rms_norm


def silu(x) -> np.ndarray:
    """SiLU (the swish with slope 1): x * sigmoid(x), written so that large
    negative x gives 0 without overflow."""
    x = _f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, x / (1.0 + e), x * e / (1.0 + e))


def mlp(m, w_gate_up, w_down) -> np.ndarray:
    """Qwen3MLP on rows m: w_gate_up is [2 I, H] (gate rows then up rows),
    w_down [H, I]."""
    w = _f64(w_gate_up)
    inter = w.shape[0] // 2
    return linear(silu(linear(m, w[:inter])) * linear(m, w[inter:]), _f64(w_down))


def decoder_layer_step(cfg, weights, mlp_weights, cache: OracleCache, x, target_hidden, ctx_offsets, positions):
    """One decoder layer step. ``weights`` are the attention's (as for
    ``layer_step``); ``mlp_weights`` has ``input_norm [H]``, ``post_norm [H]``,
    ``w_gate_up [2I, H]``, ``w_down [H, I]``. ``x [B*bs, H]`` is the noise
    stream; the other arguments are those of ``layer_step``. Returns
    ``(out [B*bs, H], new_cache)``."""
    X = _f64(x)
    a = rms_norm(X, mlp_weights.input_norm, cfg.rms_eps)
    att, new = layer_step(cfg, weights, cache, a, target_hidden, ctx_offsets, positions)
    h = X + att
    m = rms_norm(h, mlp_weights.post_norm, cfg.rms_eps)
    return h + mlp(m, mlp_weights.w_gate_up, mlp_weights.w_down), new


def draft_forward(cfg, layers, caches, x, target_hidden, ctx_offsets, positions, final_norm):
    """The draft stack: the decoder layers in order, each with its own
    attention weights, MLP weights and cache, the stream of one layer feeding
    the next, then the final RMSNorm (vLLM page "qwen3_dflash",
    DFlashQwen3Model.forward: the layers, then self.norm). ``layers`` is a list
    of ``(weights, mlp_weights)``. Returns ``(out [B*bs, H], new caches)``."""
    h = _f64(x)
    new = []
    for (w, mw), cache in zip(layers, caches):
        h, c = decoder_layer_step(cfg, w, mw, cache, h, target_hidden, ctx_offsets, positions)
        new.append(c)
    return rms_norm(h, final_norm, cfg.rms_eps), new
