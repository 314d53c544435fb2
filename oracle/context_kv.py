"""Plain float64 CPU oracle of the multi-layer context K/V precompute.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
library and its binding never do, and nothing here is shared with them.

What it computes is the vLLM page "qwen3_dflash",
``DFlashQwen3Model.precompute_and_store_context_kv`` with its helpers
``_build_context_kv_buffers``, ``_normalize_context_states``,
``_project_context_kv_token_major``, ``_project_context_kv`` and
``_normalize_context_k``: the new context rows of every draft layer are made
at once instead of inside each layer's forward.

* The raw context states are the ``fc`` output (``combine_hidden_states``):
  the features of the selected target layers, concatenated per row, times
  the ``fc`` weight (a ``ReplicatedLinear`` with no bias, from
  ``n_target_layers * target_hidden`` to ``hidden``).
* The raw context states are RMS-normalised over ``hidden``
  with the model's ``hidden_norm`` gain (``_normalize_context_states``).
* One projection with the K/V rows of every layer's fused q|k|v weight gives
  each layer's context K and V (``_build_context_kv_buffers`` stacks the rows
  after ``q_size`` of each layer; ``_project_context_kv_token_major``).
* Each K head is RMS-normalised over ``head_dim`` with that layer's k_norm
  gain (``_normalize_context_k``: one grouped norm, weight chosen by layer),
  then rotated (neox, the layers' shared RoPE) at the context positions.
* V is left raw. Each layer's K and V rows are appended to that layer's cache
  after its valid rows (the per-layer cache insert).

Each step uses only the primitives of ``ref_fp64`` (float64 matmul,
RMSNorm, RoPE); its pins live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

from .ref_fp64 import OracleCache, _f64, linear, rms_norm, rope


def combine_hidden_states(aux_states, w_fc):
    """The ``fc`` projection of the concatenated target-layer features:
    ``aux_states [rows, fc_in] . w_fc^T`` with ``w_fc [hidden, fc_in]``."""
    return linear(_f64(aux_states), _f64(w_fc))


def context_kv_precompute(cfg, weights, caches: Sequence[OracleCache], context_states, ctx_offsets,
                          positions) -> List[OracleCache]:
    """Context K/V of every draft layer, appended to each layer's cache.

    ``cfg`` has ``hidden, n_layers, n_kv_heads, head_dim, rope_theta,
    rms_eps``. ``weights`` has ``hidden_norm [H]``, ``w_kv [L, 2*nkv*d, H]``
    (layer l: its K rows, then its V rows) and ``k_norm [L, d]``.
    ``context_states [sum n_b, H]`` packs each sequence's raw context rows,
    sequence b owning rows ``ctx_offsets[b] : ctx_offsets[b+1]``, whose
    positions are ``positions`` at the same rows. Returns the L new caches."""
    H, Ln = cfg.hidden, cfg.n_layers
    if len(caches) != Ln:
        raise ValueError("one cache per layer")
    C = _f64(context_states).reshape(-1, H)
    normed = rms_norm(C, weights.hidden_norm, cfg.rms_eps)
    return [append_layer_kv(cfg, caches[layer], linear(normed, _f64(weights.w_kv[layer])),
                            weights.k_norm[layer], ctx_offsets, positions)
            for layer in range(Ln)]


def append_layer_kv(cfg, cache: OracleCache, kv, k_norm, ctx_offsets, positions) -> OracleCache:
    """One layer's part after the projection: ``kv [sum n_b, 2*nkv*d]`` holds
    that layer's K heads then V heads per context row. K is RMS-normalised with
    the layer's ``k_norm`` gain and rotated at the row positions; V stays raw;
    both are appended after each sequence's valid rows of a copy of ``cache``."""
    nkv, d = cfg.n_kv_heads, cfg.head_dim
    offs = [int(o) for o in ctx_offsets]
    pos = np.asarray(positions, dtype=np.int64)
    new = cache.copy()
    for b in range(len(offs) - 1):
        rows = kv[offs[b]:offs[b + 1]]
        k = rows[:, :nkv * d].reshape(-1, nkv, d).transpose(1, 0, 2)
        v = rows[:, nkv * d:].reshape(-1, nkv, d).transpose(1, 0, 2)
        k = rms_norm(k, _f64(k_norm), cfg.rms_eps)
        k = rope(k, pos[offs[b]:offs[b + 1]], cfg.rope_theta)
        new.k[b] = np.concatenate([new.k[b], k], axis=1)
        new.v[b] = np.concatenate([new.v[b], v], axis=1)
    return new
