"""Plain float64 CPU oracle of one DFlash draft-attention layer step and of the
draft cache crop.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
library and its binding never do, and nothing here is shared with them.

What it computes is the layer as the pages define it, evaluated exactly in
float64 with numpy (matmul, exp, cos and sin are the only library primitives):

* Q/K/V come from the draft block (``hidden_states``: one anchor plus mask
  tokens); K/V also come from the projected target context (``target_hidden``),
  with the same ``k_proj``/``v_proj`` weights, and the two K/V streams are
  concatenated along the sequence axis, context first.
  [vLLM "qwen3_dflash" API page: ``DFlashQwen3Attention.forward`` (fused
  qkv_proj, split q|k|v); "DFlash源码导读（二）" section 2 (dual-stream K/V
  concat); NeMo "draft_qwen3" page: ``Qwen3DFlashAttention`` docstring.]
* q and k are RMS-normalised per head over ``head_dim`` before RoPE, v is not.
  ["DFlash源码导读（二）" section 1 (QK-RMSNorm); vLLM page,
  ``DFlashQwen3Attention.forward`` ("Per-head RMSNorm").]
* RoPE is neox style (the two halves of a head are rotated as pairs); keys take
  every position of the window, the block's queries take its last ``q_len``
  positions. [vLLM page, ``is_neox_style=True``; NeMo page,
  ``apply_rotary_pos_emb``; "DFlash源码导读（二）" section 3.]
* Attention is non-causal grouped-query softmax attention with
  ``scaling = head_dim ** -0.5``; an optional sliding window keeps key t for the
  query that sits at key index ``k_len - q_len + i`` iff ``|Δ| < window``.
  [NeMo page: ``Qwen3DFlashAttention.scaling``, ``_sliding_window_mask``;
  "DFlash源码导读（二）" section "关键设计：非因果的块扩散注意力".]
* The cache keeps the context and block K/V of every step (post-norm,
  post-RoPE K; raw V) and is cropped back to the accepted prefix after a round.
  ["DFlash源码导读（二）" section 4 (cache update and ``crop``).]
* ``o_proj`` maps the concatenated heads back to ``hidden`` (no bias).
  [vLLM page, ``DFlashQwen3Attention.__init__`` / ``forward``.]

Every pin of this module lives in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def linear(x, w) -> np.ndarray:
    """``y = x · wᵀ`` for an ``nn.Linear`` weight ``w`` of shape ``[out, in]``,
    without bias (vLLM page, ``DFlashQwen3Attention.__init__``: ``bias`` is
    ``attention_bias``, False for Qwen3)."""
    return _f64(x) @ _f64(w).T


def rms_norm(x, gain, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: ``x / sqrt(mean(x**2) + eps) * gain``.

    The pages name the op (``Qwen3RMSNorm(head_dim, eps=rms_norm_eps)`` in
    "DFlash源码导读（二）" section 1; ``variance_epsilon`` on the vLLM page) but
    do not print its formula; eps is read as added to the mean square under the
    root, the standard RMSNorm definition."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(gain)


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Rotary frequencies ``theta ** (-2t / head_dim)`` for t < head_dim/2,
    evaluated in float64 (the NeMo page's ``_apply`` keeps them fp32 so that a
    bf16 cast cannot dephase them; float64 is the exact value they stand for)."""
    t = np.arange(head_dim // 2, dtype=np.float64)
    return float(theta) ** (-2.0 * t / head_dim)


def rope(x, positions, theta: float) -> np.ndarray:
    """Neox-style rotary embedding of ``x[..., n, d]`` at ``positions[n]``.

    The head is split into halves ``[x1 | x2]``; element t of x1 is rotated with
    element t of x2 by angle ``pos * inv_freq[t]``:
    ``x1' = x1 cos - x2 sin``, ``x2' = x2 cos + x1 sin``
    (vLLM page: ``get_rope(..., is_neox_style=True)``)."""
    x = _f64(x)
    d = x.shape[-1]
    half = d // 2
    ang = _f64(positions)[:, None] * rope_inv_freq(d, theta)[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def window_keep(q_len: int, k_len: int, window: int) -> np.ndarray:
    """Boolean ``[q_len, k_len]`` visibility of key t for block query i.

    No window (0 or None): every key is visible (non-causal, no mask). With a
    window W, query row i sits at key index ``k_len - q_len + i`` and key t is
    kept iff ``|(k_len - q_len + i) - t| < W``: both bounds strict, the band
    symmetric (NeMo page, ``_sliding_window_mask``)."""
    if not window:
        return np.ones((q_len, k_len), dtype=bool)
    qpos = k_len - q_len + np.arange(q_len)
    delta = qpos[:, None] - np.arange(k_len)[None, :]
    return np.abs(delta) < window


def attention(q, k, v, keep, scaling: float) -> np.ndarray:
    """Non-causal grouped-query softmax attention.

    ``q[nq, n, d]``, ``k[nkv, T, d]``, ``v[nkv, T, d]``, ``keep[n, T]``.
    Query head h reads KV head ``h // (nq // nkv)`` (contiguous groups of
    ``num_key_value_groups`` query heads, "DFlash源码导读（二）" section 1);
    scores are ``scaling * <q, k>`` (NeMo page, ``scaling``); masked keys get
    weight 0; the softmax subtracts the row max before exponentiating."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, nkv = q.shape[0], k.shape[0]
    groups = nq // nkv
    out = np.empty((nq, q.shape[1], v.shape[2]), dtype=np.float64)
    for h in range(nq):
        j = h // groups
        s = scaling * (q[h] @ k[j].T)
        s = np.where(keep, s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        a = np.exp(s)
        a = a / a.sum(axis=-1, keepdims=True)
        out[h] = a @ v[j]
    return out


@dataclass
class OracleCache:
    """Logical draft KV cache: per sequence, ``k[b]`` and ``v[b]`` of shape
    ``[n_kv, len_b, head_dim]`` in float64. The rows are exactly the valid
    prefix, so ``len_b`` is the array length ("DFlash源码导读（二）" section 4:
    ``past_key_values.update`` appends, ``crop`` truncates)."""

    k: List[np.ndarray] = field(default_factory=list)
    v: List[np.ndarray] = field(default_factory=list)

    @classmethod
    def from_arrays(cls, ks: Sequence, vs: Sequence) -> "OracleCache":
        return cls([_f64(a).copy() for a in ks], [_f64(a).copy() for a in vs])

    @property
    def lengths(self) -> List[int]:
        return [int(a.shape[1]) for a in self.k]

    def copy(self) -> "OracleCache":
        return OracleCache([a.copy() for a in self.k], [a.copy() for a in self.v])


def crop(cache: OracleCache, seq: int, new_len: int) -> OracleCache:
    """Rewind sequence ``seq`` of the cache to its first ``new_len`` rows.

    Crop only truncates: the rows kept are unchanged and ``new_len`` must lie in
    ``[0, len]`` ("DFlash源码导读（二）" section 4: after verification the loop
    crops the draft cache to the accepted prefix; NeMo page,
    ``assert_target_supports_rollback``: a rewind drops KV rows)."""
    if not 0 <= seq < len(cache.k):
        raise IndexError(f"sequence {seq} out of range")
    cur = cache.k[seq].shape[1]
    if not 0 <= new_len <= cur:
        raise ValueError(f"crop to {new_len} outside [0, {cur}]")
    out = cache.copy()
    out.k[seq] = out.k[seq][:, :new_len].copy()
    out.v[seq] = out.v[seq][:, :new_len].copy()
    return out


def layer_step(cfg, weights, cache: OracleCache, hidden_states, target_hidden,
               ctx_offsets, positions, o_input=None):
    """One draft-attention layer step for a batch of sequences.

    ``cfg`` has ``hidden, n_q_heads, n_kv_heads, head_dim, block_size,
    rope_theta, rms_eps, sliding_window``. ``weights`` has ``w_q [nq*d, H]``,
    ``w_k, w_v [nkv*d, H]``, ``w_o [H, nq*d]``, ``q_norm, k_norm [d]``.
    ``hidden_states [B*bs, H]`` is the draft block of every sequence;
    ``target_hidden [sum n_b, H]`` packs each sequence's new context rows,
    sequence b owning rows ``ctx_offsets[b] : ctx_offsets[b+1]``. ``positions``
    holds, for sequence b at offset ``ctx_offsets[b] + b*bs``, the positions of
    its window ``[new context | block]`` (``n_b + bs`` entries).

    Returns ``(out [B*bs, H], new_cache)``; the new cache has every new context
    and block row appended (post-norm post-RoPE K, raw V). ``o_input``, if
    given, maps the attention output rows ``[bs, nq*d]`` to what ``o_proj``
    multiplies (the identity when absent)."""
    H = cfg.hidden
    nq, nkv, d, bs = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_size
    if nq % nkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    scaling = d ** -0.5
    X = _f64(hidden_states).reshape(-1, H)
    C = _f64(target_hidden).reshape(-1, H) if target_hidden is not None else np.zeros((0, H))
    offs = [int(o) for o in ctx_offsets]
    pos_all = np.asarray(positions, dtype=np.int64)
    B = len(offs) - 1
    out = np.empty((B * bs, H), dtype=np.float64)
    new = cache.copy()
    for b in range(B):
        n_b = offs[b + 1] - offs[b]
        Xb = X[b * bs:(b + 1) * bs]
        Cb = C[offs[b]:offs[b + 1]]
        win = pos_all[offs[b] + b * bs: offs[b] + b * bs + n_b + bs]

        def heads(y, n):  # [rows, n*d] -> [n, rows, d]
            return y.reshape(y.shape[0], n, d).transpose(1, 0, 2)

        q = heads(linear(Xb, weights.w_q), nq)
        k_blk = heads(linear(Xb, weights.w_k), nkv)
        v_blk = heads(linear(Xb, weights.w_v), nkv)
        k_ctx = heads(linear(Cb, weights.w_k), nkv)
        v_ctx = heads(linear(Cb, weights.w_v), nkv)

        q = rms_norm(q, weights.q_norm, cfg.rms_eps)
        k_new = rms_norm(np.concatenate([k_ctx, k_blk], axis=1), weights.k_norm, cfg.rms_eps)
        v_new = np.concatenate([v_ctx, v_blk], axis=1)

        k_new = rope(k_new, win, cfg.rope_theta)       # keys: the whole window
        q = rope(q, win[n_b:], cfg.rope_theta)         # queries: its last bs positions

        K = np.concatenate([new.k[b], k_new], axis=1)
        V = np.concatenate([new.v[b], v_new], axis=1)
        keep = window_keep(bs, K.shape[1], cfg.sliding_window)
        o = attention(q, K, V, keep, scaling)           # [nq, bs, d]
        o_rows = o.transpose(1, 0, 2).reshape(bs, nq * d)
        out[b * bs:(b + 1) * bs] = linear(o_rows if o_input is None else o_input(o_rows), weights.w_o)
        new.k[b], new.v[b] = K, V
    return out, new
