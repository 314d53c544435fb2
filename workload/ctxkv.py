"""Seeded inputs for the multi-layer context K/V precompute.

Shapes: the draft layers of C2-C5 (hidden 4096, 8 KV heads, head_dim 128,
bf16) with L = 3 draft layers (the pages' DFlash config example extracts three
target layers, and a draft has one layer per extracted target layer).

* P1 tiny fp32: B=2, hidden 256, 2 layers, 2 KV heads, head_dim 64, cached
  rows U{0..40}, new context rows U{1..30}.
* P3 decode round: C3's batch, B=32 sequences with cached rows U{512..8192}
  and U{1..16} new context rows each (about 272 rows), 3 layers.
* P4 prefill: one 4096-row prompt into an empty cache, 3 layers.
* M1, M2: small bf16 cases for the MXFP8 projection (hidden 256 and 512, a
  multiple of 128): M1 2 layers, 2 KV heads, head_dim 64, rows U{1..30}; M2 3
  layers, 4 KV heads, head_dim 128, cached rows U{0..200}, new rows U{1..100}.

MXFP8 K/V weights (``make_mxfp8_kv_weights``) are drawn directly as bytes, not
quantised from anything: E4M3 fields sign ~ U{0,1}, exponent ~ the integer
nearest N(10, 1.2²) clipped to 1..15, mantissa ~ U{0..7} (6 at most where the
exponent is 15, which keeps clear of the NaN code), so element values sit
around 8..15; E8M0 scale bytes ~ U{116, 117}, i.e. 2^-11 or 2^-10, which
puts the weights near the bf16 recipe's N(0, 0.02²) (RMS about 0.018).

Recipe: K/V projection weights N(0, 0.02²); RMSNorm gains (hidden_norm and
every layer's k_norm) 1 + 0.02·N(0, 1); raw context states 4·N(0, 1) (the
scale hidden_norm removes); pre-existing cache rows N(0, 1); positions
L_b, L_b+1, … over each sequence's new context rows; every value rounded to
the config dtype and held as float32. Streams are SeedSequence([config_id,
seed, stream]) draws. This module holds none of the method's arithmetic.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import List, Union

import numpy as np

from .configs import Range, _draw, round_bf16


@dataclass(frozen=True)
class CtxKVConfig:
    name: str
    batch: int
    hidden: int
    n_layers: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    cached_len: Range
    new_ctx: Range
    rope_theta: float = 1e6
    rms_eps: float = 1e-6
    max_position: int = 4096 * 32
    config_id: int = 40

    def replace(self, **kw) -> "CtxKVConfig":
        return dataclasses.replace(self, **kw)


CTXKV_CONFIGS = {
    "P1": CtxKVConfig("P1", 2, 256, 2, 2, 64, "fp32", (0, 40), (1, 30), config_id=41),
    "P3": CtxKVConfig("P3", 32, 4096, 3, 8, 128, "bf16", (512, 8192), (1, 16), config_id=43),
    "P4": CtxKVConfig("P4", 1, 4096, 3, 8, 128, "bf16", 0, 4096, config_id=44),
    "M1": CtxKVConfig("M1", 2, 256, 2, 2, 64, "bf16", (0, 40), (1, 30), config_id=45),
    "M2": CtxKVConfig("M2", 3, 512, 3, 4, 128, "bf16", (0, 200), (1, 100), config_id=46),
}


@dataclass
class CtxKVWeights:
    hidden_norm: np.ndarray  # [H]
    w_kv: np.ndarray         # [L, 2*nkv*d, H]: layer l's K rows, then its V rows
    k_norm: np.ndarray       # [L, d]


@dataclass
class MXKVWeights:
    w_kv_codes: np.ndarray   # [L, 2*nkv*d, H] uint8 E4M3 codes (rows as CtxKVWeights.w_kv)
    w_kv_scales: np.ndarray  # [L, 2*nkv*d, H/32] uint8 E8M0 bytes, one per 32 consecutive k


@dataclass
class CtxKVCase:
    cfg: CtxKVConfig
    seed: int
    weights: CtxKVWeights
    context_states: np.ndarray   # [sum n_b, H] raw (before hidden_norm)
    ctx_offsets: np.ndarray      # [B+1] int32
    positions: np.ndarray        # [sum n_b] int32
    cached_len: np.ndarray       # [B] int32
    cache_k: List[List[np.ndarray]]  # [layer][sequence] -> [nkv, L_b, d]
    cache_v: List[List[np.ndarray]]

    @property
    def batch(self) -> int:
        return len(self.cached_len)

    @property
    def new_ctx(self) -> np.ndarray:
        return np.diff(self.ctx_offsets)

    def capacity(self, align: int = 64) -> int:
        t = int((self.cached_len + self.new_ctx).max()) if self.batch else 0
        return max(align, -(-t // align) * align)


def _rng(cfg: CtxKVConfig, seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.config_id, seed, stream])))


def make_ctxkv_case(cfg: Union[str, CtxKVConfig], seed: int = 0) -> CtxKVCase:
    if isinstance(cfg, str):
        cfg = CTXKV_CONFIGS[cfg]
    B, H, Ln, nkv, d = cfg.batch, cfg.hidden, cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    wr = _rng(cfg, seed, 0)
    hidden_norm = rnd(1.0 + 0.02 * wr.standard_normal(H, dtype=np.float32))
    w_kv = rnd(wr.standard_normal((Ln, 2 * nkv * d, H), dtype=np.float32) * np.float32(0.02))
    k_norm = rnd(1.0 + 0.02 * wr.standard_normal((Ln, d), dtype=np.float32))

    lr = _rng(cfg, seed, 3)
    L = _draw(lr, cfg.cached_len, B)
    n = _draw(lr, cfg.new_ctx, B)
    offs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    ctx = rnd(4.0 * _rng(cfg, seed, 2).standard_normal((int(offs[-1]), H), dtype=np.float32))
    pos = np.concatenate([np.arange(L[b], L[b] + n[b]) for b in range(B)]).astype(np.int32) \
        if B else np.zeros(0, np.int32)
    cr = _rng(cfg, seed, 4)
    ck = [[rnd(cr.standard_normal((nkv, int(L[b]), d), dtype=np.float32)) for b in range(B)]
          for _ in range(Ln)]
    cv = [[rnd(cr.standard_normal((nkv, int(L[b]), d), dtype=np.float32)) for b in range(B)]
          for _ in range(Ln)]
    return CtxKVCase(cfg, seed, CtxKVWeights(hidden_norm, w_kv, k_norm), ctx, offs, pos,
                     L.astype(np.int32), ck, cv)


def mx_bytes(r: np.random.Generator, shape):
    """E4M3 codes of ``shape`` and E8M0 scale bytes of ``shape[:-1] + (shape[-1] // 32,)``,
    drawn directly as bytes (recipe above)."""
    if shape[-1] % 32:
        raise ValueError("the reduction length must be a multiple of 32")
    sign = r.integers(0, 2, shape, dtype=np.int64)
    expo = np.clip(np.rint(r.normal(10.0, 1.2, shape)), 1, 15).astype(np.int64)
    mant = r.integers(0, 8, shape, dtype=np.int64)
    mant = np.where(expo == 15, np.minimum(mant, 6), mant)
    codes = ((sign << 7) | (expo << 3) | mant).astype(np.uint8)
    scales = r.integers(116, 118, tuple(shape[:-1]) + (shape[-1] // 32,)).astype(np.uint8)
    return codes, scales


def make_mxfp8_kv_weights(cfg: Union[str, CtxKVConfig], seed: int = 0) -> MXKVWeights:
    """Seeded MXFP8 K/V weights of ``cfg``'s shape, drawn as bytes (recipe above)."""
    if isinstance(cfg, str):
        cfg = CTXKV_CONFIGS[cfg]
    H, Ln, nkv, d = cfg.hidden, cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    return MXKVWeights(*mx_bytes(_rng(cfg, seed, 5), (Ln, 2 * nkv * d, H)))


@dataclass
class MXLayerWeights:
    w_qkv_codes: np.ndarray   # [(nq + 2 nkv) d, H] uint8, rows q | k | v
    w_qkv_scales: np.ndarray  # [(nq + 2 nkv) d, H / 32] uint8
    w_o_codes: np.ndarray     # [H, nq d] uint8
    w_o_scales: np.ndarray    # [H, nq d / 32] uint8


def make_mxfp8_layer_weights(cfg, seed: int = 0) -> MXLayerWeights:
    """Seeded MXFP8 q|k|v and o_proj weights of a layer config (a LayerConfig),
    drawn as bytes by the same recipe; q_norm / k_norm stay the bf16 case's."""
    H, nq, nkv, d = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.config_id, seed, 9])))
    wq, sq = mx_bytes(r, ((nq + 2 * nkv) * d, H))
    wo, so = mx_bytes(r, (H, nq * d))
    return MXLayerWeights(wq, sq, wo, so)


def make_fc_inputs(cfg: Union[str, CtxKVConfig], rows: int, seed: int = 0, target_layers: int = 3):
    """Inputs of the fc projection for ``rows`` context rows: the concatenated
    features of ``target_layers`` target layers ``[rows, target_layers * H]``
    ~ N(0, 1) and the fc weight ``[H, target_layers * H]`` ~ N(0, 0.02^2)
    (a target with the draft's hidden size, three extracted layers as in the
    pages' config example), rounded to the config dtype."""
    if isinstance(cfg, str):
        cfg = CTXKV_CONFIGS[cfg]
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    r = _rng(cfg, seed, 6)
    fc_in = target_layers * cfg.hidden
    w_fc = rnd(r.standard_normal((cfg.hidden, fc_in), dtype=np.float32) * np.float32(0.02))
    aux = rnd(r.standard_normal((rows, fc_in), dtype=np.float32))
    return aux, w_fc
