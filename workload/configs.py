"""The five layer-step workloads and their seeded input recipe.

Shapes (the draft layer is Qwen3-8B shaped from C2 on):

* C1 tiny fp32: B=1, hidden 256, 4 Q / 2 KV heads, head_dim 64, block 8,
  empty cache, 128 new context rows.
* C2 single bf16: B=1, hidden 4096, 32 Q / 8 KV heads, head_dim 128, block 16,
  2048 cached rows plus 16 new context rows.
* C3 ragged bf16: C2's layer at B=32, cached rows U{512..8192}, new context
  rows U{1..16}, accepted count U{0..16}.
* C4 long bf16: B=4, 32768 cached rows, 16 new context rows.
* C5 sliding window bf16: B=16, 16384 cached rows, window 4096, new context
  rows U{1..16}, accepted count U{0..16}.

Recipe: projection weights N(0, 0.02²); RMSNorm gains 1 + 0.02·N(0, 1);
``hidden_states``, ``target_hidden`` and the pre-existing cache K/V N(0, 1);
positions ``L_b, L_b+1, …`` over each sequence's window; every value rounded
to the config dtype (bf16 round-to-nearest-even) and then held as float32.
Streams are independent numpy ``SeedSequence([config_id, seed, stream])``
draws, so the weights of a config do not depend on its batch.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import List, Optional, Tuple, Union

import numpy as np

Range = Union[int, Tuple[int, int]]


@dataclass(frozen=True)
class LayerConfig:
    name: str
    batch: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                     # "fp32" or "bf16"
    cached_len: Range              # fixed, or inclusive (lo, hi) drawn per sequence
    new_ctx: Range
    accept: Range = (0, 16)
    rope_theta: float = 1e6
    rms_eps: float = 1e-6
    sliding_window: int = 0        # 0: full attention
    max_position: int = 4096 * 32
    config_id: int = 0

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "C1": LayerConfig("C1", 1, 256, 4, 2, 64, 8, "fp32", 0, 128, (0, 8), config_id=1),
    "C2": LayerConfig("C2", 1, 4096, 32, 8, 128, 16, "bf16", 2048, 16, (0, 16), config_id=2),
    "C3": LayerConfig("C3", 32, 4096, 32, 8, 128, 16, "bf16", (512, 8192), (1, 16), (0, 16),
                      config_id=3),
    "C4": LayerConfig("C4", 4, 4096, 32, 8, 128, 16, "bf16", 32768, 16, (0, 16), config_id=4),
    "C5": LayerConfig("C5", 16, 4096, 32, 8, 128, 16, "bf16", 16384, (1, 16), (0, 16),
                      sliding_window=4096, config_id=5),
}


def round_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) and return
    them as float32. Finite inputs only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _rng(cfg: LayerConfig, seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.config_id, seed, stream])))


def _draw(rng, r: Range, n: int) -> np.ndarray:
    if isinstance(r, tuple):
        return rng.integers(r[0], r[1] + 1, size=n).astype(np.int64)
    return np.full(n, int(r), dtype=np.int64)


@dataclass
class Weights:
    w_q: np.ndarray     # [nq*d, H]
    w_k: np.ndarray     # [nkv*d, H]
    w_v: np.ndarray     # [nkv*d, H]
    w_o: np.ndarray     # [H, nq*d]
    q_norm: np.ndarray  # [d]
    k_norm: np.ndarray  # [d]

    @property
    def w_qkv(self) -> np.ndarray:
        """Fused projection weight, rows ordered q heads, k heads, v heads."""
        return np.concatenate([self.w_q, self.w_k, self.w_v], axis=0)


@dataclass
class Case:
    cfg: LayerConfig
    seed: int
    weights: Weights
    hidden_states: np.ndarray      # [B*bs, H]
    target_hidden: np.ndarray      # [sum n_b, H]
    ctx_offsets: np.ndarray        # [B+1] int32
    positions: np.ndarray          # [sum(n_b + bs)] int32
    cached_len: np.ndarray         # [B] int32 (L_b)
    cache_k: List[np.ndarray]      # per sequence [nkv, L_b, d]
    cache_v: List[np.ndarray]      # per sequence [nkv, L_b, d]
    accept: np.ndarray             # [B] int32 accepted block tokens a_b

    @property
    def batch(self) -> int:
        return len(self.cached_len)

    @property
    def new_ctx(self) -> np.ndarray:
        return np.diff(self.ctx_offsets)

    @property
    def total_len(self) -> np.ndarray:
        """T_b = L_b + n_b + bs: key rows each sequence attends over."""
        return self.cached_len + self.new_ctx + self.cfg.block_size

    def capacity(self, align: int = 64) -> int:
        t = int(self.total_len.max()) if self.batch else 0
        return max(align, -(-t // align) * align)


def make_weights(cfg: LayerConfig, seed: int = 0) -> Weights:
    rng = _rng(cfg, seed, 0)
    H, nq, nkv, d = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: np.asarray(a, np.float32))

    def normal(shape, std):
        return rnd(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))

    w_q = normal((nq * d, H), 0.02)
    w_k = normal((nkv * d, H), 0.02)
    w_v = normal((nkv * d, H), 0.02)
    w_o = normal((H, nq * d), 0.02)
    q_norm = rnd(1.0 + 0.02 * rng.standard_normal(d, dtype=np.float32))
    k_norm = rnd(1.0 + 0.02 * rng.standard_normal(d, dtype=np.float32))
    return Weights(w_q, w_k, w_v, w_o, q_norm, k_norm)


def make_case(cfg: Union[str, LayerConfig], seed: int = 0, *, batch: Optional[int] = None,
              cached_len: Optional[Range] = None, new_ctx: Optional[Range] = None,
              weights: Optional[Weights] = None) -> Case:
    """Draw one seeded step input for ``cfg`` (a name in CONFIGS or a config)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if batch is not None:
        cfg = cfg.replace(batch=batch)
    if cached_len is not None:
        cfg = cfg.replace(cached_len=cached_len)
    if new_ctx is not None:
        cfg = cfg.replace(new_ctx=new_ctx)
    B, H, nkv, d, bs = cfg.batch, cfg.hidden, cfg.n_kv_heads, cfg.head_dim, cfg.block_size
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    w = weights if weights is not None else make_weights(cfg, seed)

    lens_rng = _rng(cfg, seed, 3)
    L = _draw(lens_rng, cfg.cached_len, B)
    n = _draw(lens_rng, cfg.new_ctx, B)
    acc = np.minimum(_draw(_rng(cfg, seed, 5), cfg.accept, B), bs)
    offs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)

    hs = rnd(_rng(cfg, seed, 1).standard_normal((B * bs, H), dtype=np.float32))
    th = rnd(_rng(cfg, seed, 2).standard_normal((int(offs[-1]), H), dtype=np.float32))

    pos = np.concatenate([np.arange(L[b], L[b] + n[b] + bs) for b in range(B)]).astype(np.int32) \
        if B else np.zeros(0, np.int32)

    crng = _rng(cfg, seed, 4)
    ck = [rnd(crng.standard_normal((nkv, int(L[b]), d), dtype=np.float32)) for b in range(B)]
    cv = [rnd(crng.standard_normal((nkv, int(L[b]), d), dtype=np.float32)) for b in range(B)]
    return Case(cfg, seed, w, hs, th, offs, pos, L.astype(np.int32), ck, cv, acc.astype(np.int32))
