"""Seeded MLP and norm weights of a draft decoder layer, on top of a layer-step
case (workload.configs). MLP width: 12288 for the Qwen3-8B-shaped layer of
C2-C5 (three times its hidden size, Qwen3-8B's intermediate size); small
cases pass their own. Recipe: gate/up/down weights N(0, 0.02²), the two norm
gains 1 + 0.02·N(0, 1), rounded to the dtype; stream 6 of the case's
SeedSequence. Holds none of the method's arithmetic."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .configs import Case, round_bf16

QWEN3_8B_INTERMEDIATE = 12288


@dataclass
class MLPWeights:
    input_norm: np.ndarray  # [H]
    post_norm: np.ndarray   # [H]
    w_gate_up: np.ndarray   # [2I, H]: gate rows, then up rows
    w_down: np.ndarray      # [H, I]


def make_mlp_weights(case: Case, intermediate: int) -> MLPWeights:
    cfg = case.cfg
    H = cfg.hidden
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.config_id, case.seed, 6])))
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    input_norm = rnd(1.0 + 0.02 * rng.standard_normal(H, dtype=np.float32))
    post_norm = rnd(1.0 + 0.02 * rng.standard_normal(H, dtype=np.float32))
    w_gate_up = rnd(rng.standard_normal((2 * intermediate, H), dtype=np.float32) * np.float32(0.02))
    w_down = rnd(rng.standard_normal((H, intermediate), dtype=np.float32) * np.float32(0.02))
    return MLPWeights(input_norm, post_norm, w_gate_up, w_down)
