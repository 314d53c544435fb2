"""Shared helpers of the GPU tests: put a seeded case on the device through the
binding, run the library, and compare with the oracle.

Tolerances (against the float64 oracle):
  fp32: max |err| <= 1e-4.
  bf16: max |err| <= 2e-2 and rel-RMS err <= 1e-2.
  Stored cache values (assert_close_stored): cache rows are not bounded in
  size and rounding to bf16 alone moves a value by up to 2^-8 of its
  magnitude (8 significand bits), so each element gets the bf16 bound plus
  that: |err| <= 2e-2 + 2^-8 |ref| (fp32: 1e-4 + 2^-20 |ref|), with the same
  rel-RMS bound.
Cache indexing, lengths and untouched rows: bit-exact.

Every handle the tests make has its workspace refilled with 0xFF bytes (NaN as
fp32 and as bf16) each time a step asks for it (poison_workspaces), so a kernel
that read scratch it had not written in the same step (a stale split partial,
say) would turn the result non-finite.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from workload import Case

CANARY_BF16 = 0x7FA5          # a NaN pattern: any read of a dead row poisons the result
CANARY_F32 = 0x7FC0A5A5


def torch_dtype(case: Case):
    return torch.bfloat16 if case.cfg.dtype == "bf16" else torch.float32


def dev(a, dtype, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device=device, dtype=dtype)


WORKSPACE_POISON = 0xFF


def poison_workspaces(handle):
    """Make ``handle.workspace(...)`` (used by step/append when no workspace is
    passed) return its buffer refilled with NaN bytes on every call."""
    orig = handle.workspace

    def workspace(*args, **kw):
        ws = orig(*args, **kw)
        ws.fill_(WORKSPACE_POISON)
        return ws

    handle.workspace = workspace
    return handle


def make_layer(case: Case):
    from block_diffusion_draft_qkv_amd import DFlashLayer, LayerShape
    cfg, w = case.cfg, case.weights
    dt = torch_dtype(case)
    shape = LayerShape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_size, dt,
                       cfg.rope_theta, cfg.rms_eps, cfg.sliding_window, cfg.max_position)
    return poison_workspaces(DFlashLayer(shape, dev(w.w_qkv, dt), dev(w.w_o, dt), dev(w.q_norm, dt),
                                         dev(w.k_norm, dt)))


def fill_canary(t: torch.Tensor):
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(CANARY_BF16)
    else:
        t.view(torch.int32).fill_(CANARY_F32)


def make_cache(case: Case, capacity: int = None):
    from block_diffusion_draft_qkv_amd import KVCache
    cfg = case.cfg
    dt = torch_dtype(case)
    cap = capacity or case.capacity()
    cache = KVCache(case.batch, cfg.n_kv_heads, cfg.head_dim, cap, dt)
    fill_canary(cache.k)
    fill_canary(cache.v)
    for b in range(case.batch):
        cache.write_prefix(b, dev(case.cache_k[b], dt), dev(case.cache_v[b], dt))
    return cache


def step_inputs(case: Case):
    dt = torch_dtype(case)
    hs = dev(case.hidden_states, dt)
    th = dev(case.target_hidden, dt) if case.target_hidden.size else None
    pos = torch.from_numpy(case.positions.astype(np.int32)).cuda()
    return hs, th, pos


def run_oracle(case: Case, cache: oracle.OracleCache = None, hidden=None, target=None, offsets=None,
               positions=None):
    if cache is None:
        cache = oracle.OracleCache.from_arrays(case.cache_k, case.cache_v)
    return oracle.layer_step(case.cfg, case.weights, cache,
                             case.hidden_states if hidden is None else hidden,
                             case.target_hidden if target is None else target,
                             case.ctx_offsets if offsets is None else offsets,
                             case.positions if positions is None else positions)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    den = float(np.sqrt(np.mean(ref * ref))) if ref.size else 1.0
    rel_rms = float(np.sqrt(np.mean(err * err))) / den if ref.size and den > 0 else 0.0
    return max_abs, rel_rms


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    max_abs, rel_rms = errors(got, ref)
    if dtype == "fp32":
        assert max_abs <= 1e-4, f"{what}: max abs {max_abs:.3e} > 1e-4"
    else:
        assert max_abs <= 2e-2 and rel_rms <= 1e-2, \
            f"{what}: max abs {max_abs:.3e} (<= 2e-2), rel-RMS {rel_rms:.3e} (<= 1e-2)"
    return max_abs, rel_rms


def assert_close_stored(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    rel, absb = (2.0 ** -8, 2e-2) if dtype == "bf16" else (2.0 ** -20, 1e-4)
    excess = err - (rel * np.abs(ref) + absb)
    worst = int(np.argmax(excess)) if err.size else 0
    assert not err.size or excess.flat[worst] <= 0, \
        f"{what}: |err| {err.flat[worst]:.3e} at |ref| {abs(ref.flat[worst]):.3e} > {rel:.2e}|ref| + {absb:.0e}"
    max_abs, rel_rms = errors(got, ref)
    assert rel_rms <= (1e-2 if dtype == "bf16" else 1e-5), f"{what}: rel-RMS {rel_rms:.3e}"
    return max_abs, rel_rms


def raw_bits(t: torch.Tensor) -> np.ndarray:
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).cpu().numpy()


def cache_bits(cache):
    """Raw bits of a contiguous cache in row-major form: K ``[B, nkv, cap, d]``
    and V transposed ``[B, nkv, d, cap]``."""
    return raw_bits(cache.k_rows()), raw_bits(cache.vt_rows())


def check_cache_after_step(case: Case, cache, before_k, before_v, new_cache: oracle.OracleCache):
    """New rows [L_b, T_b) match the oracle within the stored-value bound
    (assert_close_stored: V rows are raw projections, not bounded in size);
    every other row of K and V (the dead ones past T_b hold a NaN canary) is
    bit-identical to what it was; lengths equal T_b exactly."""
    L, T = case.cached_len, case.total_len
    assert cache.lengths.tolist() == T.tolist()
    k_bits, v_bits = cache_bits(cache)
    k_rows, vt_rows = cache.k_rows(), cache.vt_rows()
    for b in range(case.batch):
        lb, tb = int(L[b]), int(T[b])
        np.testing.assert_array_equal(k_bits[b, :, :lb], before_k[b, :, :lb])
        np.testing.assert_array_equal(k_bits[b, :, tb:], before_k[b, :, tb:])
        np.testing.assert_array_equal(v_bits[b, :, :, :lb], before_v[b, :, :, :lb])
        np.testing.assert_array_equal(v_bits[b, :, :, tb:], before_v[b, :, :, tb:])
        k_new = to64(k_rows[b, :, lb:tb])
        v_new = to64(vt_rows[b, :, :, lb:tb].transpose(1, 2))
        assert_close_stored(k_new, new_cache.k[b][:, lb:tb], case.cfg.dtype, f"cache K seq {b}")
        assert_close_stored(v_new, new_cache.v[b][:, lb:tb], case.cfg.dtype, f"cache V seq {b}")


def sampled_rows(n_rows: int, seed: int, n_random: int = 48, edge: int = 64, tile: int = 128) -> np.ndarray:
    """Rows to check of a large row-parallel result: the first and last `edge`
    rows, both rows on either side of every `tile`-row boundary (where the
    projection's row tiles meet), and `n_random` more drawn from the seed."""
    rows = [np.arange(min(edge, n_rows)), np.arange(max(0, n_rows - edge), n_rows)]
    b = np.arange(tile, n_rows, tile)
    rows += [b - 1, b]
    rows.append(np.random.default_rng(seed).choice(n_rows, min(n_random, n_rows), replace=False))
    return np.unique(np.concatenate(rows)).astype(np.int64)

