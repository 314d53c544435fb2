"""GPU parity of the draft decoder layer (input_layernorm, the attention layer
step, residual add, post_attention_layernorm, SwiGLU MLP, residual add) and of
the row RMSNorm (the draft model's final norm) against the float64 oracle.

The layer is checked piece by piece, each piece against the oracle fed the
kernel's own input for it (the intermediates the step leaves in its
workspace), so that each bound follows from the arithmetic of that piece alone
(u = 2^-8 for a bf16 result, 2^-24 for fp32):
  a    = RMSNorm(x) * input_norm       |err| <= (u + 2^-15) |ref|: one rounding,
                                        and at most 2^-15 relative for the fp32
                                        sum of squares, rsqrt and gain product
  att  = attention step on a           the layer step's own tolerance (bf16
                                        max-abs 2e-2 and rel-RMS 1e-2; fp32 1e-4)
  h    = x + att                        bit-exact: an fp32 add rounded once
  m    = RMSNorm(h) * post_norm         as a
  act  = silu(m Wg^T) * (m Wu^T)        one rounding of the product, plus what
                                        the fp32 sums of g and u can be off by:
                                        with MFMAs that each add c products and
                                        are accumulated one after another, a sum
                                        of K products errs by at most
                                        gamma = (K / c + c + 2) 2^-24 times the sum
                                        of the products' magnitudes S; silu has
                                        slope at most 1.1, so
                                        |err| <= u |ref| + (1 + u) (1.1 Eg (|up| + Eu)
                                        + |silu(g)| Eu) + 2^-16 |ref|
                                        with Eg = gamma S_g, Eu = gamma S_u (the
                                        last term covers the fp32 exp and divide)
  out  = h + act Wd^T                   |err| <= u |ref| + (1 + u) gamma (S_d + |h|)
and the whole output stays within rel-RMS 1e-2 (fp32 1e-5) of the float64
layer. The largest end-to-end difference is printed with its reference value.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import poison_workspaces  # noqa: E402
from harness import (assert_close, cache_bits, check_cache_after_step, dev, errors, make_cache, raw_bits,
                     step_inputs, to64, torch_dtype)
from workload import LayerConfig, make_case, make_mlp_weights

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


U = {"bf16": 2.0 ** -8, "fp32": 2.0 ** -24}
NORM_FP32 = 2.0 ** -15
MFMA_K = {"bf16": 32, "fp32": 4}  # products one MFMA adds (16x16x32 bf16, 16x16x4 fp32)


def gamma(k: int, dtype: str) -> float:
    c = MFMA_K[dtype]
    return (k // c + c + 2) * 2.0 ** -24


def check_bound(got, ref, bound, what):
    assert got.shape == ref.shape and np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    ratio = err / bound
    k = int(np.argmax(ratio))
    print(f"[{what}] max |err| {err.max():.3e}, worst err/bound {ratio.flat[k]:.3f} "
          f"(|err| {err.flat[k]:.3e}, |ref| {abs(ref.flat[k]):.3e})", flush=True)
    assert ratio.flat[k] <= 1.0, f"{what}: |err| {err.flat[k]:.3e} > bound {bound.flat[k]:.3e}"


def round_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    from workload import round_bf16
    return round_bf16(x32) if dtype == "bf16" else x32.astype(np.float32)


def check_pieces(case, mw, dec, ws, x, out):
    """Every piece of the step against the oracle fed the kernel's own input."""
    cfg, dt = case.cfg, case.cfg.dtype
    B, Mc, eps, u = case.batch, int(case.ctx_offsets[-1]), cfg.rms_eps, U[dt]
    r = {k: to64(dec.workspace_region(ws, B, Mc, k)) for k in ("a", "att", "h", "m", "act")}
    X = to64(x)
    a_ref = oracle.rms_norm(X, mw.input_norm, eps)
    check_bound(r["a"], a_ref, (u + NORM_FP32) * np.abs(a_ref) + 1e-300, f"{cfg.name} a")
    att_ref, _ = oracle.layer_step(cfg, case.weights, oracle.OracleCache.from_arrays(case.cache_k, case.cache_v),
                                   r["a"], case.target_hidden, case.ctx_offsets, case.positions)
    max_abs, rel = assert_close(r["att"], att_ref, dt, f"{cfg.name} attention sub-step")
    print(f"[{cfg.name} att] max abs {max_abs:.3e} rel-RMS {rel:.3e}", flush=True)
    h_exp = round_dtype(X.astype(np.float32) + r["att"].astype(np.float32), dt)
    np.testing.assert_array_equal(r["h"], h_exp.astype(np.float64), err_msg=f"{cfg.name} h = x + att")
    m_ref = oracle.rms_norm(r["h"], mw.post_norm, eps)
    check_bound(r["m"], m_ref, (u + NORM_FP32) * np.abs(m_ref) + 1e-300, f"{cfg.name} m")
    I = mw.w_down.shape[1]
    wg, wu = mw.w_gate_up[:I].astype(np.float64), mw.w_gate_up[I:].astype(np.float64)
    g, up = r["m"] @ wg.T, r["m"] @ wu.T
    am = np.abs(r["m"])
    gh = gamma(cfg.hidden, dt)
    e_g, e_u = gh * (am @ np.abs(wg).T), gh * (am @ np.abs(wu).T)
    sg = oracle.silu(g)
    act_ref = sg * up
    bound = u * np.abs(act_ref) + (1 + u) * (1.1 * e_g * (np.abs(up) + e_u) + np.abs(sg) * e_u) \
        + 2.0 ** -16 * np.abs(act_ref) + 1e-300
    check_bound(r["act"], act_ref, bound, f"{cfg.name} act")
    wd = mw.w_down.astype(np.float64)
    o_ref = r["h"] + r["act"] @ wd.T
    bound = u * np.abs(o_ref) + (1 + u) * gamma(I, dt) * (np.abs(r["act"]) @ np.abs(wd).T + np.abs(r["h"])) + 1e-300
    check_bound(to64(out), o_ref, bound, f"{cfg.name} out = h + act Wd^T")


def assert_close_stream(got, ref, dtype, what):
    """The whole output against the float64 layer: rel-RMS only (the pieces
    carry the per-element bounds); the largest difference is reported."""
    assert got.shape == ref.shape and np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    max_abs, rel_rms = errors(got, ref)
    k = int(np.argmax(err))
    print(f"[{what}] max abs {max_abs:.3e} at |ref| {abs(ref.flat[k]):.3e}, rel-RMS {rel_rms:.3e}", flush=True)
    assert rel_rms <= (1e-2 if dtype == "bf16" else 1e-5), f"{what}: rel-RMS {rel_rms:.3e}"
    return max_abs, rel_rms


def make_decoder(case, mw):
    from block_diffusion_draft_qkv_amd import DFlashDecoder, LayerShape
    cfg, w, dt = case.cfg, case.weights, torch_dtype(case)
    shape = LayerShape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_size, dt,
                       cfg.rope_theta, cfg.rms_eps, cfg.sliding_window, cfg.max_position)
    return poison_workspaces(DFlashDecoder(shape, mw.w_down.shape[1], dev(w.w_qkv, dt), dev(w.w_o, dt),
                                           dev(w.q_norm, dt), dev(w.k_norm, dt), dev(mw.input_norm, dt),
                                           dev(mw.post_norm, dt), dev(mw.w_gate_up, dt), dev(mw.w_down, dt)))


def small(**kw):
    base = dict(name="D", batch=5, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                dtype="bf16", cached_len=(0, 700), new_ctx=(0, 20), accept=(0, 16), config_id=61)
    base.update(kw)
    return LayerConfig(**base)


CASES = {
    "bf16_d128": (lambda: make_case(small(), seed=1), 1024),
    "fp32_d64": (lambda: make_case(small(dtype="fp32", head_dim=64, hidden=256, n_q_heads=4, block_size=8,
                                         config_id=62), seed=2), 512),
    "bf16_window": (lambda: make_case(small(sliding_window=300, cached_len=(200, 900), config_id=63), seed=3),
                    640),
    "C3": (lambda: make_case("C3", seed=0), 12288),
    # 512 rows: the gate/up projection in 256 x 192 tiles (i % 96 == 0) ...
    "bf16_wide_tiles": (lambda: make_case(small(batch=32, hidden=1024, cached_len=(0, 300), new_ctx=(0, 8),
                                                config_id=64), seed=4), 12288),
    # ... and, with i % 96 != 0 and a deep k, in two launches of 128-column tiles
    "bf16_two_launches": (lambda: make_case(small(batch=32, hidden=4096, n_q_heads=32, n_kv_heads=8,
                                                  cached_len=(0, 200), new_ctx=(0, 8), config_id=65), seed=5),
                          11008),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decoder_layer_matches_oracle(name):
    mk, inter = CASES[name]
    case = mk()
    mw = make_mlp_weights(case, inter)
    print(f"[{name}] batch {case.batch}, keys {int(case.total_len.sum())}, intermediate {inter}", flush=True)
    dec = make_decoder(case, mw)
    cache = make_cache(case)
    bk, bv = cache_bits(cache)
    x, th, pos = step_inputs(case)
    ws = dec.workspace(case.batch, int(case.ctx_offsets[-1]))  # NaN-poisoned
    out = dec.step(x, th, case.ctx_offsets, pos, cache, workspace=ws)
    torch.cuda.synchronize()
    assert dec.poll_error() == 0
    check_pieces(case, mw, dec, ws, x, out)
    ref, new = oracle.decoder_layer_step(case.cfg, case.weights, mw,
                                         oracle.OracleCache.from_arrays(case.cache_k, case.cache_v),
                                         case.hidden_states, case.target_hidden, case.ctx_offsets, case.positions)
    max_abs, rel = assert_close_stream(to64(out), ref, case.cfg.dtype, f"{name} out")
    print(f"[{name}] out max abs {max_abs:.3e} rel-RMS {rel:.3e}", flush=True)
    if name != "C3":
        check_cache_after_step(case, cache, bk, bv, new)
    dec.close()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_final_rms_norm_matches_oracle(dtype):
    from block_diffusion_draft_qkv_amd import rms_norm
    rng = np.random.default_rng(5)
    for rows, H in ((1, 64), (37, 4096), (300, 9216)):  # the last is longer than a thread's registers
        x = 3.0 * rng.standard_normal((rows, H)).astype(np.float32)
        g = (1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32)
        dt = torch.bfloat16 if dtype == "bf16" else torch.float32
        xd, gd = dev(x, dt), dev(g, dt)
        out = rms_norm(xd, gd, 1e-6)
        torch.cuda.synchronize()
        ref = oracle.rms_norm(to64(xd), to64(gd), 1e-6)
        max_abs, rel = errors(to64(out), ref)
        bound = 2.0 ** -8 * np.abs(ref) + (1e-6 if dtype == "fp32" else 1e-3)
        assert np.all(np.abs(to64(out) - ref) <= bound), (rows, H, max_abs)


def test_decoder_rejects_bad_steps_before_enqueueing():
    from block_diffusion_draft_qkv_amd import DFlashError
    case = make_case(small(batch=2, config_id=64), seed=4)
    mw = make_mlp_weights(case, 256)
    dec = make_decoder(case, mw)
    cache = make_cache(case)
    x, th, pos = step_inputs(case)
    out = torch.full_like(x, 7.0)
    lens = cache.lengths.copy()
    # a step past the capacity: the library refuses it before the first launch
    cache.lengths[0] = cache.capacity - 1
    with pytest.raises(DFlashError) as e:
        dec.step(x, th, case.ctx_offsets, pos, cache, out=out)
    assert e.value.status == 3
    cache.set_lengths(lens)
    # offsets that disagree with the rows given: refused by the binding
    big = case.ctx_offsets.copy()
    big[1:] += cache.capacity
    with pytest.raises(ValueError):
        dec.step(x, th, big, pos, cache, out=out)
    torch.cuda.synchronize()
    assert cache.lengths.tolist() == lens.tolist()
    assert torch.all(out == 7.0)


def test_two_layer_draft_stack_with_final_norm():
    """A two-layer draft stack (each layer its own weights and cache, the
    stream of one feeding the next) and the final norm, against the oracle."""
    from block_diffusion_draft_qkv_amd import rms_norm
    cfg = small(batch=3, config_id=65)
    cases = [make_case(cfg, seed=s) for s in (7, 8)]  # weights of two layers; inputs from the first
    case = cases[0]
    mws = [make_mlp_weights(c, 768) for c in cases]
    decs = [make_decoder(c, mw) for c, mw in zip(cases, mws)]
    caches = [make_cache(case), make_cache(case)]
    fin = (1.0 + 0.02 * np.random.default_rng(9).standard_normal(cfg.hidden)).astype(np.float32)
    from workload import round_bf16
    fin = round_bf16(fin)
    x, th, pos = step_inputs(case)
    h = x
    for dec, cache in zip(decs, caches):
        h = dec.step(h, th, case.ctx_offsets, pos, cache)
    out = rms_norm(h, dev(fin, torch.bfloat16), cfg.rms_eps)
    torch.cuda.synchronize()
    oc = oracle.OracleCache.from_arrays(case.cache_k, case.cache_v)
    ref, _ = oracle.draft_forward(cfg, [(c.weights, mw) for c, mw in zip(cases, mws)], [oc, oc.copy()],
                                  case.hidden_states, case.target_hidden, case.ctx_offsets, case.positions, fin)
    assert_close_stream(to64(out), ref, "bf16", "stack out")
    for d in decs:
        d.close()
