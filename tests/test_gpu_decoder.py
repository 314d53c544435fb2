"""GPU parity of the draft decoder layer (input_layernorm, the attention layer
step, residual add, post_attention_layernorm, SwiGLU MLP, residual add) and of
the row RMSNorm (the draft model's final norm) against the float64 oracle.

The output is the residual stream, which is not bounded in size, and it goes
through several bf16 roundings (the normed input, the attention output, the
residual sum, the normed sum, the MLP activation and the output, each moving a
value by up to 2^-8 of it). down_proj sums I bf16-rounded activations: at
I = 12288 that is ~3e-3 RMS of error with tails of a few times that over two
million outputs. Each element gets |err| <= 6e-2 + 2^-7 |ref|, and the whole
output rel-RMS <= 1e-2 (fp32: 2e-4 + 2^-20 |ref|, rel-RMS <= 1e-5)."""
import numpy as np
import pytest
import torch

import oracle
from harness import poison_workspaces  # noqa: E402
from harness import (cache_bits, check_cache_after_step, dev, errors, make_cache, raw_bits, step_inputs, to64,
                     torch_dtype)
from workload import LayerConfig, make_case, make_mlp_weights

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def assert_close_stream(got, ref, dtype, what):
    assert got.shape == ref.shape and np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    max_abs, rel_rms = errors(got, ref)
    print(f"[{what}] max abs {max_abs:.3e} rel-RMS {rel_rms:.3e}", flush=True)
    rel, absb = (2.0 ** -7, 6e-2) if dtype == "bf16" else (2.0 ** -20, 2e-4)
    excess = err - (rel * np.abs(ref) + absb)
    k = int(np.argmax(excess))
    assert excess.flat[k] <= 0, f"{what}: |err| {err.flat[k]:.3e} at |ref| {abs(ref.flat[k]):.3e}"
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
    out = dec.step(x, th, case.ctx_offsets, pos, cache)
    torch.cuda.synchronize()
    assert dec.poll_error() == 0
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
