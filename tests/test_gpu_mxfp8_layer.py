"""GPU parity of the layer step in its MXFP8 configuration (block and context
rows quantised for the block-scaled q|k|v projection, the bf16 attention
output quantised for the block-scaled o_proj) against the float64 oracle.

The cache is checked as in the bf16 step:
- the new rows to the stored-value bound (the block and context rows are bf16
  inputs, so both sides take the same E4M3 codes);
- every other row bit-identical, and the lengths exact.

The output has a bound of its own. The attention output is quantised on the
fly, and the kernel's differs from the oracle's fp64 one by ~2^-9 relative
(P is rounded to bf16 for the P.V product, O to bf16). Where an E4M3 rounding
boundary of step s falls between the two values, the quantised o_proj inputs
differ by s. With a block maximum amax, s <= 2^-3 amax, and the two values
differ by |delta| <= ~2^-8 |o|. So the expected squared difference is at most
2 |delta| s ~ 2^-10 |o| amax, a few percent rel-RMS through o_proj in the worst
case. The bound is therefore:
- max-abs <= 5e-2 and rel-RMS <= 3e-2;
- the output must also sit at most half as far from the oracle as the oracle
  is from itself without the quantisation of the o_proj input, which a step
  that skipped that quantisation would fail.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import poison_workspaces  # noqa: E402
from harness import cache_bits, check_cache_after_step, dev, errors, make_cache, raw_bits, step_inputs, to64
from workload import LayerConfig, make_case, make_mxfp8_layer_weights

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def small(**kw):
    base = dict(name="MXS", batch=5, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                dtype="bf16", cached_len=(0, 700), new_ctx=(0, 20), accept=(0, 16), config_id=81)
    base.update(kw)
    return LayerConfig(**base)


class MXLayerOracleWeights:
    def __init__(self, mw, w):
        self.w_qkv_codes, self.w_qkv_scales = mw.w_qkv_codes, mw.w_qkv_scales
        self.w_o_codes, self.w_o_scales = mw.w_o_codes, mw.w_o_scales
        self.q_norm, self.k_norm = w.q_norm, w.k_norm


def mx_layer(case, mw):
    from block_diffusion_draft_qkv_amd import DFlashLayer, LayerShape
    c, dt = case.cfg, torch.bfloat16
    shape = LayerShape(c.hidden, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block_size, dt, c.rope_theta,
                       c.rms_eps, c.sliding_window, c.max_position)

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    return poison_workspaces(DFlashLayer(shape, u8(mw.w_qkv_codes), u8(mw.w_o_codes), dev(case.weights.q_norm, dt),
                                         dev(case.weights.k_norm, dt), w_qkv_scale=u8(mw.w_qkv_scales),
                                         w_o_scale=u8(mw.w_o_scales)))


def run_mx(case, seed=0):
    mw = make_mxfp8_layer_weights(case.cfg, seed)
    layer = mx_layer(case, mw)
    cache = make_cache(case)
    bk, bv = cache_bits(cache)
    hs, th, pos = step_inputs(case)
    print(f"[mxfp8 step {case.cfg.name}] B={case.batch} keys={int(case.total_len.sum())}", flush=True)
    out = layer.step(hs, th, case.ctx_offsets, pos, cache)
    torch.cuda.synchronize()
    args = (case.cfg, MXLayerOracleWeights(mw, case.weights), oracle.OracleCache.from_arrays(case.cache_k, case.cache_v),
            case.hidden_states, case.target_hidden if case.target_hidden.size else None, case.ctx_offsets,
            case.positions)
    ref, new = oracle.layer_step_mxfp8(*args)
    ref_noq, _ = oracle.layer_step_mxfp8(*args, quantise_o=False)
    got = to64(out)
    assert np.all(np.isfinite(got))
    max_abs, rel = errors(got, ref)
    _, rel_noq = errors(ref_noq, ref)
    print(f"[mxfp8 step {case.cfg.name}] max abs {max_abs:.3e} rel-RMS {rel:.3e} "
          f"(unquantised o_proj input: rel-RMS {rel_noq:.3e})", flush=True)
    assert max_abs <= 5e-2 and rel <= 3e-2, (max_abs, rel)
    assert rel <= 0.5 * rel_noq, (rel, rel_noq)
    check_cache_after_step(case, cache, bk, bv, new)
    assert layer.poll_error() == 0
    return layer, cache


CASES = {
    "d128": dict(),
    "d64": dict(head_dim=64, hidden=256, n_q_heads=8, n_kv_heads=2, block_size=8, config_id=82),
    "window": dict(sliding_window=300, cached_len=(200, 900), config_id=83),
    "no_context": dict(new_ctx=0, config_id=84),
    "many_ctx": dict(batch=7, new_ctx=(30, 70), config_id=85),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_mxfp8_layer_step_matches_oracle(name):
    run_mx(make_case(small(**CASES[name]), seed=2))


def test_mxfp8_layer_step_c3():
    run_mx(make_case("C3", seed=0))


def test_mxfp8_layer_rejects_what_it_does_not_support():
    from block_diffusion_draft_qkv_amd import DFlashError, DFlashLayer, LayerShape
    case = make_case(small(batch=2, config_id=86), seed=0)
    mw = make_mxfp8_layer_weights(case.cfg, 0)
    layer = mx_layer(case, mw)
    layer.set_append_mode("separate")
    cache = make_cache(case)
    bk = raw_bits(cache.k)
    hs, th, pos = step_inputs(case)
    with pytest.raises(DFlashError):
        layer.step(hs, th, case.ctx_offsets, pos, cache)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_bits(cache.k), bk)
    assert cache.lengths.tolist() == case.cached_len.tolist()
    c = case.cfg
    f32 = LayerShape(c.hidden, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block_size, torch.float32)
    u8 = torch.zeros(1, dtype=torch.uint8, device="cuda")
    with pytest.raises(DFlashError):
        DFlashLayer(f32, torch.from_numpy(mw.w_qkv_codes).cuda(), torch.from_numpy(mw.w_o_codes).cuda(),
                    dev(case.weights.q_norm, torch.float32), dev(case.weights.k_norm, torch.float32),
                    w_qkv_scale=u8, w_o_scale=u8)


def test_mxfp8_layer_step_paged_matches_oracle():
    """The MXFP8 step on a paged cache with shuffled blocks and a NaN canary:
    output to the bound above, new rows to the stored-value bound, every other
    slot untouched."""
    from test_gpu_paged import check_paged_after, make_paged
    case = make_case(small(batch=4, config_id=87), seed=4)
    mw = make_mxfp8_layer_weights(case.cfg, 3)
    layer = mx_layer(case, mw)
    cache = make_paged(case, seed=6)
    for b in range(case.batch):
        cache.reserve(b, int(case.total_len[b]))
    cache.sync()
    bk, bv = raw_bits(cache.k), raw_bits(cache.v)
    hs, th, pos = step_inputs(case)
    out = layer.step(hs, th, case.ctx_offsets, pos, cache)
    torch.cuda.synchronize()
    assert layer.poll_error() == 0
    args = (case.cfg, MXLayerOracleWeights(mw, case.weights), oracle.OracleCache.from_arrays(case.cache_k, case.cache_v),
            case.hidden_states, case.target_hidden if case.target_hidden.size else None, case.ctx_offsets,
            case.positions)
    ref, new = oracle.layer_step_mxfp8(*args)
    ref_noq, _ = oracle.layer_step_mxfp8(*args, quantise_o=False)
    max_abs, rel = errors(to64(out), ref)
    _, rel_noq = errors(ref_noq, ref)
    print(f"[mxfp8 paged step] max abs {max_abs:.3e} rel-RMS {rel:.3e} (unquantised: {rel_noq:.3e})", flush=True)
    assert max_abs <= 5e-2 and rel <= 3e-2 and rel <= 0.5 * rel_noq, (max_abs, rel, rel_noq)
    assert cache.lengths.tolist() == case.total_len.tolist()
    check_paged_after(cache, bk, bv, case.cached_len, case.total_len, new, "bf16", "mxfp8 paged")


def test_mxfp8_layer_step_c3_paged_is_bit_identical_to_contiguous():
    """Same tiles and the same order of every sum on either cache layout."""
    case = make_case("C3", seed=1)
    mw = make_mxfp8_layer_weights(case.cfg, 1)
    layer = mx_layer(case, mw)
    hs, th, pos = step_inputs(case)
    from test_gpu_paged import make_paged
    flat = make_cache(case)
    print("[mxfp8 C3 contiguous vs paged]", flush=True)
    out_flat = layer.step(hs, th, case.ctx_offsets, pos, flat).clone()
    cache = make_paged(case, seed=8)
    for b in range(case.batch):
        cache.reserve(b, int(case.total_len[b]))
    cache.sync()
    out = layer.step(hs, th, case.ctx_offsets, pos, cache)
    torch.cuda.synchronize()
    assert layer.poll_error() == 0
    assert torch.equal(out.view(torch.int16), out_flat.view(torch.int16))
    for b in (0, 13, 31):
        k, v = cache.read(b)
        kf, vf = flat.read(b)
        assert torch.equal(k.contiguous().view(torch.int16), kf.contiguous().view(torch.int16))
        assert torch.equal(v.contiguous().view(torch.int16), vf.contiguous().view(torch.int16))
