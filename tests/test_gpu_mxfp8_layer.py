"""GPU parity of the layer step in its MXFP8 configuration (block and context
rows quantised for the block-scaled q|k|v projection, the bf16 attention
output quantised for the block-scaled o_proj) against the float64 oracle.

The cache is checked as in the bf16 step:
- the new rows to the stored-value bound (the block and context rows are bf16
  inputs, so both sides take the same E4M3 codes);
- every other row bit-identical, and the lengths exact.

The output is checked in two halves, each against what the oracle makes of
the kernel's own input for it, plus the whole:
1. o_proj of the kernel's own MXFP8 attention output (codes and scales read
   from the workspace): the fp64 product of those decoded rows with the
   decoded weight. One bf16 rounding (u = 2^-8) and an fp32 sum of K = nq d
   block-scaled products, 128 per scaled MFMA, accumulated one after another:
   |err| <= u |ref| + (1 + u) gamma S with gamma = (K / 128 + 130) 2^-24 and S
   the sum of the products' magnitudes; also the headline bf16 tolerance
   (max-abs 2e-2, rel-RMS 1e-2).
2. Those codes against mx_quantize(round_bf16(o)) of the oracle's float64
   attention output o. The kernel's o differs from it by an absolute amount
   of the order of 2^-9 of its row (P rounded to bf16 for P.V, Q to bf16, fp32
   sums): at most about 2^-8 A in a block whose largest value is A. A block
   scale differs only where the block maximum's two values straddle a power of
   two (allowed: 2 % of blocks; their codes are not compared). In a block with
   the same scale, an element with |o| >= A / 4 has an E4M3 step of at least
   2^-5 A, eight times that difference, so its code is at most one step from
   the oracle's, and off by one for at most 1/8 of those elements (the chance
   that a rounding boundary lies between the two values). Smaller elements
   have steps finer than the difference and are covered by the whole: the
   kernel's decoded MXFP8 output must be as close to the float64 o as the
   oracle's own MXFP8 rounding of it (rel-RMS within 10 %; a flipped code sits
   as close to the value as the other choice would).
3. The whole against the float64 layer: max-abs <= 5e-2 and rel-RMS <= 3e-2,
   and at most half as far from the oracle as the oracle is from itself without
   the quantisation of the o_proj input, which a step that skipped that
   quantisation would fail.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import poison_workspaces  # noqa: E402
from harness import (assert_close, cache_bits, check_cache_after_step, dev, errors, make_cache, raw_bits, step_inputs,
                     to64)
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


def check_halves(case, mw, layer, ws, out, o_star):
    """Halves 1 and 2 of the module docstring."""
    c = case.cfg
    B, Mc, Mq, od = case.batch, int(case.ctx_offsets[-1]), case.batch * c.block_size, c.n_q_heads * c.head_dim
    codes = layer.workspace_region(ws, B, Mc, "attn_out_mx").cpu().numpy()
    scales = layer.workspace_region(ws, B, Mc, "attn_out_mx_scales").cpu().numpy()
    scales = scales.transpose(1, 0, 2).reshape(Mq, od // 32)  # step-major -> [row][block]
    # 1. o_proj of the kernel's own codes
    o_in = oracle.mx_dequantize(codes, scales)
    assert np.all(np.isfinite(o_in)), "attention output codes: NaN or a NaN scale"
    wo = oracle.mx_dequantize(mw.w_o_codes, mw.w_o_scales)
    o_ref = o_in @ wo.T
    u, gam = 2.0 ** -8, (od // 128 + 130) * 2.0 ** -24
    bound = u * np.abs(o_ref) + (1 + u) * gam * (np.abs(o_in) @ np.abs(wo).T) + 1e-300
    got = to64(out)
    err = np.abs(got - o_ref)
    k = int(np.argmax(err / bound))
    print(f"[mxfp8 o_proj of own codes {c.name}] max abs {err.max():.3e}, worst err/bound "
          f"{(err / bound).flat[k]:.3f}", flush=True)
    assert np.all(err <= bound), f"o_proj: |err| {err.flat[k]:.3e} > bound {bound.flat[k]:.3e}"
    assert_close(got, o_ref, "bf16", "o_proj of the kernel's own MXFP8 attention output")
    # 2. the codes against the quantised float64 attention output
    b_star = oracle.round_bf16(o_star)
    exp_codes, exp_scales = oracle.mx_quantize(b_star)
    same_scale = scales == exp_scales                                  # [Mq, od / 32]
    frac_scale = 1.0 - same_scale.mean()
    amax = np.repeat(np.abs(b_star).reshape(Mq, od // 32, 32).max(-1), 32, axis=1)
    top = np.repeat(same_scale, 32, axis=1) & (np.abs(b_star) >= amax / 4)

    def ordinal(cd):  # E4M3 codes in value order (sign-magnitude), zero of either sign at 0
        cd = cd.astype(np.int64)
        return np.where(cd & 0x80, -(cd & 0x7F), cd & 0x7F)

    step = np.abs(ordinal(codes) - ordinal(exp_codes))[top]
    flips = float(np.mean(step > 0)) if step.size else 0.0
    dec_k, dec_o = oracle.mx_dequantize(codes, scales), oracle.mx_dequantize(exp_codes, exp_scales)
    rms_o = np.sqrt(np.mean(o_star ** 2))
    q_k, q_o = np.sqrt(np.mean((dec_k - o_star) ** 2)) / rms_o, np.sqrt(np.mean((dec_o - o_star) ** 2)) / rms_o
    print(f"[mxfp8 attention-output codes {c.name}] scales differing in {frac_scale:.3%} of blocks; elements "
          f">= amax/4: largest step {int(step.max()) if step.size else 0}, flipped {flips:.3%}; rel-RMS to the "
          f"float64 output {q_k:.4f} (oracle's own MXFP8 rounding {q_o:.4f}); all codes flipped "
          f"{np.mean(codes != exp_codes):.3%}", flush=True)
    assert frac_scale <= 0.02, frac_scale
    assert step.size == 0 or int(step.max()) <= 1, "a top-binade code more than one E4M3 step from the oracle's"
    assert flips <= 0.125, flips
    assert q_k <= 1.1 * q_o, (q_k, q_o)


def run_mx(case, seed=0):
    mw = make_mxfp8_layer_weights(case.cfg, seed)
    layer = mx_layer(case, mw)
    cache = make_cache(case)
    bk, bv = cache_bits(cache)
    hs, th, pos = step_inputs(case)
    print(f"[mxfp8 step {case.cfg.name}] B={case.batch} keys={int(case.total_len.sum())}", flush=True)
    B, Mc = case.batch, int(case.ctx_offsets[-1])
    ws = layer.workspace(B, Mc)  # NaN-poisoned
    out = layer.step(hs, th, case.ctx_offsets, pos, cache, workspace=ws)
    torch.cuda.synchronize()
    args = (case.cfg, MXLayerOracleWeights(mw, case.weights), oracle.OracleCache.from_arrays(case.cache_k, case.cache_v),
            case.hidden_states, case.target_hidden if case.target_hidden.size else None, case.ctx_offsets,
            case.positions)
    o_rows = []
    ref, new = oracle.layer_step_mxfp8(*args, o_rows_out=o_rows)
    check_halves(case, mw, layer, ws, out, np.concatenate(o_rows))
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
