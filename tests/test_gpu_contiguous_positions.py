"""Steps without a position array: the kernels then rotate every window at the
contiguous positions len_b, len_b + 1, ... (what a draft that continues its
sequence passes). The workload's positions are exactly those, so the layer
step (both append paths, bf16 and fp32, with a window), the MXFP8 layer step,
the decoder step and the multi-layer precompute must give bit-identical
outputs and caches with positions=None and with the explicit array; and a
window that would pass max_position is refused before anything runs."""
import numpy as np
import pytest
import torch

from harness import cache_bits, dev, make_cache, make_layer, step_inputs
from test_gpu_parity import small
from workload import CTXKV_CONFIGS, make_case, make_ctxkv_case

pytestmark = pytest.mark.gpu

CASES = {
    "bf16": dict(),
    "fp32_d64": dict(dtype="fp32", head_dim=64, hidden=256, block_size=8, config_id=31),
    "bf16_window": dict(sliding_window=300, cached_len=(200, 900), config_id=32),
    "no_context": dict(new_ctx=(0, 0), config_id=33),
}


def both_ways(step, case, make):
    """Run `step` with the explicit positions and with None on two identical
    caches; return (out, cache bits) of each."""
    res = []
    for use_pos in (True, False):
        cache = make()
        hs, th, pos = step_inputs(case)
        out = step(hs, th, case.ctx_offsets, pos if use_pos else None, cache)
        torch.cuda.synchronize()
        res.append((out.clone(), cache_bits(cache), cache.lengths.copy()))
    return res


@pytest.mark.parametrize("mode", ["fused", "separate"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_layer_step_without_positions_is_bit_identical(name, mode):
    case = make_case(small(**CASES[name]), seed=5)
    layer = make_layer(case)
    layer.set_append_mode(mode)
    (o1, c1, l1), (o2, c2, l2) = both_ways(layer.step, case, lambda: make_cache(case))
    assert torch.equal(o1, o2)
    np.testing.assert_array_equal(c1[0], c2[0])
    np.testing.assert_array_equal(c1[1], c2[1])
    assert l1.tolist() == l2.tolist()
    assert layer.poll_error() == 0


def test_decoder_and_mxfp8_steps_without_positions_are_bit_identical():
    from test_gpu_decoder import make_decoder
    from test_gpu_mxfp8_layer import mx_layer
    from workload import make_mlp_weights, make_mxfp8_layer_weights
    case = make_case(small(config_id=34), seed=6)
    dec = make_decoder(case, make_mlp_weights(case, 1024))
    (o1, c1, _), (o2, c2, _) = both_ways(dec.step, case, lambda: make_cache(case))
    assert torch.equal(o1, o2) and np.array_equal(c1[0], c2[0]) and np.array_equal(c1[1], c2[1])
    mx = mx_layer(case, make_mxfp8_layer_weights(case.cfg, 2))
    (o1, c1, _), (o2, c2, _) = both_ways(mx.step, case, lambda: make_cache(case))
    assert torch.equal(o1, o2) and np.array_equal(c1[0], c2[0]) and np.array_equal(c1[1], c2[1])


def test_precompute_without_positions_is_bit_identical():
    from test_gpu_context_kv import make_caches, make_precompute
    pc = CTXKV_CONFIGS["P3"].replace(batch=4, hidden=512, n_kv_heads=2, cached_len=(0, 300), new_ctx=(1, 40),
                                     config_id=35)
    case = make_ctxkv_case(pc, seed=7)
    pre = make_precompute(case)
    got = []
    for use_pos in (True, False):
        caches = make_caches(case)
        pos = torch.from_numpy(case.positions).cuda() if use_pos else None
        pre.append(dev(case.context_states, torch.bfloat16), case.ctx_offsets, pos, caches)
        torch.cuda.synchronize()
        got.append([cache_bits(c) for c in caches])
    for a, b in zip(*got):
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


def test_window_past_max_position_is_refused_up_front():
    import dataclasses
    from block_diffusion_draft_qkv_amd import DFlashError, _lib
    cfg = small(cached_len=(100, 200), new_ctx=(2, 5), config_id=36)
    case = make_case(cfg, seed=8)
    last = int(case.total_len.max())  # the longest window's positions end at last - 1
    layer = make_layer(dataclasses.replace(case, cfg=cfg.replace(max_position=last - 1)))
    cache = make_cache(case)
    bk, bv = cache_bits(cache)
    lens = cache.lengths.copy()
    hs, th, _ = step_inputs(case)
    with pytest.raises(DFlashError) as e:
        layer.step(hs, th, case.ctx_offsets, None, cache)
    assert e.value.status == _lib.DFLASH_ERR_RANGE
    torch.cuda.synchronize()
    k, v = cache_bits(cache)
    assert np.array_equal(k, bk) and np.array_equal(v, bv) and cache.lengths.tolist() == lens.tolist()
    layer = make_layer(dataclasses.replace(case, cfg=cfg.replace(max_position=last)))
    layer.step(hs, th, case.ctx_offsets, None, cache)  # every position now inside the table
    torch.cuda.synchronize()
    assert layer.poll_error() == 0
