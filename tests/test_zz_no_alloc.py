"""dflash_attn_step_noalloc, the layer step for callers that cannot allocate
device memory, against dflash_attn_step on the same inputs.

Both run the same kernels; only where the step's scratch lives differs (the
library's per-device buffer instead of the caller's workspace), so outputs,
cache rows and lengths must agree bit for bit. Two calls in a row, the second
with a smaller input: the buffer keeps the first call's contents, and a step
that read scratch it had not written would differ. The output is also held to
the oracle at the fp64 tolerance, a step near the buffer's size is compared,
and one past it is refused with nothing changed."""
import numpy as np
import pytest
import torch

from harness import assert_close, cache_bits, make_cache, make_layer, raw_bits, run_oracle, step_inputs, to64
from workload import LayerConfig, make_case

pytestmark = pytest.mark.gpu


def cfg(**kw):
    base = dict(name="NA", batch=5, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                dtype="bf16", cached_len=(0, 700), new_ctx=(0, 20), accept=(0, 16), config_id=91)
    base.update(kw)
    return LayerConfig(**base)


def both_ways(layer, case):
    """The same step through both entry points on two identical caches."""
    hs, th, pos = step_inputs(case)
    cache_a, cache_b = make_cache(case), make_cache(case)
    out_a = layer.step(hs, th, case.ctx_offsets, pos, cache_a)
    out_b = torch.full_like(out_a, float("nan"))
    layer.step_noalloc(hs, th, case.ctx_offsets, pos, cache_b, out=out_b)
    torch.cuda.synchronize()
    return (out_a, cache_a), (out_b, cache_b)


def assert_same(a, b):
    (out_a, cache_a), (out_b, cache_b) = a, b
    np.testing.assert_array_equal(raw_bits(out_b), raw_bits(out_a))
    assert cache_b.lengths.tolist() == cache_a.lengths.tolist()
    for x, y in zip(cache_bits(cache_b), cache_bits(cache_a)):
        np.testing.assert_array_equal(x, y)


def test_noalloc_matches_the_workspace_step_twice_in_a_row():
    first = make_case(cfg(), seed=3)
    second = make_case(cfg(batch=2, cached_len=(0, 150), new_ctx=(0, 5)), seed=3)
    for name in ("w_qkv", "w_o", "q_norm", "k_norm"):  # one layer serves both calls
        np.testing.assert_array_equal(getattr(first.weights, name), getattr(second.weights, name))
    layer = make_layer(first)
    for case in (first, second):
        a, b = both_ways(layer, case)
        assert_same(a, b)
        ref, _ = run_oracle(case)
        assert_close(to64(b[0]), ref, "bf16", f"noalloc step, batch {case.batch}")
        assert b[1].lengths.tolist() == case.total_len.tolist()
    layer.close()


def test_noalloc_fp32_and_separate_append():
    case = make_case(cfg(dtype="fp32", hidden=256, n_q_heads=4, head_dim=64, block_size=8, batch=3,
                         cached_len=(0, 200), config_id=92), seed=1)
    layer = make_layer(case)
    for mode in ("auto", "separate"):
        layer.set_append_mode(mode)
        a, b = both_ways(layer, case)
        assert_same(a, b)
        ref, _ = run_oracle(case)
        assert_close(to64(b[0]), ref, "fp32", f"noalloc step, fp32, {mode}")
    layer.close()


def test_noalloc_near_and_past_the_buffer_size():
    """32 query heads of head_dim 128 over 8 KV heads: 120 sequences need
    about 40 MB of scratch (inside the 64 MiB buffer), 256 need about 76 MB
    (refused before anything runs)."""
    from block_diffusion_draft_qkv_amd import DFlashError, _lib
    big = cfg(batch=120, n_q_heads=32, n_kv_heads=8, cached_len=(0, 40), new_ctx=(0, 2), config_id=93)
    case = make_case(big, seed=0)
    layer = make_layer(case)
    a, b = both_ways(layer, case)
    assert_same(a, b)
    over = make_case(big.replace(batch=256), seed=0)
    hs, th, pos = step_inputs(over)
    cache = make_cache(over)
    before = cache_bits(cache)
    lens = cache.lengths.copy()
    out = torch.zeros((over.batch * 16, over.cfg.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(DFlashError) as e:
        layer.step_noalloc(hs, th, over.ctx_offsets, pos, cache, out=out)
    assert e.value.status == _lib.DFLASH_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert cache.lengths.tolist() == lens.tolist()
    assert torch.count_nonzero(out).item() == 0
    for x, y in zip(cache_bits(cache), before):
        np.testing.assert_array_equal(x, y)
    # the workspace step still takes it
    layer.step(hs, th, over.ctx_offsets, pos, cache)
    assert cache.lengths.tolist() == over.total_len.tolist()
    layer.close()
