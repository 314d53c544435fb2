"""GPU parity of the HIP layer step against the float64 oracle on small seeded
cases that still span several key tiles, ragged tails, splits and the edge
cases of the method (empty cache, no new context, window bands, crop)."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
from harness import (assert_close, cache_bits, check_cache_after_step, make_cache, make_layer, raw_bits,
                     run_oracle, step_inputs, to64)
from workload import CONFIGS, LayerConfig, make_case

pytestmark = pytest.mark.gpu


def small(**kw):
    base = dict(name="S", batch=5, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                dtype="bf16", cached_len=(0, 700), new_ctx=(0, 20), accept=(0, 16), config_id=11)
    base.update(kw)
    return LayerConfig(**base)


def run_and_check(case, capacity=None, append_mode=None):
    layer = make_layer(case)
    if append_mode is not None:
        layer.set_append_mode(append_mode)
    cache = make_cache(case, capacity)
    bk, bv = cache_bits(cache)
    hs, th, pos = step_inputs(case)
    out = layer.step(hs, th, case.ctx_offsets, pos, cache)
    torch.cuda.synchronize()
    ref, new = run_oracle(case)
    errs = assert_close(to64(out), ref, case.cfg.dtype, f"{case.cfg.name} out")
    check_cache_after_step(case, cache, bk, bv, new)
    assert layer.poll_error() == 0
    return layer, cache, errs


APPEND_CASES = {
    "bf16_d128": dict(),
    "fp32_d128": dict(dtype="fp32", batch=3, config_id=12),
    "bf16_d64": dict(head_dim=64, hidden=256, block_size=8, config_id=13),
    "fp32_d64_mha": dict(dtype="fp32", head_dim=64, hidden=256, n_q_heads=4, n_kv_heads=4,
                         block_size=8, config_id=14),
    "bf16_window": dict(sliding_window=300, cached_len=(200, 900), config_id=15),
    "bf16_many_ctx": dict(batch=7, new_ctx=(30, 70), config_id=16),
}


@pytest.mark.parametrize("mode", ["fused", "separate"])
@pytest.mark.parametrize("name", sorted(APPEND_CASES))
def test_append_in_projection_epilogue_or_separate(name, mode):
    # The q|k|v projection either normalises, rotates and appends in its
    # epilogue (one head per tile) or leaves fp32 rows for the separate kernel;
    # both must match the oracle, cache rows included.
    run_and_check(make_case(small(**APPEND_CASES[name]), seed=3), append_mode=mode)


def test_c1_tiny_fp32():
    run_and_check(make_case("C1", seed=0))


@pytest.mark.parametrize("seed", [0, 1])
def test_ragged_bf16_d128(seed):
    run_and_check(make_case(small(), seed=seed))


def test_ragged_fp32_d128():
    run_and_check(make_case(small(dtype="fp32", batch=3, config_id=12), seed=0))


def test_ragged_bf16_d64():
    cfg = small(head_dim=64, hidden=256, n_q_heads=8, n_kv_heads=2, block_size=8, config_id=13)
    run_and_check(make_case(cfg, seed=0))


def test_ragged_fp32_d64_mha():
    cfg = small(dtype="fp32", head_dim=64, hidden=256, n_q_heads=4, n_kv_heads=4, block_size=8,
                config_id=14)
    run_and_check(make_case(cfg, seed=0))


def test_empty_cache_and_no_context():
    cfg = small(batch=3, cached_len=0, new_ctx=0, config_id=15)
    case = make_case(cfg, seed=0)
    assert case.target_hidden.shape[0] == 0
    run_and_check(case)


def test_single_sequence_split_over_many_groups():
    """One long sequence: the tiles of each KV head are spread over many
    work-groups, so every pair is merged from partials."""
    cfg = small(batch=1, cached_len=5000, new_ctx=7, config_id=16)
    run_and_check(make_case(cfg, seed=0))


@pytest.mark.parametrize("window", [1, 37, 100, 5000])
def test_sliding_window_bands(window):
    cfg = small(batch=4, cached_len=(200, 900), sliding_window=window, config_id=17)
    run_and_check(make_case(cfg, seed=window))


@pytest.mark.parametrize("edge", [-1, 0, 1])
@pytest.mark.parametrize("window", [15, 16, 17, 64, 100])
def test_window_band_edge_tiles(window, edge):
    """The band mask runs only on key tiles that start before T_b - W (or on
    every tile when W < block_size): T_b - W one key before, on and one key
    after the 64-key tile boundary at 128, with windows below, at and above
    the block size of 16."""
    T = window + 128 + edge
    cfg = small(batch=1, sliding_window=window, cached_len=T - 3 - 16, new_ctx=3,
                config_id=300 + 3 * window + edge)
    run_and_check(make_case(cfg, seed=window + edge))


def test_capacity_exactly_full():
    """T_b equal to the capacity for one sequence (last tile full, no slack)."""
    cfg = small(batch=2, cached_len=(100, 200), new_ctx=(5, 5), config_id=18)
    case = make_case(cfg, seed=0)
    cap = -(-int(case.total_len.max()) // 64) * 64
    case.cached_len[0] = cap - 5 - 16
    case.cache_k[0] = np.random.default_rng(0).standard_normal((2, cap - 21, 128)).astype(np.float32)
    case.cache_v[0] = np.random.default_rng(1).standard_normal((2, cap - 21, 128)).astype(np.float32)
    from workload import round_bf16
    case.cache_k[0] = round_bf16(case.cache_k[0])
    case.cache_v[0] = round_bf16(case.cache_v[0])
    L0 = int(case.cached_len[0])
    case.positions[:5 + 16] = np.arange(L0, L0 + 21)
    assert int(case.total_len[0]) == cap
    run_and_check(case, capacity=cap)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_capacity_changes_addresses_only(dtype):
    """The same step on caches of three capacities: the output and every
    valid cache row bit-identical (the capacity moves where a sequence's
    blocks start, nothing else)."""
    case = make_case(small(dtype=dtype, batch=4, config_id=25), seed=1)
    layer = make_layer(case)
    hs, th, pos = step_inputs(case)
    base = case.capacity()
    outs, rows = [], []
    for cap in (base, base + 64, base + 192):
        cache = make_cache(case, cap)
        print(f"[capacity {cap}]", flush=True)
        outs.append(layer.step(hs, th, case.ctx_offsets, pos, cache).clone())
        torch.cuda.synchronize()
        rows.append([cache.read(b) for b in range(case.batch)])
    bits = torch.int16 if dtype == "bf16" else torch.int32
    for o, r in zip(outs[1:], rows[1:]):
        assert torch.equal(o.view(bits), outs[0].view(bits))
        for (k, v), (k0, v0) in zip(r, rows[0]):
            assert torch.equal(k.contiguous().view(bits), k0.contiguous().view(bits))
            assert torch.equal(v.contiguous().view(bits), v0.contiguous().view(bits))


def test_max_batch():
    cfg = small(batch=256, hidden=128, n_q_heads=2, n_kv_heads=1, head_dim=64, block_size=4,
                cached_len=(0, 130), new_ctx=(0, 3), config_id=19)
    run_and_check(make_case(cfg, seed=0))


def test_steps_with_crop_match_oracle_rounds():
    """Two decode rounds: step, crop each sequence to its accepted prefix,
    step again; outputs and cache follow the oracle doing the same."""
    cfg = small(batch=4, config_id=20)
    case = make_case(cfg, seed=3)
    layer = make_layer(case)
    cache = make_cache(case)
    hs, th, pos = step_inputs(case)
    layer.step(hs, th, case.ctx_offsets, pos, cache)
    ref_cache = run_oracle(case)[1]
    for b in range(case.batch):
        new_len = int(case.cached_len[b] + case.new_ctx[b] + case.accept[b])
        cache.crop(b, new_len)
        ref_cache = oracle.crop(ref_cache, b, new_len)
    assert cache.lengths.tolist() == ref_cache.lengths
    # second round: fresh block and context, positions continue after the prefix
    case2 = make_case(cfg, seed=4)
    L2 = np.array(ref_cache.lengths)
    pos2 = np.concatenate([np.arange(L2[b], L2[b] + case2.new_ctx[b] + cfg.block_size)
                           for b in range(case.batch)]).astype(np.int32)
    hs2, th2, _ = step_inputs(case2)
    out2 = layer.step(hs2, th2, case2.ctx_offsets, torch.from_numpy(pos2).cuda(), cache)
    ref2, ref_cache2 = oracle.layer_step(cfg, case.weights, ref_cache, case2.hidden_states,
                                         case2.target_hidden, case2.ctx_offsets, pos2)
    assert_close(to64(out2), ref2, "bf16", "second step out")
    for b in range(case.batch):
        k, v = cache.read(b)
        assert_close(to64(k), ref_cache2.k[b], "bf16", f"second step cache K {b}")
        assert_close(to64(v), ref_cache2.v[b], "bf16", f"second step cache V {b}")


def test_crop_semantics_bit_exact():
    cfg = small(batch=2, config_id=21)
    case = make_case(cfg, seed=0)
    layer = make_layer(case)
    cache = make_cache(case)
    hs, th, pos = step_inputs(case)
    layer.step(hs, th, case.ctx_offsets, pos, cache)
    torch.cuda.synchronize()
    kb, vb = raw_bits(cache.k), raw_bits(cache.v)
    T = case.total_len
    cache.crop(0, int(T[0]))          # no-op
    cache.crop(1, 3)
    assert cache.lengths.tolist() == [int(T[0]), 3]
    np.testing.assert_array_equal(raw_bits(cache.k), kb)   # crop moves no data
    np.testing.assert_array_equal(raw_bits(cache.v), vb)
    from block_diffusion_draft_qkv_amd import DFlashError
    for seq, n in [(1, 4), (0, -1), (2, 0), (-1, 0)]:
        with pytest.raises(DFlashError):
            cache.crop(seq, n)
    assert cache.lengths.tolist() == [int(T[0]), 3]


def test_position_out_of_range_is_latched():
    case = make_case(small(batch=2, config_id=22), seed=0)
    layer = make_layer(case)
    cache = make_cache(case)
    hs, th, pos = step_inputs(case)
    pos[3] = 1 << 30
    layer.step(hs, th, case.ctx_offsets, pos, cache)
    assert layer.poll_error() == 4
    assert layer.poll_error() == 0   # cleared by the poll


def test_invalid_steps_change_nothing():
    from block_diffusion_draft_qkv_amd import DFlashError, _lib
    case = make_case(small(batch=2, config_id=23), seed=0)
    layer = make_layer(case)
    cache = make_cache(case)
    hs, th, pos = step_inputs(case)
    lens = cache.lengths.copy()
    out = torch.zeros((2 * 16, 512), dtype=torch.bfloat16, device="cuda")
    bad_offsets = list(case.ctx_offsets)
    bad_offsets[1] = bad_offsets[2] + 1   # decreasing
    # decreasing offsets: the binding refuses them, and so does the library
    # when called directly through the C ABI
    with pytest.raises(ValueError):
        layer.step(hs, th, bad_offsets, pos, cache, out=out)
    ws = layer.workspace(case.batch, int(case.ctx_offsets[-1]))
    c_offs = (C.c_int32 * 3)(*[int(o) for o in bad_offsets])
    st = _lib.lib().dflash_attn_step(layer._h, hs.data_ptr(), th.data_ptr(), c_offs, pos.data_ptr(),
                                     C.byref(cache.desc), out.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert st == _lib.DFLASH_ERR_SHAPE
    assert cache.lengths.tolist() == lens.tolist()
    with pytest.raises(DFlashError) as e:
        layer.step(hs, th, case.ctx_offsets, pos, cache, out=out,
                   workspace=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert e.value.status == _lib.DFLASH_ERR_WORKSPACE
    assert cache.lengths.tolist() == lens.tolist()
    # a step that would pass the capacity
    cache.lengths[0] = cache.capacity - 16
    with pytest.raises(DFlashError) as e:
        layer.step(hs, th, case.ctx_offsets, pos, cache, out=out)
    assert e.value.status == 3
    assert cache.lengths[0] == cache.capacity - 16 and cache.lengths[1] == lens[1]
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_maximum_capacity_single_sequence():
    """One sequence filling the largest capacity (2^21 rows, the 16-bit key-tile
    index at its top: 32768 tiles) at the largest positions, split over every
    work-group, so the merge folds 256 parts of one pair."""
    cap = 1 << 21
    cfg = small(batch=1, hidden=64, n_q_heads=1, n_kv_heads=1, head_dim=64, block_size=16,
                cached_len=cap - 16 - 3, new_ctx=3, max_position=cap, config_id=23)
    case = make_case(cfg, seed=0)
    assert int(case.total_len[0]) == cap and case.capacity() == cap
    print(f"[max capacity] T = {cap} keys", flush=True)
    run_and_check(case)
