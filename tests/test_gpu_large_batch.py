"""Batches above one launch's limit (DFLASH_LAUNCH_BATCH = 256 sequences): the
library runs them as consecutive launches over runs of at most 256 sequences.
The layer step at B = 600 (contiguous and paged, with and without a position
array), the no-allocation step, the decoder step and the multi-layer
precompute at B = 300 against the float64 oracle, with every dead cache slot
left alone; and bad input in the last run refused before the first runs."""
import numpy as np
import pytest
import torch

from harness import (assert_close, cache_bits, check_cache_after_step, make_cache, make_layer, run_oracle,
                     step_inputs, to64)
from test_gpu_parity import small
from workload import CTXKV_CONFIGS, make_case, make_ctxkv_case

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def big(batch, config_id, **kw):
    base = dict(batch=batch, hidden=128, n_q_heads=2, n_kv_heads=1, head_dim=64, block_size=4,
                cached_len=(0, 130), new_ctx=(0, 3), config_id=config_id)
    base.update(kw)
    return small(**base)


@pytest.mark.parametrize("positions", ["array", "none"])
def test_layer_step_of_600_sequences_matches_oracle(positions):
    case = make_case(big(600, 41), seed=0)
    print(f"[B=600] total keys {int(case.total_len.sum())}", flush=True)
    layer = make_layer(case)
    cache = make_cache(case)
    bk, bv = cache_bits(cache)
    hs, th, pos = step_inputs(case)
    out = layer.step(hs, th, case.ctx_offsets, pos if positions == "array" else None, cache)
    torch.cuda.synchronize()
    ref, new = run_oracle(case)
    assert_close(to64(out), ref, "bf16", "B=600 out")
    check_cache_after_step(case, cache, bk, bv, new)
    assert layer.poll_error() == 0


def test_paged_and_noalloc_steps_of_600_sequences_equal_the_contiguous_one():
    from test_gpu_paged import make_paged
    case = make_case(big(600, 42), seed=1)
    layer = make_layer(case)
    hs, th, pos = step_inputs(case)
    cache = make_cache(case)
    ref = layer.step(hs, th, case.ctx_offsets, pos, cache).clone()
    torch.cuda.synchronize()
    paged = make_paged(case, seed=3)
    for b in range(case.batch):
        paged.reserve(b, int(case.total_len[b]))
    paged.sync()
    out = layer.step(hs, th, case.ctx_offsets, pos, paged)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    for b in (0, 255, 256, 511, 512, 599):
        k, v = paged.read(b)
        k0, v0 = cache.read(b)
        assert torch.equal(k, k0) and torch.equal(v, v0), b
    again = make_cache(case)
    out2 = torch.empty_like(ref)
    layer.step_noalloc(hs, th, case.ctx_offsets, pos, again, out2)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref)
    assert again.lengths.tolist() == cache.lengths.tolist()


def test_bad_input_in_the_last_run_changes_nothing():
    from block_diffusion_draft_qkv_amd import DFlashError, _lib
    case = make_case(big(600, 43, cached_len=(0, 60)), seed=2)
    layer = make_layer(case)
    cache = make_cache(case, capacity=128)
    cache.lengths[599] = 128 - 1          # the last sequence cannot take its window
    bk, bv = cache_bits(cache)
    lens = cache.lengths.copy()
    hs, th, pos = step_inputs(case)
    out = torch.full_like(hs, 3.0)
    with pytest.raises(DFlashError) as e:
        layer.step(hs, th, case.ctx_offsets, pos, cache, out=out)
    assert e.value.status == _lib.DFLASH_ERR_CAPACITY
    torch.cuda.synchronize()
    k, v = cache_bits(cache)
    assert np.array_equal(k, bk) and np.array_equal(v, bv)
    assert cache.lengths.tolist() == lens.tolist() and torch.all(out == 3.0)


def test_decoder_step_of_300_sequences_matches_oracle():
    from test_gpu_decoder import check_pieces, make_decoder
    from workload import make_mlp_weights
    case = make_case(big(300, 44), seed=3)
    mw = make_mlp_weights(case, 256)
    dec = make_decoder(case, mw)
    cache = make_cache(case)
    hs, th, pos = step_inputs(case)
    ws = dec.workspace(case.batch, int(case.ctx_offsets[-1]))
    out = dec.step(hs, th, case.ctx_offsets, pos, cache, workspace=ws)
    torch.cuda.synchronize()
    assert dec.poll_error() == 0
    check_pieces(case, mw, dec, ws, hs, out)


def test_precompute_of_300_sequences_matches_oracle():
    from test_gpu_context_kv import run_and_check
    pc = CTXKV_CONFIGS["P3"].replace(batch=300, hidden=256, n_layers=2, n_kv_heads=1, cached_len=(0, 100),
                                     new_ctx=(0, 6), config_id=45)
    run_and_check(make_ctxkv_case(pc, seed=4))
