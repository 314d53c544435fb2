"""GPU parity of the paged KV cache (64-row blocks through a block table): the
layer step, the context precompute and a multi-round decode driver with
simulated accepted counts, against the float64 oracle; at C3 the paged step is
bit-identical to the contiguous one. Physical blocks are handed out in a
shuffled order and the pools start with a NaN canary: every slot the step does
not write keeps its bits, and no dead or foreign slot can reach a result."""
import numpy as np
import pytest
import torch

import oracle
from harness import poison_workspaces  # noqa: E402
from harness import (CANARY_BF16, CANARY_F32, assert_close, assert_close_stored, dev, fill_canary, make_cache,
                     make_layer, raw_bits, run_oracle, step_inputs, to64, torch_dtype)
from workload import CTXKV_CONFIGS, LayerConfig, make_case, make_ctxkv_case

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def small(**kw):
    base = dict(name="PG", batch=5, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                dtype="bf16", cached_len=(0, 700), new_ctx=(0, 20), accept=(0, 16), config_id=71)
    base.update(kw)
    return LayerConfig(**base)


def make_paged(case, spare_blocks=8, seed=0, prefix=True, extra_blocks=2):
    from block_diffusion_draft_qkv_amd import PagedKVCache
    cfg = case.cfg
    dt = torch_dtype(case)
    need = [-(-int(t) // 64) for t in case.total_len]
    max_blocks = max(need) + extra_blocks
    cache = PagedKVCache(case.batch, cfg.n_kv_heads, cfg.head_dim, sum(need) + spare_blocks, max_blocks, dt)
    fill_canary(cache.k)
    fill_canary(cache.v)
    order = cache.free
    np.random.default_rng(seed).shuffle(order)
    cache.free = order
    if prefix:
        for b in range(case.batch):
            cache.write_prefix(b, dev(case.cache_k[b], dt), dev(case.cache_v[b], dt))
    return cache


def written_slots(cache, lo, hi):
    """Mask [num_blocks, 64] of the slots holding rows [lo_b, hi_b) of every b."""
    m = np.zeros((cache.num_blocks, 64), dtype=bool)
    for b in range(cache.batch):
        for r in range(int(lo[b]), int(hi[b])):
            m[cache.table_host[b, r // 64], r % 64] = True
    return m


def check_paged_after(cache, bk, bv, lo, hi, ref_cache, dtype, what):
    m = written_slots(cache, lo, hi)
    kb, vb = raw_bits(cache.k), raw_bits(cache.v)
    keep_k = np.broadcast_to(~m[:, None, :, None], kb.shape)
    keep_v = np.broadcast_to(~m[:, None, None, :], vb.shape)
    np.testing.assert_array_equal(kb[keep_k], bk[keep_k])
    np.testing.assert_array_equal(vb[keep_v], bv[keep_v])
    for b in range(cache.batch):
        k, v = cache.read(b)
        l0, l1 = int(lo[b]), int(hi[b])
        if l1 > l0:
            assert_close_stored(to64(k[:, l0:l1]), ref_cache.k[b][:, l0:l1], dtype, f"{what} K seq {b}")
            assert_close_stored(to64(v[:, l0:l1]), ref_cache.v[b][:, l0:l1], dtype, f"{what} V seq {b}")


CASES = {
    "bf16_d128": dict(),
    "fp32_d128": dict(dtype="fp32", batch=3, config_id=72),            # 32-key tiles: half a block
    "bf16_d64": dict(head_dim=64, hidden=256, block_size=8, config_id=73),
    "fp32_d64_mha": dict(dtype="fp32", head_dim=64, hidden=256, n_q_heads=4, n_kv_heads=4, block_size=8,
                         config_id=74),
    "bf16_window": dict(sliding_window=300, cached_len=(200, 900), config_id=75),
}


@pytest.mark.parametrize("mode", ["fused", "separate"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_paged_step_matches_oracle(name, mode):
    case = make_case(small(**CASES[name]), seed=3)
    layer = make_layer(case)
    layer.set_append_mode(mode)
    cache = make_paged(case, seed=1)
    for b in range(case.batch):
        cache.reserve(b, int(case.total_len[b]))
    cache.sync()
    bk, bv = raw_bits(cache.k), raw_bits(cache.v)
    hs, th, pos = step_inputs(case)
    out = layer.step(hs, th, case.ctx_offsets, pos, cache)
    torch.cuda.synchronize()
    assert layer.poll_error() == 0
    ref, new = run_oracle(case)
    assert_close(to64(out), ref, case.cfg.dtype, f"{name} out")
    assert cache.lengths.tolist() == case.total_len.tolist()
    check_paged_after(cache, bk, bv, case.cached_len, case.total_len, new, case.cfg.dtype, name)


def test_paged_c3_step_is_bit_identical_to_contiguous():
    """Same tiles, same order of every sum: only the addresses differ."""
    case = make_case("C3", seed=0)
    layer = make_layer(case)
    hs, th, pos = step_inputs(case)
    flat = make_cache(case)
    out_flat = layer.step(hs, th, case.ctx_offsets, pos, flat).clone()
    cache = make_paged(case, seed=2)
    for b in range(case.batch):
        cache.reserve(b, int(case.total_len[b]))
    cache.sync()
    out = layer.step(hs, th, case.ctx_offsets, pos, cache)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_flat.view(torch.int16))
    for b in (0, 7, 31):
        k, v = cache.read(b)
        kf, vf = flat.read(b)
        assert torch.equal(k.contiguous().view(torch.int16), kf.contiguous().view(torch.int16))
        assert torch.equal(v.contiguous().view(torch.int16), vf.contiguous().view(torch.int16))


def test_multi_round_decode_driver_matches_oracle():
    """Four draft rounds: each appends new context rows and the block, then
    crops every sequence to its accepted prefix (simulated accepted counts),
    releasing the blocks the crop drops; later rounds reuse them. Every
    round's output and the final cache follow the oracle doing the same."""
    from block_diffusion_draft_qkv_amd import run_round
    cfg = small(batch=4, cached_len=(40, 300), new_ctx=(0, 40), config_id=76)
    case = make_case(cfg, seed=5)
    layer = make_layer(case)
    cache = make_paged(case, spare_blocks=40, seed=3, extra_blocks=6)
    ref_cache = oracle.OracleCache.from_arrays(case.cache_k, case.cache_v)
    rng = np.random.default_rng(11)
    for rnd in range(4):
        step = make_case(cfg, seed=100 + rnd, weights=case.weights)
        accept = rng.integers(0, cfg.block_size + 1, size=cfg.batch)
        hs, th, _ = step_inputs(step)
        L = np.array(ref_cache.lengths)
        n = np.diff(step.ctx_offsets)
        out = run_round(layer, cache, hs, th, step.ctx_offsets, accept)
        torch.cuda.synchronize()
        pos = np.concatenate([np.arange(L[b], L[b] + n[b] + cfg.block_size) for b in range(cfg.batch)])
        ref, ref_cache = oracle.layer_step(cfg, case.weights, ref_cache, step.hidden_states, step.target_hidden,
                                           step.ctx_offsets, pos)
        for b in range(cfg.batch):
            ref_cache = oracle.crop(ref_cache, b, int(L[b] + n[b] + accept[b]))
        assert_close(to64(out), ref, "bf16", f"round {rnd} out")
        assert cache.lengths.tolist() == ref_cache.lengths
        assert [cache.blocks_of(b) for b in range(cfg.batch)] == [-(-x // 64) for x in ref_cache.lengths]
        print(f"[round {rnd}] lengths {cache.lengths.tolist()}, free blocks {len(cache.free)}", flush=True)
    for b in range(cfg.batch):
        k, v = cache.read(b)
        assert_close_stored(to64(k), ref_cache.k[b], "bf16", f"final K seq {b}")
        assert_close_stored(to64(v), ref_cache.v[b], "bf16", f"final V seq {b}")
    assert layer.poll_error() == 0


def paged_stack(case, dt, seed, tables):
    """One paged cache per layer holding the case's prefixes, blocks for every
    sequence's new rows reserved. ``tables="shared"``: every layer takes the
    same shuffled blocks and the caches share layer 0's device table;
    ``"per_layer"``: each layer has its own pool size and its own shuffle, so
    no two layers' tables agree."""
    from block_diffusion_draft_qkv_amd import PagedKVCache
    c = case.cfg
    tot = case.cached_len + case.new_ctx
    need = [-(-int(t) // 64) for t in tot]
    rng = np.random.default_rng(seed)
    caches = []
    for layer in range(c.n_layers):
        spare = 4 if tables == "shared" else 4 + 3 * layer
        kv = PagedKVCache(case.batch, c.n_kv_heads, c.head_dim, sum(need) + spare, max(need) + 1, dt)
        fill_canary(kv.k)
        fill_canary(kv.v)
        if tables == "shared" and caches:
            kv.free = list(caches[0].free_at_start)
        else:
            order = kv.free
            rng.shuffle(order)
            kv.free = order
        kv.free_at_start = list(kv.free)
        for b in range(case.batch):
            kv.write_prefix(b, dev(case.cache_k[layer][b], dt), dev(case.cache_v[layer][b], dt))
            kv.reserve(b, int(tot[b]))
        kv.sync()
        caches.append(kv)
    if tables == "shared":
        for kv in caches[1:]:
            assert np.array_equal(kv.table_host, caches[0].table_host)
            kv.table = caches[0].table
            kv.desc.block_table = caches[0].table.data_ptr()
    else:
        for a in range(c.n_layers):
            for b in range(a + 1, c.n_layers):
                assert not np.array_equal(caches[a].table_host, caches[b].table_host)
    return caches


@pytest.mark.parametrize("mode", ["fused", "separate"])
@pytest.mark.parametrize("tables", ["shared", "per_layer"])
def test_context_precompute_into_paged_stack(tables, mode):
    """The multi-layer precompute writing three layers' paged caches, which
    share one block table or each have their own (a slot mapping for all
    layers or one per layer), in both append modes."""
    from block_diffusion_draft_qkv_amd import ContextKV, ContextKVShape
    pc = CTXKV_CONFIGS["P3"].replace(batch=4, hidden=512, n_kv_heads=2, cached_len=(0, 300), new_ctx=(1, 40),
                                     config_id=77)
    case = make_ctxkv_case(pc, seed=6)
    c, w, dt = case.cfg, case.weights, torch.bfloat16
    pre = poison_workspaces(ContextKV(ContextKVShape(c.hidden, c.n_layers, c.n_kv_heads, c.head_dim, dt,
                                                     c.rope_theta, c.rms_eps, c.max_position),
                                      dev(w.hidden_norm, dt), dev(w.w_kv.reshape(-1, c.hidden), dt),
                                      dev(w.k_norm, dt)))
    pre.set_append_mode(mode)
    tot = case.cached_len + case.new_ctx
    caches = paged_stack(case, dt, 4, tables)
    befores = [(raw_bits(kv.k), raw_bits(kv.v)) for kv in caches]
    pre.append(dev(case.context_states, dt), case.ctx_offsets, torch.from_numpy(case.positions).cuda(), caches)
    torch.cuda.synchronize()
    assert pre.poll_error() == 0
    ref = oracle.context_kv_precompute(c, w, [oracle.OracleCache.from_arrays(case.cache_k[l], case.cache_v[l])
                                              for l in range(c.n_layers)],
                                       case.context_states, case.ctx_offsets, case.positions)
    for layer, kv in enumerate(caches):
        assert kv.lengths.tolist() == tot.tolist()
        check_paged_after(kv, *befores[layer], case.cached_len, tot, ref[layer], "bf16", f"layer {layer}")


def test_paged_stack_rejections_leave_every_layer_alone():
    """A bad entry in one layer's own table (past its pools, or a block the
    append needs left out) and a mix of paged and contiguous layers are
    refused before anything runs: no layer's pools or lengths change."""
    from block_diffusion_draft_qkv_amd import ContextKV, ContextKVShape, DFlashError, KVCache, _lib
    pc = CTXKV_CONFIGS["P3"].replace(batch=3, hidden=512, n_kv_heads=2, cached_len=(0, 200), new_ctx=(1, 30),
                                     config_id=79)
    case = make_ctxkv_case(pc, seed=8)
    c, w, dt = case.cfg, case.weights, torch.bfloat16
    pre = poison_workspaces(ContextKV(ContextKVShape(c.hidden, c.n_layers, c.n_kv_heads, c.head_dim, dt,
                                                     c.rope_theta, c.rms_eps, c.max_position),
                                      dev(w.hidden_norm, dt), dev(w.w_kv.reshape(-1, c.hidden), dt),
                                      dev(w.k_norm, dt)))
    caches = paged_stack(case, dt, 9, "per_layer")
    befores = [(raw_bits(kv.k), raw_bits(kv.v), kv.lengths.copy()) for kv in caches]
    args = (dev(case.context_states, dt), case.ctx_offsets, torch.from_numpy(case.positions).cuda())
    last = caches[-1]
    good = int(last.table_host[1, 0])
    last.table_host[1, 0] = last.num_blocks              # past the last layer's pools
    with pytest.raises(DFlashError) as e:
        pre.append(*args, caches)
    assert e.value.status == _lib.DFLASH_ERR_RANGE
    last.table_host[1, 0] = good
    b = int(np.argmax(case.new_ctx > 0))
    tail = last.blocks_of(b) - 1
    blk = int(last.table_host[b, tail])
    last.table_host[b, tail] = -1                        # a block the append writes is missing
    with pytest.raises(DFlashError) as e:
        pre.append(*args, caches)
    assert e.value.status == _lib.DFLASH_ERR_RANGE
    last.table_host[b, tail] = blk
    flat = KVCache(case.batch, c.n_kv_heads, c.head_dim, last.capacity, dt)
    flat.lengths[:] = last.lengths
    with pytest.raises(DFlashError) as e:
        pre.append(*args, caches[:-1] + [flat])
    assert e.value.status == _lib.DFLASH_ERR_SHAPE
    torch.cuda.synchronize()
    for kv, (bk, bv, lens) in zip(caches, befores):
        np.testing.assert_array_equal(raw_bits(kv.k), bk)
        np.testing.assert_array_equal(raw_bits(kv.v), bv)
        assert kv.lengths.tolist() == lens.tolist()


def test_bad_block_tables_are_rejected_before_enqueueing():
    from block_diffusion_draft_qkv_amd import DFlashError
    case = make_case(small(batch=2, config_id=78), seed=7)
    layer = make_layer(case)
    cache = make_paged(case, seed=5)
    for b in range(case.batch):
        cache.reserve(b, int(case.total_len[b]))
    cache.sync()
    hs, th, pos = step_inputs(case)
    out = torch.full((case.batch * case.cfg.block_size, case.cfg.hidden), 3.0, dtype=torch.bfloat16,
                     device="cuda")
    lens = cache.lengths.copy()
    good = int(cache.table_host[1, 0])
    cache.table_host[1, 0] = cache.num_blocks        # past the pool (host mirror)
    with pytest.raises(DFlashError):
        layer.step(hs, th, case.ctx_offsets, pos, cache, out=out)
    cache.table_host[1, 0] = good
    cache.table_host[0, cache.blocks_of(0) - 1] = -1  # a block the step needs is missing
    with pytest.raises(DFlashError):
        layer.step(hs, th, case.ctx_offsets, pos, cache, out=out)
    torch.cuda.synchronize()
    assert cache.lengths.tolist() == lens.tolist()
    assert torch.all(out == 3.0)
