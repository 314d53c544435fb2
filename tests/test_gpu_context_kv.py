"""GPU parity of the multi-layer context K/V precompute (hidden_norm, one
projection for every draft layer, per-layer k_norm + RoPE, per-layer cache
append) against the float64 oracle, with every cache row outside the appended
ones bit-identical (dead rows hold a NaN canary), lengths exact, and the
layer step that follows it (no new context rows) matching the oracle doing
the same two steps."""
import numpy as np
import pytest
import torch

import oracle
from harness import sampled_rows  # noqa: E402
from harness import (assert_close, assert_close_stored, cache_bits, dev, fill_canary, poison_workspaces, raw_bits,
                     to64)
from workload import CTXKV_CONFIGS, make_ctxkv_case

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def small(**kw):
    base = dict(name="PS", batch=5, hidden=512, n_layers=3, n_kv_heads=2, head_dim=128, dtype="bf16",
                cached_len=(0, 300), new_ctx=(0, 40), config_id=45)
    base.update(kw)
    return CTXKV_CONFIGS["P3"].replace(**base)


def torch_dt(case):
    return torch.bfloat16 if case.cfg.dtype == "bf16" else torch.float32


def make_precompute(case):
    from block_diffusion_draft_qkv_amd import ContextKV, ContextKVShape
    c, w, dt = case.cfg, case.weights, torch_dt(case)
    shape = ContextKVShape(c.hidden, c.n_layers, c.n_kv_heads, c.head_dim, dt, c.rope_theta, c.rms_eps,
                           c.max_position)
    return poison_workspaces(ContextKV(shape, dev(w.hidden_norm, dt), dev(w.w_kv.reshape(-1, c.hidden), dt),
                                       dev(w.k_norm, dt)))


def make_caches(case, capacity=None):
    from block_diffusion_draft_qkv_amd import KVCache
    c, dt = case.cfg, torch_dt(case)
    cap = capacity or case.capacity()
    caches = []
    for layer in range(c.n_layers):
        kv = KVCache(case.batch, c.n_kv_heads, c.head_dim, cap, dt)
        fill_canary(kv.k)
        fill_canary(kv.v)
        for b in range(case.batch):
            kv.write_prefix(b, dev(case.cache_k[layer][b], dt), dev(case.cache_v[layer][b], dt))
        caches.append(kv)
    return caches


def oracle_caches(case):
    return [oracle.OracleCache.from_arrays(case.cache_k[layer], case.cache_v[layer])
            for layer in range(case.cfg.n_layers)]


def run_and_check(case, capacity=None, mode=None):
    pre = make_precompute(case)
    if mode is not None:
        pre.set_append_mode(mode)
    caches = make_caches(case, capacity)
    before = [cache_bits(c) for c in caches]
    dt = torch_dt(case)
    ctx = dev(case.context_states, dt)
    pos = torch.from_numpy(case.positions.astype(np.int32)).cuda()
    pre.append(ctx, case.ctx_offsets, pos, caches)
    torch.cuda.synchronize()
    assert pre.poll_error() == 0
    ref = oracle.context_kv_precompute(case.cfg, case.weights, oracle_caches(case), case.context_states,
                                       case.ctx_offsets, case.positions)
    L, n = case.cached_len, case.new_ctx
    worst = (0.0, 0.0)
    for layer, kv in enumerate(caches):
        assert kv.lengths.tolist() == (L + n).tolist()
        kb, vb = cache_bits(kv)
        bk, bv = before[layer]
        for b in range(case.batch):
            lb, tb = int(L[b]), int(L[b] + n[b])
            np.testing.assert_array_equal(kb[b, :, :lb], bk[b, :, :lb])
            np.testing.assert_array_equal(kb[b, :, tb:], bk[b, :, tb:])
            np.testing.assert_array_equal(vb[b, :, :, :lb], bv[b, :, :, :lb])
            np.testing.assert_array_equal(vb[b, :, :, tb:], bv[b, :, :, tb:])
            if tb > lb:
                e1 = assert_close_stored(to64(kv.k_rows()[b, :, lb:tb]), ref[layer].k[b][:, lb:tb], case.cfg.dtype,
                                         f"layer {layer} K seq {b}")
                e2 = assert_close_stored(to64(kv.vt_rows()[b, :, :, lb:tb].transpose(1, 2)), ref[layer].v[b][:, lb:tb],
                                         case.cfg.dtype, f"layer {layer} V seq {b}")
                worst = (max(worst[0], e1[0], e2[0]), max(worst[1], e1[1], e2[1]))
    return pre, caches, ref, worst


@pytest.mark.parametrize("mode", ["fused", "separate"])
@pytest.mark.parametrize("name", ["P1", "small_bf16", "small_bf16_d64", "one_layer", "P3"])
def test_context_kv_precompute_matches_oracle(name, mode):
    # In "fused" the projection's epilogue normalises, rotates and appends one
    # head per tile; in "separate" HK2 does it over the layers from fp32 rows.
    case = {"P1": lambda: make_ctxkv_case("P1", seed=0),
            "small_bf16": lambda: make_ctxkv_case(small(), seed=1),
            "small_bf16_d64": lambda: make_ctxkv_case(small(head_dim=64, hidden=256, n_layers=5,
                                                            config_id=46), seed=2),
            "one_layer": lambda: make_ctxkv_case(small(n_layers=1, batch=2, config_id=47), seed=3),
            "P3": lambda: make_ctxkv_case("P3", seed=0)}[name]()
    print(f"[{name} {mode}] layers {case.cfg.n_layers}, rows {int(case.ctx_offsets[-1])}", flush=True)
    _, _, _, worst = run_and_check(case, mode=mode)
    print(f"[{name} {mode}] max abs {worst[0]:.3e} rel-RMS {worst[1]:.3e}", flush=True)


def test_context_kv_prefill_rows_sampled():
    """The 4096-row prefill at full size; the oracle checks a sample of rows of
    every layer (each row is independent of the others)."""
    case = make_ctxkv_case("P4", seed=0)
    pre = make_precompute(case)
    caches = make_caches(case)
    dt = torch_dt(case)
    pre.append(dev(case.context_states, dt), case.ctx_offsets, torch.from_numpy(case.positions).cuda(), caches)
    torch.cuda.synchronize()
    assert pre.poll_error() == 0
    rows = sampled_rows(int(case.ctx_offsets[-1]), seed=0)
    sub = case.context_states[rows]
    offs = np.arange(len(rows) + 1, dtype=np.int32)
    empty = [oracle.OracleCache.from_arrays([np.zeros((case.cfg.n_kv_heads, 0, case.cfg.head_dim))] * len(rows),
                                            [np.zeros((case.cfg.n_kv_heads, 0, case.cfg.head_dim))] * len(rows))
             for _ in range(case.cfg.n_layers)]
    ref = oracle.context_kv_precompute(case.cfg, case.weights, empty, sub, offs, case.positions[rows])
    print(f"[P4] {len(rows)} rows checked: the first and last 64, both sides of every 128-row tile "
          f"boundary, 48 random", flush=True)
    for layer, kv in enumerate(caches):
        assert kv.lengths.tolist() == [4096]
        k_all = to64(kv.k_rows()[0])                  # [nkv, cap, d]
        v_all = to64(kv.vt_rows()[0]).transpose(0, 2, 1)
        for i, r in enumerate(rows):
            assert_close_stored(k_all[:, r:r + 1], ref[layer].k[i], "bf16", f"layer {layer} K row {r}")
            assert_close_stored(v_all[:, r:r + 1], ref[layer].v[i], "bf16", f"layer {layer} V row {r}")


def test_layer_step_after_precompute_matches_oracle():
    """The intended use: precompute every layer's context rows, then run a
    layer step with no new context; the output and cache follow the oracle
    doing the same (its step handed an empty context)."""
    from harness import make_layer
    from workload import make_case
    from workload.configs import LayerConfig
    pc = small(n_layers=2, hidden=512, n_kv_heads=2, head_dim=128, batch=4, config_id=48)
    case = make_ctxkv_case(pc, seed=4)
    pre, caches, ref, _ = run_and_check(case, capacity=case.capacity() + 64)
    lcfg = LayerConfig("S", case.batch, pc.hidden, 8, pc.n_kv_heads, pc.head_dim, 16, "bf16",
                       0, 0, config_id=49)
    step = make_case(lcfg, seed=4)
    # layer 1's own projection: K/V rows of the stacked weight, its k_norm
    w = step.weights
    w.w_k, w.w_v = case.weights.w_kv[1][:pc.n_kv_heads * pc.head_dim], case.weights.w_kv[1][pc.n_kv_heads * pc.head_dim:]
    w.k_norm = case.weights.k_norm[1]
    layer = make_layer(step)
    Lb = caches[1].lengths.copy()
    pos = np.concatenate([np.arange(Lb[b], Lb[b] + 16) for b in range(case.batch)]).astype(np.int32)
    hs = dev(step.hidden_states, torch.bfloat16)
    offs = np.zeros(case.batch + 1, dtype=np.int32)
    out = layer.step(hs, None, offs, torch.from_numpy(pos).cuda(), caches[1])
    torch.cuda.synchronize()
    ref_out, ref_cache = oracle.layer_step(lcfg, w, ref[1], step.hidden_states, None, offs, pos)
    assert_close(to64(out), ref_out, "bf16", "step after precompute")
    assert caches[1].lengths.tolist() == (Lb + 16).tolist()


def test_empty_context_changes_nothing_and_bad_calls_are_rejected():
    from block_diffusion_draft_qkv_amd import DFlashError
    case = make_ctxkv_case(small(batch=3, config_id=50), seed=5)
    pre = make_precompute(case)
    caches = make_caches(case)
    before = [(raw_bits(c.k), raw_bits(c.v), c.lengths.copy()) for c in caches]
    ctx = dev(case.context_states, torch.bfloat16)
    pos = torch.from_numpy(case.positions.astype(np.int32)).cuda()
    # no new rows: nothing happens
    pre.append(ctx[:0], np.zeros(4, dtype=np.int32), pos[:0], caches)
    # lengths that differ between layers: rejected before anything runs
    caches[1].lengths[0] += 1
    with pytest.raises(DFlashError):
        pre.append(ctx, case.ctx_offsets, pos, caches)
    caches[1].lengths[0] -= 1
    # a step past the capacity: rejected
    for c in caches:
        c.lengths[0] = case.capacity() - 1
    with pytest.raises(DFlashError) as e:
        pre.append(ctx, case.ctx_offsets, pos, caches)
    assert e.value.status == 3
    for c, (_, _, ln) in zip(caches, before):
        c.set_lengths(ln)
    # offsets that disagree with the rows given: refused by the binding
    with pytest.raises(ValueError):
        pre.append(ctx[:-1], case.ctx_offsets, pos, caches)
    torch.cuda.synchronize()
    for c, (k, v, ln) in zip(caches, before):
        np.testing.assert_array_equal(raw_bits(c.k), k)
        np.testing.assert_array_equal(raw_bits(c.v), v)
        assert c.lengths.tolist() == ln.tolist()


def test_position_out_of_range_is_latched():
    case = make_ctxkv_case(small(batch=2, config_id=51), seed=6)
    pre = make_precompute(case)
    caches = make_caches(case)
    bad = case.positions.copy()
    bad[0] = case.cfg.max_position + 5
    pre.append(dev(case.context_states, torch.bfloat16), case.ctx_offsets, torch.from_numpy(bad).cuda(), caches)
    assert pre.poll_error() != 0
    assert pre.poll_error() == 0  # cleared once reported


@pytest.mark.parametrize("name", ["P3", "P4"])
def test_fc_combine_matches_oracle(name):
    """The fc projection of three target layers' concatenated features
    (fc_in = 3 H) at the workload's row count, against the oracle; P4's 4096
    rows are checked on a sample of rows (each row is independent)."""
    from workload import make_fc_inputs
    case = make_ctxkv_case(name, seed=0)
    rows = int(case.ctx_offsets[-1])
    aux, w_fc = make_fc_inputs(case.cfg, rows, seed=0)
    pre = make_precompute(case)
    pre.set_fc(dev(w_fc, torch.bfloat16))
    out = pre.combine(dev(aux, torch.bfloat16))
    torch.cuda.synchronize()
    pick = np.arange(rows) if rows <= 512 else np.random.default_rng(2).choice(rows, 64, replace=False)
    ref = oracle.combine_hidden_states(aux[pick], w_fc)
    e = assert_close_stored(to64(out[torch.from_numpy(pick).cuda()]), ref, "bf16", f"{name} fc")
    print(f"[fc {name}] rows {rows} max abs {e[0]:.3e} rel-RMS {e[1]:.3e}", flush=True)


@pytest.mark.parametrize("name", ["P1", "small_bf16"])
def test_fc_then_precompute_matches_oracle(name):
    """combine, then append: the caches follow the oracle's precompute of the
    oracle's combined rows."""
    from workload import make_fc_inputs
    case = {"P1": lambda: make_ctxkv_case("P1", seed=3),
            "small_bf16": lambda: make_ctxkv_case(small(config_id=52), seed=3)}[name]()
    dt = torch_dt(case)
    rows = int(case.ctx_offsets[-1])
    aux, w_fc = make_fc_inputs(case.cfg, rows, seed=1)
    pre = make_precompute(case)
    pre.set_fc(dev(w_fc, dt))
    caches = make_caches(case)
    ctx = pre.combine(dev(aux, dt))
    pre.append(ctx, case.ctx_offsets, torch.from_numpy(case.positions.astype(np.int32)).cuda(), caches)
    torch.cuda.synchronize()
    assert pre.poll_error() == 0
    ref = oracle.context_kv_precompute(case.cfg, case.weights, oracle_caches(case),
                                       oracle.combine_hidden_states(aux, w_fc), case.ctx_offsets, case.positions)
    L, n = case.cached_len, case.new_ctx
    for layer, kv in enumerate(caches):
        assert kv.lengths.tolist() == (L + n).tolist()
        for b in range(case.batch):
            lb, tb = int(L[b]), int(L[b] + n[b])
            if tb > lb:
                assert_close_stored(to64(kv.k_rows()[b, :, lb:tb]), ref[layer].k[b][:, lb:tb], case.cfg.dtype,
                                    f"layer {layer} K seq {b}")
                assert_close_stored(to64(kv.vt_rows()[b, :, :, lb:tb].transpose(1, 2)), ref[layer].v[b][:, lb:tb],
                                    case.cfg.dtype, f"layer {layer} V seq {b}")
