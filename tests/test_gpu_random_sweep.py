"""A seeded sweep of small random layer shapes against the float64 oracle:
dtype, head_dim, KV heads, group size, block size, window, batch, ragged
lengths (empty caches and context-free sequences included), contiguous or
paged cache, append path, and with or without a position array. Each case is
small enough for the oracle to finish in well under a second, and spans
several key tiles, so the sweep reaches shape combinations the hand-picked
cases do not."""
import numpy as np
import pytest
import torch

from harness import (assert_close, cache_bits, check_cache_after_step, make_cache, make_layer, run_oracle,
                     step_inputs, to64)
from workload import LayerConfig, make_case

pytestmark = pytest.mark.gpu

N_CASES = 64


def draw(i):
    rng = np.random.default_rng(1000 + i)
    dtype = "bf16" if rng.random() < 0.75 else "fp32"
    d = int(rng.choice([64, 128]))
    nkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8]))
    bs = int(rng.choice([b for b in (1, 2, 4, 8, 16) if b * g <= 64]))
    hidden = 64 * int(rng.integers(1, 9))
    window = int(rng.choice([0, 0, 0, int(rng.integers(1, 400))]))
    B = int(rng.integers(1, 9))
    lo = int(rng.choice([0, 0, 50, 300]))
    cached = (lo, lo + int(rng.integers(0, 500)))
    new_ctx = (0, int(rng.choice([0, 5, 40])))
    cfg = LayerConfig(f"R{i}", B, hidden, nkv * g, nkv, d, bs, dtype, cached, new_ctx, config_id=200 + i,
                      sliding_window=window)
    layout = "paged" if rng.random() < 0.4 else "contiguous"
    mode = str(rng.choice(["auto", "fused", "separate"]))
    positions = bool(rng.random() < 0.7)
    return cfg, layout, mode, positions


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_matches_oracle(i):
    cfg, layout, mode, use_pos = draw(i)
    case = make_case(cfg, seed=i)
    print(f"[sweep {i}] {cfg.dtype} B={cfg.batch} H={cfg.hidden} nq={cfg.n_q_heads} nkv={cfg.n_kv_heads} "
          f"d={cfg.head_dim} bs={cfg.block_size} W={cfg.sliding_window} lens={case.cached_len.tolist()} "
          f"ctx={case.new_ctx.tolist()} {layout} {mode} positions={'array' if use_pos else 'none'}", flush=True)
    layer = make_layer(case)
    layer.set_append_mode(mode)
    if layout == "paged":
        from test_gpu_paged import check_paged_after, make_paged
        cache = make_paged(case, seed=i)
        for b in range(case.batch):
            cache.reserve(b, int(case.total_len[b]))
        cache.sync()
    else:
        cache = make_cache(case)
    bk, bv = cache_bits(cache) if layout == "contiguous" else (None, None)
    if layout == "paged":
        from harness import raw_bits
        pk, pv = raw_bits(cache.k), raw_bits(cache.v)
    hs, th, pos = step_inputs(case)
    out = layer.step(hs, th, case.ctx_offsets, pos if use_pos else None, cache)
    torch.cuda.synchronize()
    ref, new = run_oracle(case)
    assert_close(to64(out), ref, cfg.dtype, f"sweep {i} out")
    if layout == "paged":
        check_paged_after(cache, pk, pv, case.cached_len, case.total_len, new, cfg.dtype, f"sweep {i}")
    else:
        check_cache_after_step(case, cache, bk, bv, new)
    assert layer.poll_error() == 0


def draw_ctxkv(i):
    from workload import CTXKV_CONFIGS
    rng = np.random.default_rng(5000 + i)
    dtype = "bf16" if rng.random() < 0.75 else "fp32"
    d = int(rng.choice([64, 128]))
    lo = int(rng.choice([0, 0, 100]))
    pc = CTXKV_CONFIGS["P1"].replace(name=f"Q{i}", batch=int(rng.integers(1, 7)), hidden=64 * int(rng.integers(1, 9)),
                                     n_layers=int(rng.integers(1, 5)), n_kv_heads=int(rng.choice([1, 2, 4])),
                                     head_dim=d, dtype=dtype, cached_len=(lo, lo + int(rng.integers(0, 300))),
                                     new_ctx=(0, int(rng.choice([1, 20, 90]))), config_id=300 + i)
    layout = str(rng.choice(["contiguous", "shared", "per_layer"]))
    mode = str(rng.choice(["auto", "fused", "separate"]))
    positions = bool(rng.random() < 0.7)
    return pc, layout, mode, positions


@pytest.mark.parametrize("i", range(24))
def test_random_precompute_matches_oracle(i):
    import oracle
    from harness import dev, raw_bits
    from test_gpu_context_kv import make_caches, make_precompute, oracle_caches
    from test_gpu_paged import check_paged_after, paged_stack
    from workload import make_ctxkv_case
    pc, layout, mode, use_pos = draw_ctxkv(i)
    case = make_ctxkv_case(pc, seed=i)
    print(f"[precompute sweep {i}] {pc.dtype} B={pc.batch} H={pc.hidden} L={pc.n_layers} nkv={pc.n_kv_heads} "
          f"d={pc.head_dim} lens={case.cached_len.tolist()} ctx={case.new_ctx.tolist()} {layout} {mode} "
          f"positions={'array' if use_pos else 'none'}", flush=True)
    dt = torch.bfloat16 if pc.dtype == "bf16" else torch.float32
    pre = make_precompute(case)
    pre.set_append_mode(mode)
    caches = make_caches(case) if layout == "contiguous" else paged_stack(case, dt, i, layout)
    before = [cache_bits(c) if layout == "contiguous" else (raw_bits(c.k), raw_bits(c.v)) for c in caches]
    pos = torch.from_numpy(case.positions).cuda() if use_pos else None
    pre.append(dev(case.context_states, dt), case.ctx_offsets, pos, caches)
    torch.cuda.synchronize()
    assert pre.poll_error() == 0
    ref = oracle.context_kv_precompute(pc, case.weights, oracle_caches(case), case.context_states,
                                       case.ctx_offsets, case.positions)
    tot = case.cached_len + case.new_ctx
    for layer, kv in enumerate(caches):
        assert kv.lengths.tolist() == tot.tolist()
        if layout == "contiguous":
            from harness import assert_close_stored
            k, v = kv.k_rows(), kv.vt_rows()
            kb, vb = cache_bits(kv)
            for b in range(case.batch):
                lb, tb = int(case.cached_len[b]), int(tot[b])
                if tb > lb:
                    assert_close_stored(to64(k[b, :, lb:tb]), ref[layer].k[b][:, lb:tb], pc.dtype, f"{i} K {b}")
                    assert_close_stored(to64(v[b, :, :, lb:tb].transpose(1, 2)), ref[layer].v[b][:, lb:tb],
                                        pc.dtype, f"{i} V {b}")
            # nothing outside the appended rows changed
            kept = np.ones(kb.shape, bool)
            keptv = np.ones(vb.shape, bool)
            for b in range(case.batch):
                lb, tb = int(case.cached_len[b]), int(tot[b])
                kept[b, :, lb:tb] = False
                keptv[b, :, :, lb:tb] = False
            np.testing.assert_array_equal(kb[kept], before[layer][0][kept])
            np.testing.assert_array_equal(vb[keptv], before[layer][1][keptv])
        else:
            check_paged_after(kv, *before[layer], case.cached_len, tot, ref[layer], pc.dtype, f"sweep {i} layer {layer}")


@pytest.mark.parametrize("i", range(12))
def test_random_decoder_matches_oracle(i):
    """The decoder layer on random shapes, every piece against the oracle fed
    the kernel's own intermediates within its derived bound."""
    from test_gpu_decoder import check_pieces, make_decoder
    from workload import make_mlp_weights
    cfg, layout, mode, use_pos = draw(100 + i)
    case = make_case(cfg, seed=i)
    inter = 64 * int(np.random.default_rng(7000 + i).integers(1, 13))
    print(f"[decoder sweep {i}] {cfg.dtype} B={cfg.batch} H={cfg.hidden} nq={cfg.n_q_heads} nkv={cfg.n_kv_heads} "
          f"d={cfg.head_dim} bs={cfg.block_size} W={cfg.sliding_window} I={inter}", flush=True)
    mw = make_mlp_weights(case, inter)
    dec = make_decoder(case, mw)
    cache = make_cache(case)
    x, th, pos = step_inputs(case)
    ws = dec.workspace(case.batch, int(case.ctx_offsets[-1]))
    out = dec.step(x, th, case.ctx_offsets, pos if use_pos else None, cache, workspace=ws)
    torch.cuda.synchronize()
    assert dec.poll_error() == 0
    check_pieces(case, mw, dec, ws, x, out)


@pytest.mark.parametrize("i", range(8))
def test_random_mxfp8_layer_matches_oracle(i):
    """The MXFP8 layer step on random bf16 shapes (hidden and nq * d multiples
    of 128), through the same derived checks as the hand-picked cases."""
    from test_gpu_mxfp8_layer import run_mx
    rng = np.random.default_rng(9000 + i)
    d = int(rng.choice([64, 128]))
    nkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([2, 4, 8])) if d == 64 else int(rng.choice([1, 2, 4]))
    bs = int(rng.choice([b for b in (2, 4, 8, 16) if b * g <= 64]))
    cfg = LayerConfig(f"X{i}", int(rng.integers(1, 7)), 128 * int(rng.integers(1, 5)), nkv * g, nkv, d, bs, "bf16",
                      (0, int(rng.integers(1, 600))), (0, int(rng.choice([0, 8, 40]))), config_id=400 + i,
                      sliding_window=int(rng.choice([0, 0, int(rng.integers(1, 300))])))
    assert (cfg.n_q_heads * d) % 128 == 0
    run_mx(make_case(cfg, seed=i), seed=i)
