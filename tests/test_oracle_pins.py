"""Pins of the float64 oracle against what the pages and mathematics fix.

The pages print no numeric worked example for this layer, so every pin here is
a closed form, an invariant, a special case that reduces to an independent
library routine, or brute force on tiny inputs in pure Python. Each is chosen so
that a plausible slip in the oracle (a dropped gain or eps, a wrong sign, an
interleaved instead of half-split RoPE pairing, a prefix instead of suffix of
positions, ``h % nkv`` instead of ``h // g``, a causal mask, ``<=`` instead of
``<`` in the band, a transposed weight) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from workload import LayerConfig, Weights

RNG = np.random.default_rng(1234)


def tiny_cfg(**kw):
    base = dict(name="tiny", batch=1, hidden=12, n_q_heads=4, n_kv_heads=2, head_dim=6,
                block_size=3, dtype="fp32", cached_len=2, new_ctx=3, rope_theta=10000.0,
                rms_eps=1e-6, sliding_window=0)
    base.update(kw)
    return LayerConfig(**base)


def rand_weights(cfg, rng, gain_lo=0.5, gain_hi=1.5):
    H, nq, nkv, d = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    return Weights(w_q=rng.standard_normal((nq * d, H)) * 0.3,
                   w_k=rng.standard_normal((nkv * d, H)) * 0.3,
                   w_v=rng.standard_normal((nkv * d, H)) * 0.3,
                   w_o=rng.standard_normal((H, nq * d)) * 0.3,
                   q_norm=rng.uniform(gain_lo, gain_hi, d),
                   k_norm=rng.uniform(gain_lo, gain_hi, d))


def rand_inputs(cfg, rng, lens, news):
    B, H, nkv, d, bs = len(lens), cfg.hidden, cfg.n_kv_heads, cfg.head_dim, cfg.block_size
    offs = np.concatenate([[0], np.cumsum(news)]).astype(np.int64)
    X = rng.standard_normal((B * bs, H))
    C = rng.standard_normal((int(offs[-1]), H))
    cache = oracle.OracleCache.from_arrays(
        [rng.standard_normal((nkv, L, d)) for L in lens],
        [rng.standard_normal((nkv, L, d)) for L in lens])
    pos = np.concatenate([np.arange(L, L + n + bs) for L, n in zip(lens, news)])
    return X, C, offs, pos, cache


# ---------------------------------------------------------------- brute force

def brute_step(cfg, w, cache, X, C, offs, pos, o_in=None):
    """The whole layer step in pure-Python loops and the math module only
    (``o_in``, if given, maps each attention output row before o_proj)."""
    H, nq, nkv, d, bs = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_size
    g, half, W = nq // nkv, d // 2, cfg.sliding_window
    B = len(offs) - 1
    out = [[0.0] * H for _ in range(B * bs)]

    def lin(x, wm, rows):
        return [sum(x[c] * float(wm[r][c]) for c in range(len(x))) for r in rows]

    def norm(v, gain):
        ms = sum(t * t for t in v) / len(v)
        return [v[i] / math.sqrt(ms + cfg.rms_eps) * float(gain[i]) for i in range(len(v))]

    def rot(v, p):
        o = list(v)
        for t in range(half):
            a = p * cfg.rope_theta ** (-2.0 * t / d)
            o[t] = v[t] * math.cos(a) - v[t + half] * math.sin(a)
            o[t + half] = v[t + half] * math.cos(a) + v[t] * math.sin(a)
        return o

    new_k, new_v = [], []
    for b in range(B):
        n = int(offs[b + 1] - offs[b])
        base = int(offs[b]) + b * bs
        rows_src = [list(map(float, C[int(offs[b]) + r])) for r in range(n)] + \
                   [list(map(float, X[b * bs + i])) for i in range(bs)]
        Kb = [[list(map(float, cache.k[b][j, t])) for t in range(cache.k[b].shape[1])] for j in range(nkv)]
        Vb = [[list(map(float, cache.v[b][j, t])) for t in range(cache.v[b].shape[1])] for j in range(nkv)]
        for r, x in enumerate(rows_src):
            p = int(pos[base + r])
            for j in range(nkv):
                kk = lin(x, w.w_k, range(j * d, (j + 1) * d))
                vv = lin(x, w.w_v, range(j * d, (j + 1) * d))
                Kb[j].append(rot(norm(kk, w.k_norm), p))
                Vb[j].append(vv)
        T = len(Kb[0])
        for i in range(bs):
            x = list(map(float, X[b * bs + i]))
            p = int(pos[base + n + i])
            concat = []
            for h in range(nq):
                q = rot(norm(lin(x, w.w_q, range(h * d, (h + 1) * d)), w.q_norm), p)
                j = h // g
                qi = T - bs + i
                vis = [t for t in range(T) if not W or abs(qi - t) < W]
                s = [sum(q[c] * Kb[j][t][c] for c in range(d)) / math.sqrt(d) for t in vis]
                mx = max(s)
                e = [math.exp(v - mx) for v in s]
                z = sum(e)
                o = [sum(e[u] / z * Vb[j][t][c] for u, t in enumerate(vis)) for c in range(d)]
                concat += o
            out[b * bs + i] = lin(o_in(concat) if o_in else concat, w.w_o, range(H))
        new_k.append(Kb)
        new_v.append(Vb)
    return np.array(out), new_k, new_v


@pytest.mark.parametrize("window", [0, 3])
def test_layer_step_matches_pure_python_brute_force(window):
    cfg = tiny_cfg(batch=2, sliding_window=window)
    rng = np.random.default_rng(7 + window)
    w = rand_weights(cfg, rng)
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens=[2, 4], news=[3, 0])
    out, new = oracle.layer_step(cfg, w, cache, X, C, offs, pos)
    ref, bk, bv = brute_step(cfg, w, cache, X, C, offs, pos)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11)
    for b in range(2):
        np.testing.assert_allclose(new.k[b], np.array(bk[b]), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(new.v[b], np.array(bv[b]), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- projection

def test_linear_is_x_times_w_transposed():
    x = RNG.standard_normal((3, 5))
    w = RNG.standard_normal((4, 5))
    ref = [[sum(x[i, c] * w[r, c] for c in range(5)) for r in range(4)] for i in range(3)]
    np.testing.assert_allclose(oracle.linear(x, w), ref, rtol=1e-13)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_unit_rms_before_gain_closed_form():
    x = RNG.standard_normal((50, 128)) * RNG.uniform(0.001, 10, (50, 1))
    eps = 1e-6
    y = oracle.rms_norm(x, np.ones(128), eps)
    ms = np.mean(x * x, axis=-1)
    rms_y = np.sqrt(np.mean(y * y, axis=-1))
    np.testing.assert_allclose(rms_y, np.sqrt(ms / (ms + eps)), rtol=1e-13)
    # large inputs: RMS exactly 1 up to eps / (2 ms)
    assert np.all(np.abs(rms_y - 1) <= eps / (2 * ms) * 1.01 + 1e-15)


def test_rmsnorm_gain_eps_and_zero_vector():
    x = np.array([3.0, -4.0, 0.0, 0.0])
    gain = np.array([2.0, 0.5, 7.0, 1.0])
    eps = 0.25
    denom = math.sqrt((9 + 16) / 4 + 0.25)
    np.testing.assert_allclose(oracle.rms_norm(x, gain, eps), [6 / denom, -2 / denom, 0, 0], rtol=1e-15)
    assert np.all(oracle.rms_norm(np.zeros(8), np.ones(8), 1e-6) == 0)


# ---------------------------------------------------------------- RoPE

def test_rope_pairs_halves_with_standard_frequencies():
    d, theta = 8, 1e6
    for t in range(d // 2):
        x = np.zeros((1, d))
        x[0, t] = 1.0
        p = 37
        y = oracle.rope(x, [p], theta)[0]
        a = p * theta ** (-2.0 * t / d)
        expect = np.zeros(d)
        expect[t] = math.cos(a)
        expect[t + d // 2] = math.sin(a)   # x2' = x2 cos + x1 sin
        np.testing.assert_allclose(y, expect, atol=1e-15)
        x = np.zeros((1, d))
        x[0, t + d // 2] = 1.0
        y = oracle.rope(x, [p], theta)[0]
        expect = np.zeros(d)
        expect[t] = -math.sin(a)           # x1' = x1 cos - x2 sin
        expect[t + d // 2] = math.cos(a)
        np.testing.assert_allclose(y, expect, atol=1e-15)


def test_rope_identity_norm_and_composition():
    d = 64
    x = RNG.standard_normal((5, d))
    np.testing.assert_array_equal(oracle.rope(x, [0] * 5, 1e6), x)
    y = oracle.rope(x, [1, 100, 5000, 32800, 131071], 1e6)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    m, n = 1234, 777
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, [m] * 5, 1e6), [n] * 5, 1e6),
                               oracle.rope(x, [m + n] * 5, 1e6), atol=1e-11)


def test_rope_fp32_angle_would_lose_precision_at_long_context():
    """Why the GPU path reads a cos/sin table built in float64: an fp32 angle
    ``pos * inv_freq`` at position 32800 errs by ~7e-4 rad, far beyond the
    fp32 parity tolerance of 1e-4, while the fp64 angle is exact to ~1e-11."""
    inv = oracle.rope_inv_freq(128, 1e6)
    exact = 32800 * inv
    f32 = (np.float32(32800) * inv.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(f32 - exact)) > 5e-4


def test_scores_invariant_under_shift_of_all_positions():
    """RoPE relative invariance through the whole step: shifting every window
    position by the same amount (empty cache) leaves the output unchanged."""
    cfg = tiny_cfg(head_dim=8, hidden=16)
    rng = np.random.default_rng(3)
    w = rand_weights(cfg, rng)
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens=[0], news=[5])
    out0, _ = oracle.layer_step(cfg, w, cache, X, C, offs, pos)
    out1, _ = oracle.layer_step(cfg, w, cache, X, C, offs, pos + 991)
    np.testing.assert_allclose(out0, out1, rtol=1e-10, atol=1e-12)
    out2, _ = oracle.layer_step(cfg, w, cache, X, C, offs, pos * 2)  # not a shift: must differ
    assert np.max(np.abs(out2 - out0)) > 1e-3


# ---------------------------------------------------------------- suffix rule

def test_queries_take_the_trailing_positions_of_the_window():
    """With identical q and k projections and gains, block row i's query equals
    its own key before RoPE; rotated at the same position (the suffix rule) the
    score with its own key is the unrotated <q, q> / sqrt(d) exactly."""
    cfg = tiny_cfg(n_q_heads=2, n_kv_heads=2, head_dim=8, hidden=16, block_size=4)
    rng = np.random.default_rng(11)
    w = rand_weights(cfg, rng)
    w.w_k = w.w_q.copy()
    w.k_norm = w.q_norm.copy()
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens=[0], news=[3])
    pos = pos * 7 + 5  # distinct positions, so a wrong alignment shows
    _, new = oracle.layer_step(cfg, w, cache, X, C, offs, pos)
    q_unrot = oracle.rms_norm(oracle.linear(X, w.w_q).reshape(4, 2, 8), w.q_norm, cfg.rms_eps)
    K = new.k[0]  # [2, 7, 8]; block keys are rows 3..6
    for i in range(4):
        for h in range(2):
            q_rot = oracle.rope(q_unrot[i, h][None], [pos[3 + i]], cfg.rope_theta)[0]
            np.testing.assert_allclose(q_rot @ K[h, 3 + i], q_unrot[i, h] @ q_unrot[i, h], rtol=1e-12)
            # the prefix alignment (position i instead of 3+i) would not match
            q_bad = oracle.rope(q_unrot[i, h][None], [pos[i]], cfg.rope_theta)[0]
            assert abs(q_bad @ K[h, 3 + i] - q_unrot[i, h] @ q_unrot[i, h]) > 1e-6


# ---------------------------------------------------------------- GQA

def test_gqa_equals_mha_with_repeated_kv_heads():
    cfg = tiny_cfg(n_q_heads=6, n_kv_heads=2, head_dim=4, hidden=8)
    rng = np.random.default_rng(5)
    w = rand_weights(cfg, rng)
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens=[3], news=[2])
    out, new = oracle.layer_step(cfg, w, cache, X, C, offs, pos)
    g, d = 3, 4
    rep = lambda m: np.repeat(m.reshape(2, d, -1), g, axis=0).reshape(6 * d, -1)  # noqa: E731
    mha_cfg = cfg.replace(n_kv_heads=6)
    w_mha = Weights(w.w_q, rep(w.w_k), rep(w.w_v), w.w_o, w.q_norm, w.k_norm)
    cache_mha = oracle.OracleCache.from_arrays([np.repeat(cache.k[0], g, axis=0)],
                                               [np.repeat(cache.v[0], g, axis=0)])
    out_mha, _ = oracle.layer_step(mha_cfg, w_mha, cache_mha, X, C, offs, pos)
    np.testing.assert_allclose(out, out_mha, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- attention

def test_attention_reduces_to_torch_sdpa_at_position_zero():
    """Positions all 0 make RoPE the identity; with an empty cache the step is
    plain non-causal SDPA over [context | block], which torch computes in fp64
    on the CPU (with the KV heads repeated for GQA)."""
    torch = pytest.importorskip("torch")
    cfg = tiny_cfg(n_q_heads=4, n_kv_heads=2, head_dim=8, hidden=16, block_size=4)
    rng = np.random.default_rng(9)
    w = rand_weights(cfg, rng)
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens=[0], news=[5])
    pos = np.zeros_like(pos)
    out, _ = oracle.layer_step(cfg, w, cache, X, C, offs, pos)
    T = torch.from_numpy
    q = T(oracle.rms_norm((X @ w.w_q.T).reshape(4, 4, 8), w.q_norm, 1e-6)).transpose(0, 1)
    src = np.concatenate([C, X])
    k = T(oracle.rms_norm((src @ w.w_k.T).reshape(9, 2, 8), w.k_norm, 1e-6)).transpose(0, 1)
    v = T((src @ w.w_v.T).reshape(9, 2, 8)).transpose(0, 1)
    k = k.repeat_interleave(2, dim=0)
    v = v.repeat_interleave(2, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=False)[0]
    ref = o.transpose(0, 1).reshape(4, 32).numpy() @ w.w_o.T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_single_key_returns_its_value():
    cfg = tiny_cfg(block_size=1)
    rng = np.random.default_rng(2)
    w = rand_weights(cfg, rng)
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens=[0], news=[0])
    out, new = oracle.layer_step(cfg, w, cache, X, C, offs, pos)
    v = new.v[0][:, 0, :]  # [nkv, d], the only key
    o = np.concatenate([v[h // 2] for h in range(4)])
    np.testing.assert_allclose(out[0], w.w_o @ o, rtol=1e-12)


def test_zero_input_gives_uniform_weights():
    """X = 0 and C = 0 make q = 0 (RMSNorm of zero is zero), so every visible
    key gets the same weight and the output is o_proj of the mean value row."""
    cfg = tiny_cfg()
    rng = np.random.default_rng(4)
    w = rand_weights(cfg, rng)
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens=[4], news=[2])
    out, new = oracle.layer_step(cfg, w, cache, np.zeros_like(X), np.zeros_like(C), offs, pos)
    mean_v = new.v[0].mean(axis=1)  # [nkv, d]
    o = np.concatenate([mean_v[h // 2] for h in range(4)])
    for i in range(cfg.block_size):
        np.testing.assert_allclose(out[i], w.w_o @ o, rtol=1e-12, atol=1e-14)


def test_block_queries_are_not_causal():
    """Permuting the block rows together with their positions permutes the
    output rows: no query is masked from later block keys."""
    cfg = tiny_cfg(block_size=4)
    rng = np.random.default_rng(6)
    w = rand_weights(cfg, rng)
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens=[3], news=[2])
    perm = np.array([3, 1, 0, 2])
    out, _ = oracle.layer_step(cfg, w, cache, X, C, offs, pos)
    pos_p = pos.copy()
    pos_p[2:] = pos[2:][perm]
    out_p, _ = oracle.layer_step(cfg, w, cache, X[perm], C, offs, pos_p)
    np.testing.assert_allclose(out_p, out[perm], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- sliding window

def test_window_at_least_the_keys_is_full_attention():
    cfg = tiny_cfg()
    rng = np.random.default_rng(8)
    w = rand_weights(cfg, rng)
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens=[5], news=[2])
    full, _ = oracle.layer_step(cfg, w, cache, X, C, offs, pos)
    T = 5 + 2 + cfg.block_size
    banded, _ = oracle.layer_step(cfg.replace(sliding_window=T), w, cache, X, C, offs, pos)
    np.testing.assert_array_equal(full, banded)
    narrower, _ = oracle.layer_step(cfg.replace(sliding_window=T - cfg.block_size), w, cache, X, C, offs, pos)
    assert np.max(np.abs(narrower - full)) > 1e-6


def test_window_one_sees_only_its_own_key():
    """Strict band: W = 1 keeps only |Δ| = 0, the query's own block key."""
    cfg = tiny_cfg(sliding_window=1)
    rng = np.random.default_rng(10)
    w = rand_weights(cfg, rng)
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens=[4], news=[2])
    out, new = oracle.layer_step(cfg, w, cache, X, C, offs, pos)
    T = new.v[0].shape[1]
    for i in range(cfg.block_size):
        v = new.v[0][:, T - cfg.block_size + i, :]
        o = np.concatenate([v[h // 2] for h in range(4)])
        np.testing.assert_allclose(out[i], w.w_o @ o, rtol=1e-12)


def test_window_keep_band_edges():
    keep = oracle.window_keep(2, 10, 3)  # queries at key index 8, 9
    assert keep[0].tolist() == [False] * 6 + [True] * 4   # |8 - t| < 3: t in 6..9
    assert keep[1].tolist() == [False] * 7 + [True] * 3   # |9 - t| < 3: t in 7..9


# ---------------------------------------------------------------- cache and crop

def test_incremental_steps_with_crop_equal_one_shot():
    """Step 1 (ctx1, block1), crop the block off (accepted count 0), step 2
    (ctx2, block2) equals one step on (ctx1 ‖ ctx2, block2) from the same
    starting cache: the cache holds exactly the accepted prefix."""
    cfg = tiny_cfg(batch=1)
    rng = np.random.default_rng(12)
    w = rand_weights(cfg, rng)
    X1, C1, _, _, cache = rand_inputs(cfg, rng, lens=[2], news=[3])
    X2 = rng.standard_normal(X1.shape)
    C2 = rng.standard_normal((4, cfg.hidden))
    bs = cfg.block_size
    _, c1 = oracle.layer_step(cfg, w, cache, X1, C1, [0, 3], np.arange(2, 2 + 3 + bs))
    c1 = oracle.crop(c1, 0, 2 + 3)
    out_inc, c2 = oracle.layer_step(cfg, w, c1, X2, C2, [0, 4], np.arange(5, 5 + 4 + bs))
    out_one, c3 = oracle.layer_step(cfg, w, cache, X2, np.concatenate([C1, C2]), [0, 7],
                                    np.arange(2, 2 + 7 + bs))
    np.testing.assert_allclose(out_inc, out_one, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(c2.k[0], c3.k[0], rtol=1e-13, atol=1e-15)


def test_crop_keeps_exact_prefix_and_rejects_growth():
    rng = np.random.default_rng(13)
    cache = oracle.OracleCache.from_arrays([rng.standard_normal((2, 9, 4))], [rng.standard_normal((2, 9, 4))])
    c = oracle.crop(cache, 0, 5)
    assert c.lengths == [5]
    np.testing.assert_array_equal(c.k[0], cache.k[0][:, :5])
    np.testing.assert_array_equal(c.v[0], cache.v[0][:, :5])
    assert oracle.crop(cache, 0, 9).lengths == [9]
    assert oracle.crop(cache, 0, 0).lengths == [0]
    for bad in (10, -1):
        with pytest.raises(ValueError):
            oracle.crop(cache, 0, bad)
    with pytest.raises(IndexError):
        oracle.crop(cache, 1, 0)


# ------------------------------------------- multi-layer context K/V precompute

def ctxkv_tiny(**kw):
    from workload import CtxKVConfig
    base = dict(name="ctxkv-tiny", batch=2, hidden=10, n_layers=3, n_kv_heads=2, head_dim=4,
                dtype="fp32", cached_len=2, new_ctx=3, rope_theta=10000.0, rms_eps=1e-6)
    base.update(kw)
    return CtxKVConfig(**base)


def ctxkv_inputs(cfg, rng, lens, news):
    from workload import CtxKVWeights
    H, Ln, nkv, d = cfg.hidden, cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    w = CtxKVWeights(hidden_norm=rng.uniform(0.5, 1.5, H),
                     w_kv=rng.standard_normal((Ln, 2 * nkv * d, H)) * 0.3,
                     k_norm=rng.uniform(0.5, 1.5, (Ln, d)))
    offs = np.concatenate([[0], np.cumsum(news)]).astype(np.int64)
    C = 3.0 * rng.standard_normal((int(offs[-1]), H))
    pos = np.concatenate([np.arange(L, L + n) for L, n in zip(lens, news)])
    caches = [oracle.OracleCache.from_arrays([rng.standard_normal((nkv, L, d)) for L in lens],
                                             [rng.standard_normal((nkv, L, d)) for L in lens])
              for _ in range(Ln)]
    return w, C, offs, pos, caches


def test_context_kv_precompute_matches_pure_python_brute_force():
    """hidden_norm over the row, each layer's K/V rows of the stacked weight,
    that layer's k_norm, neox rotation at the context positions, raw V, rows
    appended after each layer's cache: in loops and the math module only."""
    cfg = ctxkv_tiny()
    rng = np.random.default_rng(7)
    lens, news = [2, 0], [3, 2]
    w, C, offs, pos, caches = ctxkv_inputs(cfg, rng, lens, news)
    got = oracle.context_kv_precompute(cfg, w, caches, C, offs, pos)
    H, nkv, d, half = cfg.hidden, cfg.n_kv_heads, cfg.head_dim, cfg.head_dim // 2
    for layer in range(cfg.n_layers):
        for b in range(len(lens)):
            for r in range(news[b]):
                x = [float(v) for v in C[offs[b] + r]]
                ms = sum(v * v for v in x) / H
                xn = [x[c] / math.sqrt(ms + cfg.rms_eps) * float(w.hidden_norm[c]) for c in range(H)]
                p = int(pos[offs[b] + r])
                for j in range(nkv):
                    k = [sum(xn[c] * float(w.w_kv[layer][j * d + e][c]) for c in range(H)) for e in range(d)]
                    v = [sum(xn[c] * float(w.w_kv[layer][(nkv + j) * d + e][c]) for c in range(H))
                         for e in range(d)]
                    mk = sum(t * t for t in k) / d
                    k = [k[e] / math.sqrt(mk + cfg.rms_eps) * float(w.k_norm[layer][e]) for e in range(d)]
                    kr = list(k)
                    for t in range(half):
                        a = p * cfg.rope_theta ** (-2.0 * t / d)
                        kr[t] = k[t] * math.cos(a) - k[t + half] * math.sin(a)
                        kr[t + half] = k[t + half] * math.cos(a) + k[t] * math.sin(a)
                    row = lens[b] + r
                    np.testing.assert_allclose(got[layer].k[b][j, row], kr, rtol=1e-12, atol=1e-12)
                    np.testing.assert_allclose(got[layer].v[b][j, row], v, rtol=1e-12, atol=1e-12)
            # the old rows stay as they were
            np.testing.assert_array_equal(got[layer].k[b][:, :lens[b]], caches[layer].k[b])
            np.testing.assert_array_equal(got[layer].v[b][:, :lens[b]], caches[layer].v[b])
            assert got[layer].lengths[b] == lens[b] + news[b]


def test_context_kv_precompute_equals_each_layer_step_on_normed_context():
    """Precomputing is only a reordering: layer l's context rows equal those
    that its own step appends when handed the hidden_norm-ed context."""
    cfg = ctxkv_tiny(n_layers=2, hidden=12, head_dim=6)
    rng = np.random.default_rng(8)
    lens, news = [1, 4], [2, 3]
    w, C, offs, pos, caches = ctxkv_inputs(cfg, rng, lens, news)
    got = oracle.context_kv_precompute(cfg, w, caches, C, offs, pos)
    normed = oracle.rms_norm(C, w.hidden_norm, cfg.rms_eps)
    lcfg = tiny_cfg(hidden=cfg.hidden, n_q_heads=cfg.n_kv_heads, n_kv_heads=cfg.n_kv_heads,
                    head_dim=cfg.head_dim, block_size=1, rope_theta=cfg.rope_theta)
    nkv, d = cfg.n_kv_heads, cfg.head_dim
    for layer in range(cfg.n_layers):
        lw = Weights(w_q=rng.standard_normal((nkv * d, cfg.hidden)), w_k=w.w_kv[layer][:nkv * d],
                     w_v=w.w_kv[layer][nkv * d:], w_o=rng.standard_normal((cfg.hidden, nkv * d)),
                     q_norm=np.ones(d), k_norm=w.k_norm[layer])
        X = rng.standard_normal((len(lens), cfg.hidden))
        # the step's window is [context | one block token]: positions continue
        wpos = np.concatenate([np.concatenate([pos[offs[b]:offs[b + 1]], [lens[b] + news[b]]])
                               for b in range(len(lens))])
        _, ref = oracle.layer_step(lcfg, lw, caches[layer], X, normed, offs, wpos)
        for b in range(len(lens)):
            n = lens[b] + news[b]
            np.testing.assert_allclose(got[layer].k[b], ref.k[b][:, :n], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(got[layer].v[b], ref.v[b][:, :n], rtol=1e-12, atol=1e-12)


def test_context_kv_precompute_removes_the_scale_of_the_context():
    """hidden_norm makes the result independent of the context rows' scale
    (exactly so with eps = 0): a dropped hidden_norm fails this."""
    cfg = ctxkv_tiny(rms_eps=0.0)
    rng = np.random.default_rng(9)
    w, C, offs, pos, caches = ctxkv_inputs(cfg, rng, [1, 2], [2, 2])
    a = oracle.context_kv_precompute(cfg, w, caches, C, offs, pos)
    b = oracle.context_kv_precompute(cfg, w, caches, 37.5 * C, offs, pos)
    for layer in range(cfg.n_layers):
        for s in range(2):
            np.testing.assert_allclose(a[layer].k[s], b[layer].k[s], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(a[layer].v[s], b[layer].v[s], rtol=1e-12, atol=1e-12)
    # ... while the raw V of one layer scales with the hidden_norm gain
    from workload import CtxKVWeights
    w2 = CtxKVWeights(2.0 * w.hidden_norm, w.w_kv, w.k_norm)
    c = oracle.context_kv_precompute(cfg, w2, caches, C, offs, pos)
    np.testing.assert_allclose(c[0].v[1][:, 2:], 2.0 * a[0].v[1][:, 2:], rtol=1e-12)
    np.testing.assert_allclose(c[0].k[1], a[0].k[1], rtol=1e-12, atol=1e-12)  # k_norm undoes it


def test_context_kv_precompute_layers_use_their_own_weights():
    """Reversing the layers' weights and caches reverses the results (no layer
    reads another layer's K/V rows or k_norm gain)."""
    from workload import CtxKVWeights
    cfg = ctxkv_tiny()
    rng = np.random.default_rng(10)
    w, C, offs, pos, caches = ctxkv_inputs(cfg, rng, [3, 1], [1, 3])
    a = oracle.context_kv_precompute(cfg, w, caches, C, offs, pos)
    wr = CtxKVWeights(w.hidden_norm, w.w_kv[::-1].copy(), w.k_norm[::-1].copy())
    r = oracle.context_kv_precompute(cfg, wr, caches[::-1], C, offs, pos)
    for layer in range(cfg.n_layers):
        for s in range(2):
            np.testing.assert_array_equal(a[layer].k[s], r[cfg.n_layers - 1 - layer].k[s])
            np.testing.assert_array_equal(a[layer].v[s], r[cfg.n_layers - 1 - layer].v[s])


# ----------------------------------------------------------- draft decoder layer

def test_silu_closed_forms_and_limits():
    xs = np.array([-700.0, -30.0, -1.0, -1e-3, 0.0, 1e-3, 1.0, 30.0, 700.0])
    s = oracle.silu(xs)
    assert s[4] == 0.0
    np.testing.assert_allclose(s[6], 1.0 / (1.0 + math.exp(-1.0)), rtol=1e-15)
    # silu(x) - silu(-x) = x(sigmoid(x) + sigmoid(-x)) = x
    np.testing.assert_allclose(s[5:] - s[:4][::-1], xs[5:], rtol=1e-12, atol=1e-300)
    assert s[-1] == 700.0 and abs(s[0]) < 1e-300 and np.all(np.isfinite(s))
    # slope 1/2 at 0
    assert abs((oracle.silu(np.array([1e-7]))[0] - oracle.silu(np.array([-1e-7]))[0]) / 2e-7 - 0.5) < 1e-6


def decoder_inputs(cfg, rng, inter):
    from workload import MLPWeights
    H = cfg.hidden
    mw = MLPWeights(input_norm=rng.uniform(0.5, 1.5, H), post_norm=rng.uniform(0.5, 1.5, H),
                    w_gate_up=rng.standard_normal((2 * inter, H)) * 0.3,
                    w_down=rng.standard_normal((H, inter)) * 0.3)
    return mw


def test_decoder_layer_matches_pure_python_brute_force():
    """input_layernorm, the layer step (its own brute force), residual add,
    post_attention_layernorm, silu(gate) * up, down, residual add: in loops and
    the math module only."""
    cfg = tiny_cfg(batch=2)
    rng = np.random.default_rng(21)
    w = rand_weights(cfg, rng)
    mw = decoder_inputs(cfg, rng, inter=5)
    lens, news = [2, 1], [3, 0]
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens, news)
    got, new = oracle.decoder_layer_step(cfg, w, mw, cache, X, C, offs, pos)
    H, eps = cfg.hidden, cfg.rms_eps

    def norm(v, gain):
        ms = sum(t * t for t in v) / len(v)
        return [v[i] / math.sqrt(ms + eps) * float(gain[i]) for i in range(len(v))]

    rows = [list(map(float, r)) for r in X]
    a = np.array([norm(r, mw.input_norm) for r in rows])
    att, _, _ = brute_step(cfg, w, cache, a, C, offs, pos)
    inter = mw.w_gate_up.shape[0] // 2
    for i, r in enumerate(rows):
        h = [r[c] + float(att[i][c]) for c in range(H)]
        m = norm(h, mw.post_norm)
        act = []
        for j in range(inter):
            g = sum(m[c] * float(mw.w_gate_up[j][c]) for c in range(H))
            u = sum(m[c] * float(mw.w_gate_up[inter + j][c]) for c in range(H))
            act.append(g / (1.0 + math.exp(-g)) * u)
        o = [h[c] + sum(act[j] * float(mw.w_down[c][j]) for j in range(inter)) for c in range(H)]
        np.testing.assert_allclose(got[i], o, rtol=1e-11, atol=1e-11)


def test_decoder_layer_with_silent_branches_passes_the_stream_through():
    """With o_proj and down_proj zero both branches add exactly 0: the output
    is the input stream bit for bit, while the cache still gets its rows."""
    cfg = tiny_cfg(batch=2)
    rng = np.random.default_rng(22)
    w = rand_weights(cfg, rng)
    w.w_o = np.zeros_like(w.w_o)
    mw = decoder_inputs(cfg, rng, inter=4)
    mw.w_down = np.zeros_like(mw.w_down)
    X, C, offs, pos, cache = rand_inputs(cfg, rng, [1, 3], [2, 1])
    got, new = oracle.decoder_layer_step(cfg, w, mw, cache, X, C, offs, pos)
    np.testing.assert_array_equal(got, X)
    assert new.lengths == [1 + 2 + cfg.block_size, 3 + 1 + cfg.block_size]


def test_draft_stack_is_layers_in_order_then_final_norm():
    """Two layers feed each other in order (swapping them changes the result)
    and the final RMSNorm is applied once at the end."""
    cfg = tiny_cfg(batch=1)
    rng = np.random.default_rng(23)
    layers = [(rand_weights(cfg, rng), decoder_inputs(cfg, rng, inter=4)) for _ in range(2)]
    X, C, offs, pos, cache = rand_inputs(cfg, rng, [2], [1])
    fin = rng.uniform(0.5, 1.5, cfg.hidden)
    got, new = oracle.draft_forward(cfg, layers, [cache, cache.copy()], X, C, offs, pos, fin)
    h1, c1 = oracle.decoder_layer_step(cfg, *layers[0], cache, X, C, offs, pos)
    h2, c2 = oracle.decoder_layer_step(cfg, *layers[1], cache.copy(), h1, C, offs, pos)
    ms = (h2 * h2).mean(axis=-1, keepdims=True)
    np.testing.assert_allclose(got, h2 / np.sqrt(ms + cfg.rms_eps) * fin, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(new[1].k[0], c2.k[0])
    swapped, _ = oracle.draft_forward(cfg, layers[::-1], [cache, cache.copy()], X, C, offs, pos, fin)
    assert np.abs(swapped - got).max() > 1e-3


def test_combine_hidden_states_matches_pure_python_and_feeds_the_precompute():
    """The fc projection of concatenated target features: a pure-Python dot
    product per output, and the precompute of the combined rows equals the
    precompute handed those rows."""
    rng = np.random.default_rng(31)
    rows, fc_in, H = 4, 3 * 10, 10
    aux = rng.standard_normal((rows, fc_in))
    w_fc = rng.standard_normal((H, fc_in)) * 0.2
    got = oracle.combine_hidden_states(aux, w_fc)
    for r in range(rows):
        for o in range(H):
            want = sum(float(aux[r][c]) * float(w_fc[o][c]) for c in range(fc_in))
            assert abs(got[r][o] - want) <= 1e-12 * (1 + abs(want))
    # the layers' features are concatenated per row: permuting whole layer
    # chunks of the input together with the weight's columns changes nothing
    perm = np.concatenate([np.arange(20, 30), np.arange(0, 10), np.arange(10, 20)])
    np.testing.assert_allclose(oracle.combine_hidden_states(aux[:, perm], w_fc[:, perm]), got, rtol=1e-12, atol=1e-12)
