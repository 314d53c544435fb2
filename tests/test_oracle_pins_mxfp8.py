"""Pins of the MXFP8 oracle (E4M3 elements, E8M0 block scales, the
block-scaled context K/V projection) against what the format's definition and
an independent library fix.

The pages print no MXFP8 example. So the pins are:
* torch's float8_e4m3fn conversions, an independent library routine;
* closed forms of the format (largest value, subnormals, ties to even,
  saturation);
* invariants of the shared-exponent rule;
* a brute force that quantises by searching the whole code table;
* a pure-Python brute force of the whole precompute on a tiny case.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def e4m3_table():
    """Values of the 256 codes from the field definitions, in plain Python."""
    out = []
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            out.append(float("nan"))
        elif e == 0:
            out.append(s * m / 8 * 2.0 ** -6)
        else:
            out.append(s * (1 + m / 8) * 2.0 ** (e - 7))
    return out


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.e4m3_value(codes), lib)


def test_e4m3_decode_closed_forms():
    v = oracle.e4m3_value(np.array([0x7E, 0x01, 0x07, 0x08, 0x38, 0x40, 0x80, 0xFE, 0x7F, 0xFF], np.uint8))
    assert v[0] == 448.0 and v[1] == 2.0 ** -9 and v[2] == 7 * 2.0 ** -9 and v[3] == 2.0 ** -6
    assert v[4] == 1.0 and v[5] == 2.0 and v[6] == 0.0 and math.copysign(1, v[6]) < 0 and v[7] == -448.0
    assert np.isnan(v[8]) and np.isnan(v[9])
    np.testing.assert_array_equal(oracle.e4m3_value(np.arange(256, dtype=np.uint8)), e4m3_table())


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000) * 60, rng.standard_normal(20000) * 2.0 ** -7,
                        rng.uniform(-448, 448, 20000)]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(x), lib)


def test_e4m3_encode_ties_go_to_the_even_code_and_codes_roundtrip():
    table = e4m3_table()
    for c in range(0x00, 0x7E):          # every pair of neighbouring positive codes
        lo, hi = table[c], table[c + 1]
        mid = (lo + hi) / 2
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(np.array([mid]))[0] == want, hex(c)
        assert oracle.e4m3_encode(np.array([-mid]))[0] == want | 0x80, hex(c)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(oracle.e4m3_value(finite)), finite)


def test_e4m3_encode_saturates_and_keeps_the_sign_of_zero():
    c = oracle.e4m3_encode(np.array([448.0, 449.0, 464.0, 479.0, 1e9, -500.0, -1e-30, 1e-30, 2.0 ** -10,
                                     2.0 ** -10 * 1.0000001]))
    assert list(c[:6]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert c[6] == 0x80 and c[7] == 0x00
    assert c[8] == 0x00 and c[9] == 0x01           # half the smallest subnormal ties to 0; above it rounds up
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([np.nan]))


def brute_quantize_block(xs):
    """Shared exponent by doubling/halving, elements by nearest-code search."""
    table = e4m3_table()
    amax = max(abs(v) for v in xs)
    if amax == 0:
        k = -127 - 8
    else:
        k = 0
        while 2.0 ** k > amax:
            k -= 1
        while 2.0 ** (k + 1) <= amax:
            k += 1
    shared = min(max(k - 8, -127), 127)
    codes = []
    for v in xs:
        t = v / 2.0 ** shared
        best = None
        for c in range(256):
            if math.isnan(table[c]) or (table[c] == 0 and c == 0x80):
                continue
            d = abs(table[c] - t)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
                best = (d, c)
        c = best[1]
        if table[c] == 0 and (t < 0 or (t == 0 and math.copysign(1, t) < 0)):
            c = 0x80
        codes.append(c)
    return codes, shared + 127


def test_mx_quantize_matches_brute_force_code_search():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 96)) * np.exp(rng.uniform(-6, 6, (3, 96)))
    x[1, :32] *= 1e-3
    x[2, 32:64] = 0.0
    x[2, 64] = -1e-40                     # tiny against its block: rounds to -0
    codes, scales = oracle.mx_quantize(x)
    for r in range(3):
        for blk in range(3):
            bc, bs = brute_quantize_block([float(v) for v in x[r, 32 * blk:32 * blk + 32]])
            assert scales[r, blk] == bs
            assert list(codes[r, 32 * blk:32 * blk + 32]) == bc


def test_mx_quantize_scale_rule_closed_forms():
    base = np.linspace(-1, 1, 32) * 0.5
    for k in (-20, -3, 0, 5, 30):
        for top, code in ((1.75, 0x7E), (1.0, 0x78), (1.9, 0x7E), (1.999, 0x7E)):
            x = base * 2.0 ** k
            x[7] = top * 2.0 ** k
            c, s = oracle.mx_quantize(x)
            assert s[0] == k - 8 + 127
            assert c[7] == code               # 1.9 and 1.999 saturate at 448
    c, s = oracle.mx_quantize(np.zeros(64))
    assert list(s) == [0, 0] and not c.any()
    # the shared exponent is clamped to the E8M0 range [-127, 127]
    tiny = np.zeros(32)
    tiny[3] = 2.0 ** -125                   # floor(log2) - 8 = -133 -> -127: element 2^2
    c, s = oracle.mx_quantize(tiny)
    assert s[0] == 0 and c[3] == 0x48
    huge = np.zeros(32)
    huge[0] = -(2.0 ** 140)                 # 140 - 8 = 132 -> 127: element 2^13 saturates
    c, s = oracle.mx_quantize(huge)
    assert s[0] == 254 and c[0] == 0xFE


def test_mx_quantize_power_of_two_invariance():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 128))
    c0, s0 = oracle.mx_quantize(x)
    for j in (-30, -1, 1, 17):
        c, s = oracle.mx_quantize(x * 2.0 ** j)
        np.testing.assert_array_equal(c, c0)
        np.testing.assert_array_equal(s.astype(int), s0.astype(int) + j)


def test_mx_dequantize_error_within_the_format_bound():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((16, 256)) * np.exp(rng.uniform(-3, 3, (16, 1)))
    c, s = oracle.mx_quantize(x)
    dq = oracle.mx_dequantize(c, s)
    scale = np.repeat(oracle.e8m0_value(s), 32, axis=-1)
    t = np.abs(x) / scale
    normal = (t >= 2.0 ** -6) & (t <= 448)
    assert np.all(np.abs(dq - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])     # half a 3-bit ulp
    assert np.all(np.abs(dq - x)[t < 2.0 ** -6] <= 2.0 ** -10 * scale[t < 2.0 ** -6])
    sat = t > 448
    assert np.all(np.abs(dq[sat]) == 448 * scale[sat])


def test_mxfp8_linear_is_the_plain_product_when_quantisation_is_exact():
    rng = np.random.default_rng(9)
    M, N, K = 5, 7, 96
    exps = rng.integers(-4, 4, (M, K // 32))
    table = np.array(e4m3_table())
    ok = np.flatnonzero(~np.isnan(table) & (np.abs(table) <= 448))
    xe = table[rng.choice(ok, (M, K))]
    xe[:, ::32] = 448.0                      # every block's amax is 448 * 2^e: exact quantisation
    x = xe * np.repeat(2.0 ** exps, 32, axis=1)
    wc = rng.choice(ok, (N, K)).astype(np.uint8)
    ws = rng.integers(120, 134, (N, K // 32)).astype(np.uint8)
    w = oracle.mx_dequantize(wc, ws)
    np.testing.assert_array_equal(oracle.mxfp8_linear(x, wc, ws), x @ w.T)
    xc, xs = oracle.mx_quantize(x)
    np.testing.assert_array_equal(oracle.mx_dequantize(xc, xs), x)


def bf16_py(v):
    """Nearest bf16 value of a Python float (8 significant bits, ties to even)."""
    if v == 0:
        return v
    m, e = math.frexp(v)
    return round(m * 256) / 256 * 2.0 ** e


def test_context_kv_precompute_mxfp8_matches_pure_python_brute_force():
    """hidden_norm, rounding to bf16, MX quantisation of the row, the block-
    scaled product with each layer's K/V rows, k_norm, neox rotation, raw V,
    the append: loops, the code table and the math module only."""
    from workload import CtxKVConfig
    cfg = CtxKVConfig(name="mx-tiny", batch=2, hidden=64, n_layers=2, n_kv_heads=2, head_dim=4, dtype="bf16",
                      cached_len=1, new_ctx=2, rope_theta=10000.0, rms_eps=1e-6)
    rng = np.random.default_rng(21)
    H, Ln, nkv, d, half = 64, 2, 2, 4, 2
    table = np.array(e4m3_table())
    ok = np.flatnonzero(~np.isnan(table))

    class W:
        hidden_norm = rng.uniform(0.5, 1.5, H)
        w_kv_codes = rng.choice(ok, (Ln, 2 * nkv * d, H)).astype(np.uint8)
        w_kv_scales = rng.integers(118, 124, (Ln, 2 * nkv * d, H // 32)).astype(np.uint8)
        k_norm = rng.uniform(0.5, 1.5, (Ln, d))

    lens, news = [1, 3], [2, 1]
    offs = np.array([0, 2, 3])
    C = 3.0 * rng.standard_normal((3, H))
    pos = np.array([1, 2, 3])
    caches = [oracle.OracleCache.from_arrays([rng.standard_normal((nkv, L, d)) for L in lens],
                                             [rng.standard_normal((nkv, L, d)) for L in lens])
              for _ in range(Ln)]
    got = oracle.context_kv_precompute_mxfp8(cfg, W, caches, C, offs, pos)
    tab = e4m3_table()
    for b in range(2):
        for r in range(news[b]):
            x = [float(v) for v in C[offs[b] + r]]
            ms = sum(v * v for v in x) / H
            xn = [bf16_py(x[c] / math.sqrt(ms + cfg.rms_eps) * float(W.hidden_norm[c])) for c in range(H)]
            xq = []
            for blk in range(H // 32):
                codes, sbyte = brute_quantize_block(xn[32 * blk:32 * blk + 32])
                xq += [tab[c] * 2.0 ** (sbyte - 127) for c in codes]
            p = int(pos[offs[b] + r])
            for layer in range(Ln):
                def wrow(n):
                    return [tab[int(W.w_kv_codes[layer][n][c])] * 2.0 ** (int(W.w_kv_scales[layer][n][c // 32]) - 127)
                            for c in range(H)]
                for j in range(nkv):
                    k = [sum(a * w for a, w in zip(xq, wrow(j * d + e))) for e in range(d)]
                    v = [sum(a * w for a, w in zip(xq, wrow((nkv + j) * d + e))) for e in range(d)]
                    mk = sum(t * t for t in k) / d
                    k = [k[e] / math.sqrt(mk + cfg.rms_eps) * float(W.k_norm[layer][e]) for e in range(d)]
                    kr = list(k)
                    for t in range(half):
                        a = p * cfg.rope_theta ** (-2.0 * t / d)
                        kr[t] = k[t] * math.cos(a) - k[t + half] * math.sin(a)
                        kr[t + half] = k[t + half] * math.cos(a) + k[t] * math.sin(a)
                    row = lens[b] + r
                    np.testing.assert_allclose(got[layer].k[b][j, row], kr, rtol=1e-12, atol=1e-12)
                    np.testing.assert_allclose(got[layer].v[b][j, row], v, rtol=1e-12, atol=1e-12)
    for layer in range(Ln):
        for b in range(2):
            np.testing.assert_array_equal(got[layer].k[b][:, :lens[b]], caches[layer].k[b])
            assert got[layer].lengths[b] == lens[b] + news[b]


def test_layer_step_mxfp8_matches_pure_python_brute_force():
    """The MXFP8 layer step against the pure-Python brute force of the layer
    step fed what an MXFP8 linear multiplies: block and context rows
    quantised by the code-table search, weights decoded from the field
    definitions, and each attention output row rounded to bf16 and quantised
    the same way before o_proj."""
    from test_oracle_pins import brute_step, rand_inputs, tiny_cfg
    cfg = tiny_cfg(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=8, block_size=3)
    rng = np.random.default_rng(17)
    H, nq, nkv, d = 64, 4, 2, 8
    table = e4m3_table()
    ok = np.flatnonzero(~np.isnan(np.array(table)))

    class MW:
        w_qkv_codes = rng.choice(ok, ((nq + 2 * nkv) * d, H)).astype(np.uint8)
        w_qkv_scales = rng.integers(118, 124, ((nq + 2 * nkv) * d, H // 32)).astype(np.uint8)
        w_o_codes = rng.choice(ok, (H, nq * d)).astype(np.uint8)
        w_o_scales = rng.integers(118, 124, (H, nq * d // 32)).astype(np.uint8)
        q_norm = rng.uniform(0.5, 1.5, d)
        k_norm = rng.uniform(0.5, 1.5, d)

    lens, news = [2, 0], [3, 1]
    X, C, offs, pos, cache = rand_inputs(cfg, rng, lens, news)
    got, got_cache = oracle.layer_step_mxfp8(cfg, MW, cache, X, C, offs, pos)

    def dec(codes, scales):
        return [[table[int(codes[r][c])] * 2.0 ** (int(scales[r][c // 32]) - 127) for c in range(codes.shape[1])]
                for r in range(codes.shape[0])]

    def qrow(v):
        out = []
        for blk in range(len(v) // 32):
            codes, sbyte = brute_quantize_block([float(t) for t in v[32 * blk:32 * blk + 32]])
            out += [table[c] * 2.0 ** (sbyte - 127) for c in codes]
        return out

    wq = dec(MW.w_qkv_codes, MW.w_qkv_scales)

    class W:
        w_q, w_k, w_v = wq[:nq * d], wq[nq * d:(nq + nkv) * d], wq[(nq + nkv) * d:]
        w_o = dec(MW.w_o_codes, MW.w_o_scales)
        q_norm, k_norm = MW.q_norm, MW.k_norm

    Xq = np.array([qrow(r) for r in X])
    Cq = np.array([qrow(r) for r in C])
    want, want_k, want_v = brute_step(cfg, W, cache, Xq, Cq, offs, pos, o_in=lambda v: qrow([bf16_py(t) for t in v]))
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11)
    for b in range(len(lens)):
        np.testing.assert_allclose(got_cache.k[b], np.array(want_k[b]), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got_cache.v[b], np.array(want_v[b]), rtol=1e-12, atol=1e-12)
