"""GPU parity of the MXFP8 context K/V precompute and of its quantiser.

* The quantiser is bit-exact against the oracle's OCP MX rule on the same bf16
  inputs. Both sides decide every code from the same values, so any
  difference is an error. The cases are random blocks over a wide range of
  scales, exact ties, saturation, all-zero blocks, tiny and subnormal blocks,
  and negative values that round to zero.
* The precompute (hidden_norm rounded to bf16, MXFP8 quantisation, block-scaled
  projection, k_norm, RoPE, append) is checked in two parts. The kernel
  computes hidden_norm in fp32 and the oracle in float64; where the two land on
  either side of a bf16 rounding boundary (about 2^-15 of the elements: the
  fp32 value is off by ~2^-23 relative, a bf16 step is 2^-8) the bf16 values
  differ by one step, and in 1/16 of those (a bf16 step against an E4M3 step)
  so do the E4M3 codes. So:
  1. the kernel's activation codes (left in the workspace) against the
     oracle's quantisation of its float64 hidden_norm rounded to bf16: scales
     equal but in at most 2^-12 of the blocks, codes at most one E4M3 step
     apart, and at most max(4, 2^-16 N) of the N codes apart (about 8 times the
     expected 2^-19 N; the 4096-row prefill has 16.7 M codes);
  2. the cache rows against the oracle's projection, k_norm, RoPE and append
     of those same codes, to the stored-value bound; and the new rows as a whole
     against the float64 precompute within rel-RMS 1e-2. (A context row that
     repeats a value sitting on a bf16 rounding boundary can collect several
     such flips: the 4096-row prefill has one row with six, which moved its K by
     2.6e-2, past the stored-value bound against the float64 precompute.)
  Cache rows outside the appended ones must be bit-identical and lengths exact.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import sampled_rows  # noqa: E402
from harness import poison_workspaces  # noqa: E402
from harness import assert_close_stored, cache_bits, dev, raw_bits, to64
from test_gpu_context_kv import make_caches, oracle_caches
from workload import make_ctxkv_case, make_mxfp8_kv_weights, round_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def bf16_matrix_with_edges(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-20, 20, (rows, cols // 32))).repeat(32, axis=1)
    x = round_bf16(x).astype(np.float64)
    blk = x[0].reshape(-1, 32)
    blk[0] = 0.0                                            # all-zero block
    blk[1] = 0.0
    blk[1, 5] = 2.0 ** -126                                 # smallest normal alone: exponent clamped to -127
    blk[2] = -(2.0 ** -133) * np.arange(1, 33)              # bf16 subnormals m * 2^-133
    blk[3] = [1.0, 1.0625, 1.1875, -1.0625, 1.3125, 1.4375, 0.5, 0.53125] * 4
    blk[3] *= 2.0 ** -3                                     # exact E4M3 ties at amax 2^-3 (scale 2^-11)
    blk[4] = 0.0
    blk[4, 0] = 1.90625                                     # saturates at 448
    blk[4, 1:] = -(2.0 ** -20)                              # rounds to -0 (code 0x80)
    blk[5] = -0.0
    x[0] = blk.reshape(-1)
    return x


@pytest.mark.parametrize("rows,cols", [(257, 640), (4096, 4096)])
def test_mxfp8_quantize_is_bit_exact(rows, cols):
    from block_diffusion_draft_qkv_amd import mxfp8_quantize
    x = bf16_matrix_with_edges(rows, cols, seed=rows)
    print(f"[quantize {rows}x{cols}]", flush=True)
    codes, scales = mxfp8_quantize(dev(x, torch.bfloat16))
    torch.cuda.synchronize()
    want_c, want_s = oracle.mx_quantize(x)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    np.testing.assert_array_equal(got_s, want_s)
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:4].tolist()}: " \
                          f"{got_c[tuple(bad[0])]:#x} vs {want_c[tuple(bad[0])]:#x}"


class MXW:
    def __init__(self, case, mx):
        self.hidden_norm = case.weights.hidden_norm
        self.k_norm = case.weights.k_norm
        self.w_kv_codes = mx.w_kv_codes
        self.w_kv_scales = mx.w_kv_scales


def make_mx_precompute(case, mx):
    from block_diffusion_draft_qkv_amd import ContextKV, ContextKVShape
    c, w = case.cfg, case.weights
    shape = ContextKVShape(c.hidden, c.n_layers, c.n_kv_heads, c.head_dim, torch.bfloat16, c.rope_theta,
                           c.rms_eps, c.max_position)
    codes = torch.from_numpy(mx.w_kv_codes.reshape(-1, c.hidden)).cuda()
    scales = torch.from_numpy(mx.w_kv_scales.reshape(-1, c.hidden // 32)).cuda()
    return poison_workspaces(ContextKV(shape, dev(w.hidden_norm, torch.bfloat16), codes,
                                       dev(w.k_norm, torch.bfloat16), w_kv_scale=scales))


def run_mx(case, seed):
    mx = make_mxfp8_kv_weights(case.cfg, seed)
    pre = make_mx_precompute(case, mx)
    caches = make_caches(case)
    before = [cache_bits(c) for c in caches]
    pos = torch.from_numpy(case.positions.astype(np.int32)).cuda()
    ws = pre.workspace(int(case.ctx_offsets[-1]))  # NaN-poisoned
    pre.append(dev(case.context_states, torch.bfloat16), case.ctx_offsets, pos, caches, workspace=ws)
    torch.cuda.synchronize()
    assert pre.poll_error() == 0
    mc = int(case.ctx_offsets[-1])
    codes = pre.workspace_region(ws, mc, "normed").cpu().numpy()
    scales = pre.workspace_region(ws, mc, "normed_mx_scales").cpu().numpy().transpose(1, 0, 2).reshape(mc, -1)
    return mx, pre, caches, before, (codes, scales)


def check_activation_codes(case, act):
    """Part 1 of the module docstring: the kernel's MXFP8 context rows against
    the oracle's quantisation of its float64 hidden_norm."""
    codes, scales = act
    c = case.cfg
    want_c, want_s = oracle.mx_quantize(oracle.round_bf16(oracle.rms_norm(case.context_states, case.weights.hidden_norm,
                                                                          c.rms_eps)))
    same = scales == want_s
    mask = np.repeat(same, 32, axis=1)

    def ordinal(cd):
        cd = cd.astype(np.int64)
        return np.where(cd & 0x80, -(cd & 0x7F), cd & 0x7F)

    step = np.abs(ordinal(codes) - ordinal(want_c))[mask]
    n = codes.size
    flips = int(np.count_nonzero(step))
    print(f"[mxfp8 activation codes {c.name}] {n} codes: {flips} one step apart, "
          f"{int(np.count_nonzero(~same))} of {same.size} scales differ", flush=True)
    assert np.count_nonzero(~same) <= same.size * 2.0 ** -12
    assert step.size == 0 or int(step.max()) <= 1
    assert flips <= max(4, n * 2.0 ** -16)


def own_codes_reference(case, mx, act, rows=None):
    """Part 2's reference: every layer's K/V from the kernel's own activation
    codes (all rows, or the listed rows of a single sequence appended to empty
    caches)."""
    from oracle.context_kv import append_layer_kv
    c = case.cfg
    x = oracle.mx_dequantize(*act)
    if rows is None:
        caches, offs, pos = oracle_caches(case), case.ctx_offsets, case.positions
    else:
        x = x[rows]
        empty = [np.zeros((c.n_kv_heads, 0, c.head_dim))] * len(rows)
        caches = [oracle.OracleCache.from_arrays(empty, empty) for _ in range(c.n_layers)]
        offs, pos = np.arange(len(rows) + 1), case.positions[rows]
    return [append_layer_kv(c, caches[layer], x @ oracle.mx_dequantize(mx.w_kv_codes[layer], mx.w_kv_scales[layer]).T,
                            case.weights.k_norm[layer], offs, pos)
            for layer in range(c.n_layers)]


@pytest.mark.parametrize("name", ["M1", "M2", "P3"])
def test_mxfp8_precompute_matches_oracle(name):
    case = make_ctxkv_case(name, seed=0)
    print(f"[mxfp8 {name}] layers {case.cfg.n_layers}, rows {int(case.ctx_offsets[-1])}", flush=True)
    mx, pre, caches, before, act = run_mx(case, seed=0)
    check_activation_codes(case, act)
    ref = own_codes_reference(case, mx, act)
    full = oracle.context_kv_precompute_mxfp8(case.cfg, MXW(case, mx), oracle_caches(case), case.context_states,
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
                e1 = assert_close_stored(to64(kv.k_rows()[b, :, lb:tb]), ref[layer].k[b][:, lb:tb], "bf16",
                                         f"layer {layer} K seq {b}")
                e2 = assert_close_stored(to64(kv.vt_rows()[b, :, :, lb:tb].transpose(1, 2)), ref[layer].v[b][:, lb:tb],
                                         "bf16", f"layer {layer} V seq {b}")
                worst = (max(worst[0], e1[0], e2[0]), max(worst[1], e1[1], e2[1]))
        # the new rows as a whole against the float64 precompute
        got = np.concatenate([to64(kv.k_rows()[b, :, int(L[b]):int(L[b] + n[b])]).ravel() for b in range(case.batch)])
        want = np.concatenate([full[layer].k[b][:, int(L[b]):int(L[b] + n[b])].ravel() for b in range(case.batch)])
        rel = float(np.sqrt(np.mean((got - want) ** 2)) / np.sqrt(np.mean(want ** 2)))
        assert rel <= 1e-2, (layer, rel)
    print(f"[mxfp8 {name}] max abs {worst[0]:.3e} rel-RMS {worst[1]:.3e} (against the kernel's own codes)", flush=True)


def test_mxfp8_prefill_rows_sampled():
    """The 4096-row prefill at full size: every activation code is checked
    (part 1); the cache rows of a sample of rows of every layer against the
    oracle fed the kernel's codes (part 2; rows are independent: quantisation is
    per row)."""
    case = make_ctxkv_case("P4", seed=0)
    mx, pre, caches, _, act = run_mx(case, seed=1)
    check_activation_codes(case, act)
    rows = sampled_rows(int(case.ctx_offsets[-1]), seed=1)
    ref = own_codes_reference(case, mx, act, rows)
    print(f"[P4] {len(rows)} rows checked: the first and last 64, both sides of every 128-row tile "
          f"boundary, 48 random", flush=True)
    for layer, kv in enumerate(caches):
        assert kv.lengths.tolist() == [4096]
        k_all = to64(kv.k_rows()[0])                  # [nkv, cap, d]
        v_all = to64(kv.vt_rows()[0]).transpose(0, 2, 1)
        for i, r in enumerate(rows):
            assert_close_stored(k_all[:, r:r + 1], ref[layer].k[i], "bf16", f"layer {layer} K row {r}")
            assert_close_stored(v_all[:, r:r + 1], ref[layer].v[i], "bf16", f"layer {layer} V row {r}")


def test_mxfp8_rejections_leave_the_caches_alone():
    from block_diffusion_draft_qkv_amd import ContextKV, ContextKVShape, DFlashError, mxfp8_quantize
    case = make_ctxkv_case("M1", seed=0)
    mx = make_mxfp8_kv_weights(case.cfg, 0)
    c = case.cfg
    codes = torch.from_numpy(mx.w_kv_codes.reshape(-1, c.hidden)).cuda()
    scales = torch.from_numpy(mx.w_kv_scales.reshape(-1, c.hidden // 32)).cuda()
    f32 = ContextKVShape(c.hidden, c.n_layers, c.n_kv_heads, c.head_dim, torch.float32, c.rope_theta, c.rms_eps,
                         c.max_position)
    with pytest.raises(DFlashError):
        ContextKV(f32, dev(case.weights.hidden_norm, torch.float32), codes,
                  dev(case.weights.k_norm, torch.float32), w_kv_scale=scales)
    pre = make_mx_precompute(case, mx)
    pre.set_append_mode("separate")
    caches = make_caches(case)
    before = [(raw_bits(k.k), k.lengths.copy()) for k in caches]
    with pytest.raises(DFlashError):
        pre.append(dev(case.context_states, torch.bfloat16), case.ctx_offsets,
                   torch.from_numpy(case.positions.astype(np.int32)).cuda(), caches)
    torch.cuda.synchronize()
    for (bits, lens), kv in zip(before, caches):
        np.testing.assert_array_equal(raw_bits(kv.k), bits)
        assert kv.lengths.tolist() == lens.tolist()
    with pytest.raises(DFlashError):
        mxfp8_quantize(torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("tables", ["shared", "per_layer"])
def test_mxfp8_precompute_into_paged_stack(tables):
    """The MXFP8 precompute writing three layers' paged caches with one shared
    shuffled block table or a table per layer, against the oracle, dead slots
    untouched."""
    from test_gpu_paged import check_paged_after, paged_stack
    from workload import CTXKV_CONFIGS
    pc = CTXKV_CONFIGS["M2"].replace(batch=4, cached_len=(0, 300), new_ctx=(1, 40), config_id=78)
    case = make_ctxkv_case(pc, seed=7)
    c, dt = case.cfg, torch.bfloat16
    mx = make_mxfp8_kv_weights(c, 2)
    pre = make_mx_precompute(case, mx)
    tot = case.cached_len + case.new_ctx
    caches = paged_stack(case, dt, 5, tables)
    befores = [(raw_bits(kv.k), raw_bits(kv.v)) for kv in caches]
    pre.append(dev(case.context_states, dt), case.ctx_offsets, torch.from_numpy(case.positions).cuda(), caches)
    torch.cuda.synchronize()
    assert pre.poll_error() == 0
    ref = oracle.context_kv_precompute_mxfp8(c, MXW(case, mx), oracle_caches(case), case.context_states,
                                             case.ctx_offsets, case.positions)
    for layer, kv in enumerate(caches):
        check_paged_after(kv, *befores[layer], case.cached_len, tot, ref[layer], "bf16", f"layer {layer}")
