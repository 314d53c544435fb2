"""Float64 CPU oracle of the MXFP8 context K/V projection.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
library and its binding never do, and nothing here is shared with them.

The vLLM page "qwen3_dflash" (``_build_context_kv_buffers``,
``_build_mxfp8_context_kv_proj``, ``_project_context_kv_token_major``) runs the
multi-layer context K/V projection as one MXFP8 GEMM when every draft layer's
``qkv_proj`` is an MXFP8 linear. The K/V rows of each layer's weight are
stacked with their block scales as they are, because the scales belong to
output rows. Everything before and after that GEMM is the precompute of
``context_kv``.

The pages name the format but do not define it. MXFP8 is the OCP Microscaling
(MX v1.0) format with FP8 E4M3 elements:

* E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits. Exponent
  field 0 holds the subnormals m/8 * 2^-6. There are no infinities; S.1111.111
  is NaN, so the largest finite value is 1.75 * 2^8 = 448.
* A block of 32 consecutive elements along the reduction axis shares one E8M0
  scale byte s, worth 2^(s - 127) (255 is NaN).
* The value of an element is its E4M3 value times its block's scale.

Readings taken where the pages are silent:

* The activation is quantised on the fly, per row, in the same format. This
  follows the MX specification's conversion. The shared exponent is
  floor(log2(amax)) - 8, where amax is the block's largest magnitude and 8 is
  E4M3's largest exponent; it is clamped to [-127, 127]. Each element x /
  2^exponent is rounded to the nearest E4M3 value, ties to even, and
  saturated to +-448. The sign of an element that rounds to zero is kept
  (code 0x80). An all-zero block gets exponent -127 (scale byte 0).
* The quantiser's input is hidden_norm's output rounded to bf16, the
  activation dtype. The page's ``ops.rms_norm`` writes into a tensor of the
  states' dtype before the projection.
* The block products are exact, and this oracle sums them exactly enough
  (float64).
* In that configuration the layer's own projections are MXFP8 too (the
  precompute takes the MXFP8 path exactly when every layer's ``qkv_proj`` is
  an MXFP8 linear; ``o_proj`` is taken to be one as well). The draft block's
  rows and the new context rows (bf16 activations) are quantised once for the
  fused q|k|v projection. The attention output, which the model holds in
  bf16, is rounded to bf16 and quantised for ``o_proj``.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

from types import SimpleNamespace

from .context_kv import append_layer_kv
from .ref_fp64 import OracleCache, _f64, layer_step, linear, rms_norm

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest binade (448 = 1.75 * 2^8)
MX_BLOCK = 32


def round_to_binary_float(x, mant_bits: int, emin: int):
    """Round to the nearest value with ``mant_bits`` stored mantissa bits and
    smallest normal exponent ``emin`` (subnormals below it), ties to even; no
    overflow handling. Exact in float64 for the formats used here (bf16, E4M3)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e2 = np.frexp(a)                       # a = f * 2^e2, f in [0.5, 1)
    e = np.maximum(e2 - 1, emin)              # exponent of a's binade (floored at emin)
    quantum = np.ldexp(1.0, e - mant_bits)
    q = np.round(a / quantum) * quantum       # numpy rounds halves to even
    return np.copysign(q, x)


def round_bf16(x):
    """float64 -> nearest bf16 value (8 significant bits, ties to even)."""
    return round_to_binary_float(x, 7, -126)


def e4m3_value(codes):
    """Value of each E4M3 code (uint8); NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(x):
    """Nearest E4M3 code (ties to even), saturating at +-448; the sign of a
    zero result is x's sign. x must not be NaN."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no saturating E4M3 encoding here")
    q = np.minimum(np.abs(round_to_binary_float(x, 3, -6)), E4M3_MAX)
    _, e2 = np.frexp(q)
    normal = q >= 2.0 ** -6
    e = np.where(normal, e2 - 1 + 7, 0)                       # biased exponent field
    m = np.where(normal, q / np.ldexp(1.0, e - 7) * 8 - 8, q / 2.0 ** -9)
    code = (e.astype(np.int64) << 3) | np.rint(m).astype(np.int64)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def e8m0_value(s):
    s = np.asarray(s, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def mx_quantize(x, block: int = MX_BLOCK):
    """MXFP8 codes and E8M0 scale bytes of ``x [..., K]`` (K a multiple of
    ``block``), blocks along the last axis: ``(codes [..., K] uint8, scales
    [..., K / block] uint8)``."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % block:
        raise ValueError("reduction length must be a multiple of the block")
    xb = x.reshape(*x.shape[:-1], K // block, block)
    amax = np.abs(xb).max(axis=-1)
    _, e2 = np.frexp(amax)
    shared = np.where(amax > 0, e2 - 1 - E4M3_EMAX, -127)
    shared = np.clip(shared, -127, 127)
    codes = e4m3_encode(xb / np.ldexp(1.0, shared)[..., None])
    return codes.reshape(x.shape), (shared + 127).astype(np.uint8)


def mx_dequantize(codes, scales, block: int = MX_BLOCK):
    """Values of MXFP8 ``codes [..., K]`` with scale bytes ``[..., K / block]``."""
    v = e4m3_value(codes)
    K = v.shape[-1]
    vb = v.reshape(*v.shape[:-1], K // block, block) * e8m0_value(scales)[..., None]
    return vb.reshape(v.shape)


def mxfp8_linear(x, w_codes, w_scales):
    """nn.Linear y = x W^T with MXFP8 operands: the activation ``x [M, K]`` is
    quantised per row (``mx_quantize``), the weight is given as codes ``[N, K]``
    and scale bytes ``[N, K / 32]`` (blocks along K of each output row)."""
    xc, xs = mx_quantize(x)
    return linear(mx_dequantize(xc, xs), mx_dequantize(w_codes, w_scales))


def context_kv_precompute_mxfp8(cfg, weights, caches: Sequence[OracleCache], context_states, ctx_offsets,
                                positions) -> List[OracleCache]:
    """``context_kv_precompute`` with the MXFP8 projection. ``weights`` has
    ``hidden_norm [H]``, ``w_kv_codes [L, 2*nkv*d, H]`` (uint8 E4M3; layer l:
    its K rows, then its V rows), ``w_kv_scales [L, 2*nkv*d, H/32]`` (uint8
    E8M0) and ``k_norm [L, d]``. The hidden_norm-ed rows are rounded to bf16
    and quantised once; every layer's K/V rows come from the one block-scaled
    product."""
    H, Ln = cfg.hidden, cfg.n_layers
    if len(caches) != Ln:
        raise ValueError("one cache per layer")
    C = _f64(context_states).reshape(-1, H)
    normed = round_bf16(rms_norm(C, weights.hidden_norm, cfg.rms_eps))
    xc, xs = mx_quantize(normed)
    xq = mx_dequantize(xc, xs)
    return [append_layer_kv(cfg, caches[layer],
                            linear(xq, mx_dequantize(weights.w_kv_codes[layer], weights.w_kv_scales[layer])),
                            weights.k_norm[layer], ctx_offsets, positions)
            for layer in range(Ln)]


def _mx_rows(x):
    """Rows as the MXFP8 linear sees them: quantised, then decoded."""
    c, sc = mx_quantize(x)
    return mx_dequantize(c, sc)


def layer_step_mxfp8(cfg, weights, cache: OracleCache, hidden_states, target_hidden, ctx_offsets, positions,
                     quantise_o: bool = True, o_rows_out: list = None):
    """``layer_step`` with MXFP8 projections. ``weights`` has ``w_qkv_codes
    [(nq+2nkv)*d, H]`` and ``w_qkv_scales [.., H/32]`` (rows q | k | v),
    ``w_o_codes [H, nq*d]`` and ``w_o_scales [H, nq*d/32]`` (uint8), and
    ``q_norm, k_norm [d]``. ``quantise_o=False`` feeds o_proj the bf16
    attention output unquantised (a reference point for tests, not the
    method). ``o_rows_out``, if given, receives each sequence's attention
    output rows ``[bs, nq*d]`` (float64, before any rounding), in order."""
    H, nq, nkv, d = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    wqkv = mx_dequantize(weights.w_qkv_codes, weights.w_qkv_scales)
    plain = SimpleNamespace(w_q=wqkv[:nq * d], w_k=wqkv[nq * d:(nq + nkv) * d], w_v=wqkv[(nq + nkv) * d:],
                            w_o=mx_dequantize(weights.w_o_codes, weights.w_o_scales),
                            q_norm=weights.q_norm, k_norm=weights.k_norm)
    X = _mx_rows(_f64(hidden_states).reshape(-1, H))
    C = _mx_rows(_f64(target_hidden).reshape(-1, H)) if target_hidden is not None else None
    def o_input(o):
        if o_rows_out is not None:
            o_rows_out.append(o)
        return _mx_rows(round_bf16(o)) if quantise_o else round_bf16(o)

    return layer_step(cfg, plain, cache, X, C, ctx_offsets, positions, o_input=o_input)
