"""Host-side argument checks, on the CPU.

The C ABI takes bare pointers and no sizes, so the binding checks every tensor
before the call (shape, dtype, contiguity, device) and the library checks every
configuration and length before it enqueues anything. Both run here without a
GPU: a layer object with no handle (its device set to the CPU) gets as far as
the library, which refuses the null handle; a bad argument is refused earlier,
by the binding, with ValueError. The create calls are refused before any HIP
call, leaving the output handle NULL."""
import ctypes as C
import os

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_diffusion_draft_qkv_amd", "libdflash.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdflash.so not built")

CPU = torch.device("cpu")
B, BS, H, NQ, NKV, D = 2, 4, 128, 4, 2, 64


def shape(dtype=torch.bfloat16):
    from block_diffusion_draft_qkv_amd import LayerShape
    return LayerShape(H, NQ, NKV, D, BS, dtype)


class NullStream:
    """Stands for the default stream (handle 0) without touching a device."""
    cuda_stream = 0


def handleless(cls, device=CPU, **fields):
    obj = object.__new__(cls)
    obj._h = None
    obj._ws = None
    obj._weights = []
    obj.device = device
    for k, v in fields.items():
        setattr(obj, k, v)
    return obj


def good_args(dtype=torch.bfloat16, n_ctx=(3, 2)):
    from block_diffusion_draft_qkv_amd import KVCache
    cache = KVCache(B, NKV, D, 128, dtype, device="cpu")
    cache.set_lengths([10, 20])
    offs = np.concatenate([[0], np.cumsum(n_ctx)]).astype(np.int32)
    mc = int(offs[-1])
    return dict(hidden_states=torch.zeros(B * BS, H, dtype=dtype),
                target_hidden=torch.zeros(mc, H, dtype=dtype), ctx_offsets=offs,
                positions=torch.zeros(mc + B * BS, dtype=torch.int32), cache=cache)


def call_step(layer, a):
    return layer.step(a["hidden_states"], a["target_hidden"], a["ctx_offsets"], a["positions"], a["cache"],
                      out=a.get("out"), workspace=a.get("workspace"), stream=NullStream())


def test_good_arguments_reach_the_library():
    from block_diffusion_draft_qkv_amd import DFlashError, DFlashLayer, _lib
    layer = handleless(DFlashLayer, shape=shape())
    a = good_args()
    a["out"] = torch.empty(B * BS, H, dtype=torch.bfloat16)
    a["workspace"] = torch.empty(256, dtype=torch.uint8)
    with pytest.raises(DFlashError) as e:
        call_step(layer, a)
    assert e.value.status == _lib.DFLASH_ERR_ARG  # the null handle, after every binding check passed
    assert a["cache"].lengths.tolist() == [10, 20]
    # no context rows at all: target_hidden may be None
    a = good_args(n_ctx=(0, 0))
    a["target_hidden"] = None
    a["workspace"] = torch.empty(256, dtype=torch.uint8)
    with pytest.raises(DFlashError):
        call_step(layer, a)


@pytest.mark.parametrize("what", [
    "hidden_rows", "hidden_dtype", "hidden_noncontig", "target_rows", "target_missing", "target_dtype",
    "positions_len", "positions_dtype", "out_shape", "out_dtype", "out_alias", "offsets_len",
    "offsets_decreasing", "offsets_nonzero_start", "workspace_dtype", "cache_heads", "cache_dtype",
])
def test_bad_layer_step_arguments_raise_before_the_call(what):
    from block_diffusion_draft_qkv_amd import DFlashLayer
    layer = handleless(DFlashLayer, shape=shape())
    a = good_args()
    mc = int(a["ctx_offsets"][-1])
    if what == "hidden_rows":
        a["hidden_states"] = torch.zeros(B * BS + 1, H, dtype=torch.bfloat16)
    elif what == "hidden_dtype":
        a["hidden_states"] = torch.zeros(B * BS, H, dtype=torch.float32)
    elif what == "hidden_noncontig":
        a["hidden_states"] = torch.zeros(H, B * BS, dtype=torch.bfloat16).t()
    elif what == "target_rows":
        a["target_hidden"] = torch.zeros(mc - 1, H, dtype=torch.bfloat16)
    elif what == "target_missing":
        a["target_hidden"] = None
    elif what == "target_dtype":
        a["target_hidden"] = torch.zeros(mc, H, dtype=torch.float16)
    elif what == "positions_len":
        a["positions"] = torch.zeros(mc + B * BS - 1, dtype=torch.int32)
    elif what == "positions_dtype":
        a["positions"] = torch.zeros(mc + B * BS, dtype=torch.int64)
    elif what == "out_shape":
        a["out"] = torch.empty(B * BS, H + 64, dtype=torch.bfloat16)
    elif what == "out_dtype":
        a["out"] = torch.empty(B * BS, H, dtype=torch.float32)
    elif what == "out_alias":
        a["out"] = a["hidden_states"]
    elif what == "offsets_len":
        a["ctx_offsets"] = a["ctx_offsets"][:-1]
    elif what == "offsets_decreasing":
        a["ctx_offsets"] = np.array([0, 4, 2], dtype=np.int32)
    elif what == "offsets_nonzero_start":
        a["ctx_offsets"] = a["ctx_offsets"] + 1
    elif what == "workspace_dtype":
        a["workspace"] = torch.empty(64, dtype=torch.float32)
    elif what == "cache_heads":
        from block_diffusion_draft_qkv_amd import KVCache
        a["cache"] = KVCache(B, NKV + 1, D, 128, torch.bfloat16, device="cpu")
    elif what == "cache_dtype":
        from block_diffusion_draft_qkv_amd import KVCache
        a["cache"] = KVCache(B, NKV, D, 128, torch.float32, device="cpu")
    lens = a["cache"].lengths.copy()
    with pytest.raises(ValueError):
        call_step(layer, a)
    assert a["cache"].lengths.tolist() == lens.tolist()


def test_host_tensors_for_a_device_layer_are_refused():
    """A kernel would dereference a host pointer: every tensor must be on the
    layer's device (here a CUDA device that this CPU test never touches)."""
    from block_diffusion_draft_qkv_amd import DFlashLayer, KVCache
    layer = handleless(DFlashLayer, device=torch.device("cuda", 0), shape=shape())
    with pytest.raises(ValueError, match="cuda:0"):
        call_step(layer, good_args())
    # also when only one tensor is misplaced: build the check's view of a
    # device cache without allocating on a device
    cache = KVCache(B, NKV, D, 128, torch.bfloat16, device="cpu")
    cache.k = cache.k.to("meta")
    cache.v = cache.v.to("meta")
    meta = handleless(DFlashLayer, device=torch.device("meta"), shape=shape())
    a = good_args()
    a["cache"] = cache
    with pytest.raises(ValueError, match="hidden_states must be on meta"):
        call_step(meta, a)


def test_decoder_step_checks():
    from block_diffusion_draft_qkv_amd import DFlashDecoder, DFlashError, _lib
    dec = handleless(DFlashDecoder, shape=shape(), intermediate=256)
    a = good_args()
    a["workspace"] = torch.empty(256, dtype=torch.uint8)
    with pytest.raises(DFlashError) as e:
        dec.step(a["hidden_states"], a["target_hidden"], a["ctx_offsets"], a["positions"], a["cache"],
                 workspace=a["workspace"], stream=NullStream())
    assert e.value.status == _lib.DFLASH_ERR_ARG
    with pytest.raises(ValueError):
        dec.step(a["hidden_states"][:-1], a["target_hidden"], a["ctx_offsets"], a["positions"], a["cache"])
    with pytest.raises(ValueError):
        dec.step(a["hidden_states"], a["target_hidden"], a["ctx_offsets"], a["positions"], a["cache"],
                 out=a["hidden_states"])


def test_context_kv_append_checks():
    from block_diffusion_draft_qkv_amd import ContextKV, ContextKVShape, DFlashError, KVCache, _lib
    pre = handleless(ContextKV, shape=ContextKVShape(H, 2, NKV, D, torch.bfloat16))
    caches = [KVCache(B, NKV, D, 128, torch.bfloat16, device="cpu") for _ in range(2)]
    offs = np.array([0, 3, 5], dtype=np.int32)
    ctx = torch.zeros(5, H, dtype=torch.bfloat16)
    pos = torch.zeros(5, dtype=torch.int32)
    ws = torch.empty(256, dtype=torch.uint8)
    with pytest.raises(DFlashError) as e:
        pre.append(ctx, offs, pos, caches, workspace=ws, stream=NullStream())
    assert e.value.status == _lib.DFLASH_ERR_ARG
    bad = [
        (ctx[:4], offs, pos, caches),
        (ctx, offs, pos[:4], caches),
        (ctx.float(), offs, pos, caches),
        (ctx, offs, pos, caches[:1]),
        (ctx, offs, pos, [caches[0], KVCache(B + 1, NKV, D, 128, torch.bfloat16, device="cpu")]),
        (ctx, np.array([0, 3], dtype=np.int32), pos, caches),
    ]
    for args in bad:
        with pytest.raises(ValueError):
            pre.append(*args, workspace=ws)


def test_rms_norm_checks():
    from block_diffusion_draft_qkv_amd import rms_norm
    x = torch.zeros(3, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rms_norm(x, torch.zeros(64, dtype=torch.bfloat16), 1e-6)
    with pytest.raises(ValueError):
        rms_norm(x, torch.zeros(128, dtype=torch.float32), 1e-6)
    with pytest.raises(ValueError):
        rms_norm(x, torch.zeros(128, dtype=torch.bfloat16), 1e-6, out=torch.empty(3, 64, dtype=torch.bfloat16))


# ---------------------------------------------------------------- create-time

def _cfg(**kw):
    from block_diffusion_draft_qkv_amd import _lib
    base = dict(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16, sliding_window=0,
                max_position=4096, dtype=_lib.DFLASH_BF16, rope_theta=1e6, rms_eps=1e-6)
    base.update(kw)
    return _lib.Config(**base)


DUMMY = 256  # non-null pointers the rejected calls never dereference


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=6, n_kv_heads=4), "SHAPE"),     # n_q % n_kv != 0 (the vLLM page asserts divisibility)
    (dict(head_dim=96), "UNSUPPORTED"),             # only 64 and 128 are built
    (dict(block_size=32), "UNSUPPORTED"),           # bs * g = 128 query rows > 64 per KV head
    (dict(dtype=7), "ARG"),                         # not a dtype
    (dict(hidden=500), "SHAPE"),                    # hidden % 64
    (dict(n_kv_heads=0), "SHAPE"),
    (dict(max_position=0), "SHAPE"),
    (dict(sliding_window=-1), "SHAPE"),
    (dict(rope_theta=0.0), "ARG"),
    (dict(rms_eps=-1.0), "ARG"),
    (dict(n_q_heads=512, n_kv_heads=512, block_size=1), "UNSUPPORTED"),  # more KV heads than built
])
def test_layer_create_rejects_bad_configs_before_any_allocation(kw, status):
    from block_diffusion_draft_qkv_amd import _lib
    h = _lib.lib()
    cfg = _cfg(**kw)
    w = _lib.Weights(DUMMY, DUMMY, DUMMY, DUMMY)
    out = C.c_void_p(DUMMY)
    assert h.dflash_layer_create(C.byref(cfg), C.byref(w), C.byref(out)) == getattr(_lib, f"DFLASH_ERR_{status}")
    assert out.value is None  # the handle is cleared and nothing was created
    # the decoder and the MXFP8 layer go through the same checks
    dcfg = _lib.DecoderConfig(cfg, 256)
    dw = _lib.DecoderWeights(w, DUMMY, DUMMY, DUMMY, DUMMY)
    out = C.c_void_p(DUMMY)
    assert h.dflash_decoder_create(C.byref(dcfg), C.byref(dw), C.byref(out)) == getattr(_lib, f"DFLASH_ERR_{status}")
    assert out.value is None


def test_other_create_rejections():
    from block_diffusion_draft_qkv_amd import _lib
    h = _lib.lib()
    w = _lib.Weights(DUMMY, DUMMY, DUMMY, DUMMY)
    # missing weight pointers
    out = C.c_void_p(DUMMY)
    assert h.dflash_layer_create(C.byref(_cfg()), C.byref(_lib.Weights(DUMMY, None, DUMMY, DUMMY)),
                                 C.byref(out)) == _lib.DFLASH_ERR_ARG
    assert out.value is None
    # decoder: MLP width not a multiple of 64, misaligned norm gain
    dcfg = _lib.DecoderConfig(_cfg(), 100)
    out = C.c_void_p(DUMMY)
    assert h.dflash_decoder_create(C.byref(dcfg), C.byref(_lib.DecoderWeights(w, DUMMY, DUMMY, DUMMY, DUMMY)),
                                   C.byref(out)) == _lib.DFLASH_ERR_SHAPE
    assert out.value is None
    out = C.c_void_p(DUMMY)
    assert h.dflash_decoder_create(C.byref(_lib.DecoderConfig(_cfg(), 256)),
                                   C.byref(_lib.DecoderWeights(w, DUMMY + 2, DUMMY, DUMMY, DUMMY)),
                                   C.byref(out)) == _lib.DFLASH_ERR_ARG
    assert out.value is None
    # MXFP8 layer: fp32 config, missing or misaligned scales, hidden % 128
    mw = _lib.MXFP8Weights(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY)
    for cfg, weights, st in [
        (_cfg(dtype=_lib.DFLASH_F32), mw, _lib.DFLASH_ERR_UNSUPPORTED),
        (_cfg(), _lib.MXFP8Weights(DUMMY, None, DUMMY, DUMMY, DUMMY, DUMMY), _lib.DFLASH_ERR_ARG),
        (_cfg(), _lib.MXFP8Weights(DUMMY, DUMMY + 1, DUMMY, DUMMY, DUMMY, DUMMY), _lib.DFLASH_ERR_ARG),
        (_cfg(hidden=576), mw, _lib.DFLASH_ERR_SHAPE),
    ]:
        out = C.c_void_p(DUMMY)
        assert h.dflash_layer_create_mxfp8(C.byref(cfg), C.byref(weights), C.byref(out)) == st
        assert out.value is None
    # context K/V precompute: head_dim, layer count, misaligned weights, dtype
    ccfg = dict(hidden=512, n_layers=2, n_kv_heads=2, head_dim=128, max_position=4096, dtype=_lib.DFLASH_BF16,
                rope_theta=1e6, rms_eps=1e-6)
    cw = _lib.CtxKVWeights(DUMMY, DUMMY, DUMMY)
    for kw, weights, st in [
        (dict(head_dim=96), cw, _lib.DFLASH_ERR_UNSUPPORTED),
        (dict(n_layers=17), cw, _lib.DFLASH_ERR_UNSUPPORTED),
        (dict(n_layers=0), cw, _lib.DFLASH_ERR_SHAPE),
        (dict(dtype=3), cw, _lib.DFLASH_ERR_ARG),
        (dict(), _lib.CtxKVWeights(DUMMY + 8, DUMMY, DUMMY), _lib.DFLASH_ERR_ARG),
    ]:
        c = dict(ccfg)
        c.update(kw)
        out = C.c_void_p(DUMMY)
        assert h.dflash_ctxkv_create(C.byref(_lib.CtxKVConfig(**c)), C.byref(weights), C.byref(out)) == st
        assert out.value is None
