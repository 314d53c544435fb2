"""ctypes mirror of include/dflash.h and the loader of libdflash.so.

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

# The in-tree build only: nothing in the environment can substitute another library.
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash.so")

DFLASH_OK = 0
DFLASH_ERR_ARG = 1
DFLASH_ERR_SHAPE = 2
DFLASH_ERR_CAPACITY = 3
DFLASH_ERR_RANGE = 4
DFLASH_ERR_UNSUPPORTED = 5
DFLASH_ERR_HIP = 6
DFLASH_ERR_WORKSPACE = 7
DFLASH_F32 = 0
DFLASH_BF16 = 1
DFLASH_MAX_BATCH = 65536
DFLASH_LAUNCH_BATCH = 256
DFLASH_NOALLOC_SCRATCH_BYTES = 64 << 20
APPEND_MODES = {"auto": 0, "fused": 1, "separate": 2}
KERNEL_NAMES = ("gemm_qkv", "norm_rope", "attn", "merge", "gemm_o", "attn_merge")
PROFILE_MODES = {False: 0, True: 1, "off": 0, "kernels": 1, "attn_span": 2}

# Every symbol include/dflash.h declares.
EXPORTS = (
    "dflash_layer_create", "dflash_layer_destroy", "dflash_workspace_bytes",
    "dflash_attn_step", "dflash_attn_step_noalloc", "dflash_cache_crop", "dflash_layer_poll_error",
    "dflash_layer_set_profiling", "dflash_layer_kernel_times", "dflash_status_string",
    "dflash_layer_set_append_mode",
    "dflash_ctxkv_create", "dflash_ctxkv_destroy", "dflash_ctxkv_workspace_bytes",
    "dflash_ctxkv_append", "dflash_ctxkv_poll_error", "dflash_ctxkv_set_append_mode",
    "dflash_ctxkv_create_mxfp8", "dflash_mxfp8_quantize", "dflash_cache_crop_all",
    "dflash_layer_create_mxfp8", "dflash_ctxkv_set_fc", "dflash_ctxkv_combine",
    "dflash_ctxkv_combine_workspace_bytes",
    "dflash_decoder_create", "dflash_decoder_destroy", "dflash_decoder_attention",
    "dflash_decoder_workspace_bytes", "dflash_decoder_step", "dflash_rms_norm",
    "dflash_workspace_offset", "dflash_decoder_workspace_offset", "dflash_ctxkv_workspace_offset",
    "dflash_block_pool_create", "dflash_block_pool_destroy", "dflash_block_pool_free_count",
    "dflash_block_pool_get_free", "dflash_block_pool_set_free", "dflash_cache_reserve", "dflash_cache_reserve_all",
    "dflash_cache_release", "dflash_cache_release_all", "dflash_cache_push_table", "dflash_block_pool_pending",
    "dflash_block_pool_drop_pending",
)
CTX_WS_REGIONS = {"normed": 0, "normed_mx_scales": 1}
WS_REGIONS = {"attn_out": 0, "attn_out_mx": 1, "attn_out_mx_scales": 2}
DEC_WS_REGIONS = {"a": 0, "att": 1, "h": 2, "m": 3, "act": 4}


class Config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("block_size", C.c_int32), ("sliding_window", C.c_int32),
                ("max_position", C.c_int32), ("dtype", C.c_int32), ("rope_theta", C.c_double),
                ("rms_eps", C.c_double)]


class Weights(C.Structure):
    _fields_ = [("w_qkv", C.c_void_p), ("w_o", C.c_void_p), ("q_norm", C.c_void_p),
                ("k_norm", C.c_void_p)]


class MXFP8Weights(C.Structure):
    _fields_ = [("w_qkv", C.c_void_p), ("w_qkv_scale", C.c_void_p), ("w_o", C.c_void_p),
                ("w_o_scale", C.c_void_p), ("q_norm", C.c_void_p), ("k_norm", C.c_void_p)]


class KVCacheDesc(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("len", C.POINTER(C.c_int32)),
                ("batch", C.c_int32), ("capacity", C.c_int32),
                ("block_table", C.c_void_p), ("block_table_host", C.POINTER(C.c_int32)),
                ("max_blocks", C.c_int32), ("num_blocks", C.c_int32)]


class CtxKVConfig(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_layers", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("max_position", C.c_int32), ("dtype", C.c_int32),
                ("rope_theta", C.c_double), ("rms_eps", C.c_double)]


class CtxKVWeights(C.Structure):
    _fields_ = [("hidden_norm", C.c_void_p), ("w_kv", C.c_void_p), ("k_norm", C.c_void_p)]


class CtxKVMXFP8Weights(C.Structure):
    _fields_ = [("hidden_norm", C.c_void_p), ("w_kv", C.c_void_p), ("w_kv_scale", C.c_void_p),
                ("k_norm", C.c_void_p)]


class DecoderConfig(C.Structure):
    _fields_ = [("attn", Config), ("intermediate", C.c_int32)]


class DecoderWeights(C.Structure):
    _fields_ = [("attn", Weights), ("input_norm", C.c_void_p), ("post_norm", C.c_void_p),
                ("w_gate_up", C.c_void_p), ("w_down", C.c_void_p)]


class DFlashError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_diffusion_draft_qkv_amd.build`")
        h = C.CDLL(LIB_PATH)
        h.dflash_layer_create.argtypes = [C.POINTER(Config), C.POINTER(Weights), C.POINTER(C.c_void_p)]
        h.dflash_layer_create.restype = C.c_int
        h.dflash_layer_create_mxfp8.argtypes = [C.POINTER(Config), C.POINTER(MXFP8Weights), C.POINTER(C.c_void_p)]
        h.dflash_layer_create_mxfp8.restype = C.c_int
        h.dflash_layer_destroy.argtypes = [C.c_void_p]
        h.dflash_layer_destroy.restype = None
        h.dflash_workspace_bytes.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_int64]
        h.dflash_workspace_bytes.restype = C.c_size_t
        h.dflash_attn_step.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(C.c_int32),
                                       C.c_void_p, C.POINTER(KVCacheDesc), C.c_void_p, C.c_void_p,
                                       C.c_size_t, C.c_void_p]
        h.dflash_attn_step.restype = C.c_int
        h.dflash_attn_step_noalloc.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(C.c_int32),
                                               C.c_void_p, C.POINTER(KVCacheDesc), C.c_void_p, C.c_void_p]
        h.dflash_attn_step_noalloc.restype = C.c_int
        h.dflash_cache_crop.argtypes = [C.POINTER(KVCacheDesc), C.c_int32, C.c_int32]
        h.dflash_cache_crop.restype = C.c_int
        h.dflash_layer_poll_error.argtypes = [C.c_void_p, C.c_void_p]
        h.dflash_layer_poll_error.restype = C.c_int
        h.dflash_layer_set_append_mode.argtypes = [C.c_void_p, C.c_int32]
        h.dflash_layer_set_append_mode.restype = C.c_int
        h.dflash_layer_set_profiling.argtypes = [C.c_void_p, C.c_int32]
        h.dflash_layer_set_profiling.restype = C.c_int
        h.dflash_layer_kernel_times.argtypes = [C.c_void_p, C.POINTER(C.c_double), C.POINTER(C.c_int64)]
        h.dflash_layer_kernel_times.restype = C.c_int
        h.dflash_ctxkv_create.argtypes = [C.POINTER(CtxKVConfig), C.POINTER(CtxKVWeights),
                                          C.POINTER(C.c_void_p)]
        h.dflash_ctxkv_create.restype = C.c_int
        h.dflash_ctxkv_create_mxfp8.argtypes = [C.POINTER(CtxKVConfig), C.POINTER(CtxKVMXFP8Weights),
                                                C.POINTER(C.c_void_p)]
        h.dflash_ctxkv_create_mxfp8.restype = C.c_int
        h.dflash_mxfp8_quantize.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]
        h.dflash_mxfp8_quantize.restype = C.c_int
        h.dflash_ctxkv_set_fc.argtypes = [C.c_void_p, C.c_void_p, C.c_int32]
        h.dflash_ctxkv_set_fc.restype = C.c_int
        h.dflash_ctxkv_combine.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                           C.c_size_t, C.c_void_p]
        h.dflash_ctxkv_combine.restype = C.c_int
        h.dflash_ctxkv_combine_workspace_bytes.argtypes = [C.c_void_p, C.c_int64]
        h.dflash_ctxkv_combine_workspace_bytes.restype = C.c_size_t
        h.dflash_cache_crop_all.argtypes = [C.POINTER(KVCacheDesc), C.POINTER(C.c_int32)]
        h.dflash_cache_crop_all.restype = C.c_int
        h.dflash_block_pool_create.argtypes = [C.c_int32, C.POINTER(C.c_void_p)]
        h.dflash_block_pool_create.restype = C.c_int
        h.dflash_block_pool_destroy.argtypes = [C.c_void_p]
        h.dflash_block_pool_destroy.restype = None
        h.dflash_block_pool_free_count.argtypes = [C.c_void_p]
        h.dflash_block_pool_free_count.restype = C.c_int32
        h.dflash_block_pool_get_free.argtypes = [C.c_void_p, C.POINTER(C.c_int32), C.c_int32]
        h.dflash_block_pool_get_free.restype = C.c_int
        h.dflash_block_pool_set_free.argtypes = [C.c_void_p, C.POINTER(C.c_int32), C.c_int32]
        h.dflash_block_pool_set_free.restype = C.c_int
        for name in ("dflash_cache_reserve", "dflash_cache_release"):
            getattr(h, name).argtypes = [C.POINTER(KVCacheDesc), C.c_void_p, C.c_int32, C.c_int64]
            getattr(h, name).restype = C.c_int
        for name in ("dflash_cache_reserve_all", "dflash_cache_release_all"):
            getattr(h, name).argtypes = [C.POINTER(KVCacheDesc), C.c_void_p, C.POINTER(C.c_int64)]
            getattr(h, name).restype = C.c_int
        h.dflash_cache_push_table.argtypes = [C.POINTER(KVCacheDesc), C.c_void_p, C.c_void_p]
        h.dflash_cache_push_table.restype = C.c_int
        h.dflash_block_pool_pending.argtypes = [C.c_void_p]
        h.dflash_block_pool_pending.restype = C.c_int32
        h.dflash_block_pool_drop_pending.argtypes = [C.c_void_p]
        h.dflash_block_pool_drop_pending.restype = C.c_int
        h.dflash_ctxkv_destroy.argtypes = [C.c_void_p]
        h.dflash_ctxkv_destroy.restype = None
        h.dflash_ctxkv_workspace_bytes.argtypes = [C.c_void_p, C.c_int64]
        h.dflash_ctxkv_workspace_bytes.restype = C.c_size_t
        h.dflash_ctxkv_append.argtypes = [C.c_void_p, C.c_void_p, C.POINTER(C.c_int32), C.c_void_p,
                                          C.POINTER(C.POINTER(KVCacheDesc)), C.c_void_p, C.c_size_t,
                                          C.c_void_p]
        h.dflash_ctxkv_append.restype = C.c_int
        h.dflash_ctxkv_poll_error.argtypes = [C.c_void_p, C.c_void_p]
        h.dflash_ctxkv_poll_error.restype = C.c_int
        h.dflash_ctxkv_set_append_mode.argtypes = [C.c_void_p, C.c_int32]
        h.dflash_ctxkv_set_append_mode.restype = C.c_int
        h.dflash_decoder_create.argtypes = [C.POINTER(DecoderConfig), C.POINTER(DecoderWeights),
                                            C.POINTER(C.c_void_p)]
        h.dflash_decoder_create.restype = C.c_int
        h.dflash_decoder_destroy.argtypes = [C.c_void_p]
        h.dflash_decoder_destroy.restype = None
        h.dflash_decoder_attention.argtypes = [C.c_void_p]
        h.dflash_decoder_attention.restype = C.c_void_p
        h.dflash_decoder_workspace_bytes.argtypes = [C.c_void_p, C.c_int32, C.c_int64]
        h.dflash_decoder_workspace_bytes.restype = C.c_size_t
        h.dflash_decoder_step.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(C.c_int32), C.c_void_p,
                                          C.POINTER(KVCacheDesc), C.c_void_p, C.c_void_p, C.c_size_t,
                                          C.c_void_p]
        h.dflash_decoder_step.restype = C.c_int
        h.dflash_rms_norm.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_double,
                                      C.c_int32, C.c_void_p]
        h.dflash_rms_norm.restype = C.c_int
        h.dflash_workspace_offset.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_int32, C.POINTER(C.c_size_t)]
        h.dflash_workspace_offset.restype = C.c_int
        h.dflash_decoder_workspace_offset.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_int32,
                                                      C.POINTER(C.c_size_t)]
        h.dflash_decoder_workspace_offset.restype = C.c_int
        h.dflash_ctxkv_workspace_offset.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.POINTER(C.c_size_t)]
        h.dflash_ctxkv_workspace_offset.restype = C.c_int
        h.dflash_status_string.argtypes = [C.c_int]
        h.dflash_status_string.restype = C.c_char_p
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().dflash_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != DFLASH_OK:
        raise DFlashError(status, where)
