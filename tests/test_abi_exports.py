"""The C-ABI library loads and exports every entry point include/dflash.h
declares; host-only entry points behave without a GPU (no compute calls)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")
LIB = os.path.join(ROOT, "block_diffusion_draft_qkv_amd", "libdflash.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdflash.so not built")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    from block_diffusion_draft_qkv_amd import _lib
    assert sorted(_lib.EXPORTS) == declared()


def test_every_declared_symbol_is_exported():
    lib = C.CDLL(LIB)
    for name in declared():
        assert hasattr(lib, name), name


def test_host_only_entry_points_without_gpu():
    from block_diffusion_draft_qkv_amd import _lib
    h = _lib.lib()
    assert h.dflash_status_string(0) == b"ok"
    assert h.dflash_status_string(3).startswith(b"step would exceed")
    assert h.dflash_workspace_bytes(None, 1, 0, 0) == 0
    # crop is host-only: lengths change, nothing else
    lens = (C.c_int32 * 2)(10, 5)
    cache = _lib.KVCacheDesc(None, None, C.cast(lens, C.POINTER(C.c_int32)), 2, 64)
    assert h.dflash_cache_crop(C.byref(cache), 0, 7) == 0 and list(lens) == [7, 5]
    assert h.dflash_cache_crop(C.byref(cache), 1, 6) == _lib.DFLASH_ERR_RANGE
    assert h.dflash_cache_crop(C.byref(cache), 1, -1) == _lib.DFLASH_ERR_RANGE
    assert h.dflash_cache_crop(C.byref(cache), 2, 0) == _lib.DFLASH_ERR_ARG
    assert h.dflash_cache_crop(None, 0, 0) == _lib.DFLASH_ERR_ARG
    assert list(lens) == [7, 5]
    # a step with no layer is rejected before any HIP call
    assert h.dflash_attn_step(None, None, None, None, None, None, None, None, 0, None) == _lib.DFLASH_ERR_ARG
    assert h.dflash_layer_create(None, None, None) == _lib.DFLASH_ERR_ARG
