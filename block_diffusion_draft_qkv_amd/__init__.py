"""DFlash draft-model attention layer step on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``include/dflash.h`` (``libdflash.so``):
it marshals torch tensors (device memory and streams only) into plain
pointers. Every step of the layer runs in the library's HIP kernels; there is
no Python or CPU fallback, and loading fails loudly without the built library.

    layer = DFlashLayer(LayerShape(...), w_qkv, w_o, q_norm, k_norm)
    cache = KVCache(batch, n_kv_heads, head_dim, capacity, dtype)
    out = layer.step(hidden_states, target_hidden, ctx_offsets, positions, cache)
    cache.crop(seq, new_len)
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import DFlashError, check  # noqa: F401

__all__ = ["DFlashLayer", "KVCache", "PagedKVCache", "LayerShape", "ContextKV", "ContextKVShape",
           "DFlashDecoder", "rms_norm", "mxfp8_quantize", "run_round", "DFlashError", "KERNEL_NAMES"]
KERNEL_NAMES = _lib.KERNEL_NAMES

_DTYPES = {torch.float32: _lib.DFLASH_F32, torch.bfloat16: _lib.DFLASH_BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def _check_tensor(t: torch.Tensor, name: str, dtype: torch.dtype, shape, device: torch.device) -> None:
    """The C ABI takes bare pointers and no sizes, so everything the kernels
    assume about a tensor is checked here: exact shape, dtype, contiguity and
    the layer's device (a host tensor would be dereferenced by a kernel)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _check_workspace(ws: torch.Tensor, device: torch.device) -> None:
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if ws.device != device:
        raise ValueError(f"workspace must be on {device}, got {ws.device}")


def _ctx_offsets(ctx_offsets, batch: int) -> np.ndarray:
    offs = np.asarray([int(o) for o in ctx_offsets], dtype=np.int64)
    if offs.shape != (batch + 1,):
        raise ValueError("ctx_offsets must have batch + 1 entries")
    if offs[0] != 0 or (np.diff(offs) < 0).any() or offs[-1] > np.iinfo(np.int32).max:
        raise ValueError("ctx_offsets must start at 0 and be non-decreasing")
    return offs


def _check_cache(cache, shape: "LayerShape", device: torch.device, n_kv_heads: int, head_dim: int) -> None:
    if not isinstance(cache, (KVCache, PagedKVCache)):
        raise ValueError("cache must be a KVCache or PagedKVCache")
    if cache.dtype != shape.dtype or cache.n_kv_heads != n_kv_heads or cache.head_dim != head_dim:
        raise ValueError("cache dtype, KV heads and head_dim must match the layer")
    if cache.k.device != device:
        raise ValueError(f"cache must be on {device}, got {cache.k.device}")
    if isinstance(cache, PagedKVCache) and cache.table.device != device:
        raise ValueError(f"the block table must be on {device}")


def _check_step_args(shape: "LayerShape", device: torch.device, act_dtype: torch.dtype, x: torch.Tensor,
                     target_hidden: Optional[torch.Tensor], ctx_offsets, positions: torch.Tensor, cache,
                     out: Optional[torch.Tensor], workspace: Optional[torch.Tensor], x_name: str):
    """Host checks of a layer (or decoder) step's arguments; returns the
    offsets and the target rows to pass (None when there are none)."""
    _check_cache(cache, shape, device, shape.n_kv_heads, shape.head_dim)
    B, bs, H = cache.batch, shape.block_size, shape.hidden
    offs = _ctx_offsets(ctx_offsets, B)
    mc = int(offs[-1])
    _check_tensor(x, x_name, act_dtype, (B * bs, H), device)
    if target_hidden is not None and target_hidden.numel() == 0 and mc == 0:
        target_hidden = None
    if mc > 0 or target_hidden is not None:
        if target_hidden is None:
            raise ValueError(f"target_hidden is required for {mc} new context rows")
        _check_tensor(target_hidden, "target_hidden", act_dtype, (mc, H), device)
    if positions is not None:  # None: contiguous positions len_b, len_b + 1, ... (the library's)
        _check_tensor(positions, "positions", torch.int32, (mc + B * bs,), device)
    if out is not None:
        _check_tensor(out, "out", act_dtype, (B * bs, H), device)
        if out.data_ptr() == x.data_ptr():
            raise ValueError(f"out must not alias {x_name}")
    if workspace is not None:
        _check_workspace(workspace, device)
    return offs, target_hidden


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    dtype: torch.dtype = torch.bfloat16
    rope_theta: float = 1e6
    rms_eps: float = 1e-6
    sliding_window: int = 0
    max_position: int = 4096 * 32


class KVCache:
    """Draft KV cache of ``batch`` sequences in device memory, block-major.

    Rows come in blocks of 64; block ``i`` of sequence ``b`` holds rows
    ``64 i .. 64 i + 63`` of every KV head: ``k`` is ``[batch, capacity / 64,
    n_kv, 64, head_dim]`` and ``v``, transposed within the block, is ``[batch,
    capacity / 64, n_kv, head_dim, 64]`` (the paged pools' layout with the
    blocks of a sequence in order). ``k_rows()`` and ``vt_rows()`` return
    row-major copies. ``lengths`` is the host array of valid rows that the
    library reads and updates."""

    def __init__(self, batch: int, n_kv_heads: int, head_dim: int, capacity: int,
                 dtype: torch.dtype = torch.bfloat16, device="cuda"):
        if capacity <= 0 or capacity % 64:
            raise ValueError("capacity must be a positive multiple of 64")
        self.batch, self.n_kv_heads, self.head_dim, self.capacity = batch, n_kv_heads, head_dim, capacity
        self.dtype = dtype
        nb = capacity // 64
        self.k = torch.empty((batch, nb, n_kv_heads, 64, head_dim), dtype=dtype, device=device)
        self.v = torch.empty((batch, nb, n_kv_heads, head_dim, 64), dtype=dtype, device=device)
        self._len = (C.c_int32 * max(batch, 1))()
        self.lengths = np.ctypeslib.as_array(self._len)[:batch]
        self.desc = _lib.KVCacheDesc(self.k.data_ptr(), self.v.data_ptr(),
                                     C.cast(self._len, C.POINTER(C.c_int32)), batch, capacity)

    def k_rows(self) -> torch.Tensor:
        """K as ``[batch, n_kv, capacity, head_dim]`` (a copy)."""
        return self.k.permute(0, 2, 1, 3, 4).reshape(self.batch, self.n_kv_heads, self.capacity, self.head_dim)

    def vt_rows(self) -> torch.Tensor:
        """V transposed, ``[batch, n_kv, head_dim, capacity]`` (a copy)."""
        return self.v.permute(0, 2, 3, 1, 4).reshape(self.batch, self.n_kv_heads, self.head_dim, self.capacity)

    def set_lengths(self, lengths: Sequence[int]) -> None:
        self.lengths[:] = np.asarray(lengths, dtype=np.int32)

    def write_prefix(self, seq: int, k: torch.Tensor, v: torch.Tensor) -> None:
        """Place rows ``[0, L)`` of sequence ``seq`` (``k``, ``v``: ``[n_kv, L, d]``)
        and set its length to L."""
        L = k.shape[1]
        if L > self.capacity:
            raise ValueError("prefix longer than the capacity")
        full, rest = divmod(L, 64)
        nkv, d = self.n_kv_heads, self.head_dim
        if full:
            kb = k[:, :full * 64].reshape(nkv, full, 64, d)
            vb = v[:, :full * 64].reshape(nkv, full, 64, d)
            self.k[seq, :full].copy_(kb.transpose(0, 1))
            self.v[seq, :full].copy_(vb.permute(1, 0, 3, 2))
        if rest:
            self.k[seq, full, :, :rest].copy_(k[:, full * 64:])
            self.v[seq, full, :, :, :rest].copy_(v[:, full * 64:].transpose(1, 2))
        self.lengths[seq] = L

    def read(self, seq: int):
        """Valid rows of sequence ``seq`` as ``(k, v)``, each ``[n_kv, len, d]`` (copies)."""
        L = int(self.lengths[seq])
        nb = -(-L // 64)
        nkv, d = self.n_kv_heads, self.head_dim
        k = self.k[seq, :nb].transpose(0, 1).reshape(nkv, nb * 64, d)[:, :L]
        v = self.v[seq, :nb].permute(1, 0, 3, 2).reshape(nkv, nb * 64, d)[:, :L]
        return k, v

    def crop(self, seq: int, new_len: int) -> None:
        check(_lib.lib().dflash_cache_crop(C.byref(self.desc), int(seq), int(new_len)), "dflash_cache_crop")

    def crop_all(self, new_lengths) -> None:
        """Crop every sequence at once (all checked before any changes)."""
        arr = np.ascontiguousarray(new_lengths, dtype=np.int32)
        if arr.shape != (self.batch,):
            raise ValueError("one length per sequence")
        check(_lib.lib().dflash_cache_crop_all(C.byref(self.desc), arr.ctypes.data_as(C.POINTER(C.c_int32))),
              "dflash_cache_crop_all")


class DFlashLayer:
    """One DFlash draft-attention layer over borrowed device weights.

    ``w_qkv`` is ``[(nq + 2 nkv) d, H]`` (rows q heads, k heads, v heads),
    ``w_o`` ``[H, nq d]``, ``q_norm``/``k_norm`` ``[d]``, all in ``shape.dtype``
    on the current device.

    With ``w_qkv_scale`` and ``w_o_scale`` the projections are MXFP8 (bf16
    layers only): ``w_qkv`` and ``w_o`` hold E4M3 codes (uint8) and the scales
    ``[rows, cols / 32]`` their E8M0 bytes."""

    def __init__(self, shape: LayerShape, w_qkv: torch.Tensor, w_o: torch.Tensor,
                 q_norm: torch.Tensor, k_norm: torch.Tensor, w_qkv_scale: Optional[torch.Tensor] = None,
                 w_o_scale: Optional[torch.Tensor] = None):
        self.shape = shape
        self.mxfp8 = w_qkv_scale is not None or w_o_scale is not None
        if self.mxfp8 and (w_qkv_scale is None or w_o_scale is None):
            raise ValueError("MXFP8 layers need both scale tensors")
        self._weights = [t.contiguous() for t in (w_qkv, w_o, q_norm, k_norm)]
        for i, t in enumerate(self._weights):
            want = torch.uint8 if (self.mxfp8 and i < 2) else shape.dtype
            if t.dtype != want or not t.is_cuda:
                raise ValueError("weights must be device tensors of the layer dtype (uint8 codes for MXFP8)")
        cfg = _lib.Config(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                          shape.block_size, shape.sliding_window, shape.max_position,
                          _DTYPES[shape.dtype], float(shape.rope_theta), float(shape.rms_eps))
        handle = C.c_void_p()
        with torch.cuda.device(self._weights[0].device):
            if self.mxfp8:
                scales = [t.contiguous() for t in (w_qkv_scale, w_o_scale)]
                if any(t.dtype != torch.uint8 or not t.is_cuda for t in scales):
                    raise ValueError("scales must be uint8 device tensors")
                self._weights += scales
                wq, wo, qn, kn, sq, so = self._weights
                w = _lib.MXFP8Weights(wq.data_ptr(), sq.data_ptr(), wo.data_ptr(), so.data_ptr(), qn.data_ptr(),
                                      kn.data_ptr())
                check(_lib.lib().dflash_layer_create_mxfp8(C.byref(cfg), C.byref(w), C.byref(handle)),
                      "dflash_layer_create_mxfp8")
            else:
                w = _lib.Weights(*[t.data_ptr() for t in self._weights])
                check(_lib.lib().dflash_layer_create(C.byref(cfg), C.byref(w), C.byref(handle)),
                      "dflash_layer_create")
        self._h = handle
        self.device = self._weights[0].device
        self._ws: Optional[torch.Tensor] = None

    # ------------------------------------------------------------------ api
    def workspace_bytes(self, batch: int, total_ctx: int, total_keys: int = 0) -> int:
        return int(_lib.lib().dflash_workspace_bytes(self._h, batch, total_ctx, total_keys))

    def workspace(self, batch: int, total_ctx: int) -> torch.Tensor:
        need = self.workspace_bytes(batch, total_ctx)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def step(self, hidden_states: torch.Tensor, target_hidden: Optional[torch.Tensor],
             ctx_offsets, positions: torch.Tensor, cache: KVCache,
             out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
        s = self.shape
        offs, target_hidden = _check_step_args(s, self.device, s.dtype, hidden_states, target_hidden, ctx_offsets,
                                               positions, cache, out, workspace, "hidden_states")
        c_offs = (C.c_int32 * (cache.batch + 1))(*offs.tolist())
        if out is None:
            out = torch.empty((cache.batch * s.block_size, s.hidden), dtype=s.dtype, device=self.device)
        if workspace is None:
            workspace = self.workspace(cache.batch, int(offs[-1]))
        st = _lib.lib().dflash_attn_step(self._h, _ptr(hidden_states), _ptr(target_hidden), c_offs,
                                         _ptr(positions), C.byref(cache.desc), _ptr(out),
                                         _ptr(workspace), workspace.numel(), _stream_handle(stream))
        check(st, "dflash_attn_step")
        return out

    def step_noalloc(self, hidden_states: torch.Tensor, target_hidden: Optional[torch.Tensor], ctx_offsets,
                     positions: torch.Tensor, cache: KVCache, out: torch.Tensor, stream=None) -> torch.Tensor:
        """``step`` for callers that cannot allocate: no workspace, the
        library's per-device scratch instead (``out`` must be given; calls on
        one device must not overlap)."""
        s = self.shape
        if out is None:
            raise ValueError("step_noalloc writes a caller-given out")
        offs, target_hidden = _check_step_args(s, self.device, s.dtype, hidden_states, target_hidden, ctx_offsets,
                                               positions, cache, out, None, "hidden_states")
        c_offs = (C.c_int32 * (cache.batch + 1))(*offs.tolist())
        st = _lib.lib().dflash_attn_step_noalloc(self._h, _ptr(hidden_states), _ptr(target_hidden), c_offs,
                                                 _ptr(positions), C.byref(cache.desc), _ptr(out),
                                                 _stream_handle(stream))
        check(st, "dflash_attn_step_noalloc")
        return out

    def workspace_region(self, workspace: torch.Tensor, batch: int, total_ctx: int, region: str) -> torch.Tensor:
        """A view into ``workspace`` (as passed to ``step``) of an intermediate
        the step left there: ``"attn_out"`` ``[B*bs, nq*d]`` in the dtype,
        ``"attn_out_mx"`` (E4M3 codes, uint8, same shape) or
        ``"attn_out_mx_scales"`` (``[nq*d/128, B*bs, 4]`` E8M0 bytes)."""
        off = C.c_size_t()
        check(_lib.lib().dflash_workspace_offset(self._h, int(batch), int(total_ctx), _lib.WS_REGIONS[region],
                                                 C.byref(off)), "dflash_workspace_offset")
        s = self.shape
        rows, od = batch * s.block_size, s.n_q_heads * s.head_dim
        if region == "attn_out":
            es = 2 if s.dtype == torch.bfloat16 else 4
            return workspace[off.value:off.value + rows * od * es].view(s.dtype).view(rows, od)
        if region == "attn_out_mx":
            return workspace[off.value:off.value + rows * od].view(rows, od)
        return workspace[off.value:off.value + rows * od // 32].view(od // 128, rows, 4)

    def poll_error(self, stream=None) -> int:
        return int(_lib.lib().dflash_layer_poll_error(self._h, _stream_handle(stream)))

    def set_append_mode(self, mode: str) -> None:
        """Where q/k are normalised and rotated and the cache rows appended:
        ``"auto"`` (default), ``"fused"`` (projection epilogue) or ``"separate"``."""
        check(_lib.lib().dflash_layer_set_append_mode(self._h, _lib.APPEND_MODES[mode]), "set_append_mode")

    def set_profiling(self, enable) -> None:
        """``True`` / ``"kernels"``: HIP events around each kernel of a step;
        ``"attn_span"``: one pair around the attention and its merge
        (``"attn_merge"`` in ``kernel_times``); ``False`` / ``"off"``."""
        if enable not in _lib.PROFILE_MODES:
            raise ValueError(f"unknown profiling mode {enable!r}")
        check(_lib.lib().dflash_layer_set_profiling(self._h, _lib.PROFILE_MODES[enable]), "set_profiling")

    def kernel_times(self):
        """``{kernel name: (total ms, launches)}`` since profiling was enabled."""
        ms = (C.c_double * len(KERNEL_NAMES))()
        cnt = (C.c_int64 * len(KERNEL_NAMES))()
        check(_lib.lib().dflash_layer_kernel_times(self._h, ms, cnt), "kernel_times")
        return {n: (ms[i], cnt[i]) for i, n in enumerate(KERNEL_NAMES)}

    def close(self) -> None:
        if getattr(self, "_h", None):
            _lib.lib().dflash_layer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


@dataclass(frozen=True)
class ContextKVShape:
    hidden: int
    n_layers: int
    n_kv_heads: int
    head_dim: int
    dtype: torch.dtype = torch.bfloat16
    rope_theta: float = 1e6
    rms_eps: float = 1e-6
    max_position: int = 4096 * 32


class ContextKV:
    """Context K/V of every draft layer at once (the multi-layer precompute):
    ``hidden_norm`` ``[H]``, ``w_kv`` ``[L * 2 * nkv * d, H]`` (each layer's K
    rows then V rows), ``k_norm`` ``[L, d]``, device tensors in ``shape.dtype``.

    With ``w_kv_scale`` the weights are MXFP8 (bf16 only): ``w_kv`` holds E4M3
    codes (uint8) and ``w_kv_scale`` ``[L * 2 * nkv * d, H / 32]`` their E8M0
    block scales (uint8), and the projection is the block-scaled GEMM."""

    def __init__(self, shape: ContextKVShape, hidden_norm: torch.Tensor, w_kv: torch.Tensor,
                 k_norm: torch.Tensor, w_kv_scale: Optional[torch.Tensor] = None):
        self.shape = shape
        self.mxfp8 = w_kv_scale is not None
        self._weights = [t.contiguous() for t in (hidden_norm, w_kv, k_norm)]
        for i, t in enumerate(self._weights):
            want = torch.uint8 if (self.mxfp8 and i == 1) else shape.dtype
            if t.dtype != want or not t.is_cuda:
                raise ValueError("weights must be device tensors of the dtype (uint8 codes for MXFP8)")
        cfg = _lib.CtxKVConfig(shape.hidden, shape.n_layers, shape.n_kv_heads, shape.head_dim,
                               shape.max_position, _DTYPES[shape.dtype], float(shape.rope_theta),
                               float(shape.rms_eps))
        handle = C.c_void_p()
        with torch.cuda.device(self._weights[0].device):
            if self.mxfp8:
                sc = w_kv_scale.contiguous()
                if sc.dtype != torch.uint8 or not sc.is_cuda:
                    raise ValueError("w_kv_scale must be a uint8 device tensor")
                self._weights.append(sc)
                hn, wk, kn = self._weights[:3]
                w = _lib.CtxKVMXFP8Weights(hn.data_ptr(), wk.data_ptr(), sc.data_ptr(), kn.data_ptr())
                check(_lib.lib().dflash_ctxkv_create_mxfp8(C.byref(cfg), C.byref(w), C.byref(handle)),
                      "dflash_ctxkv_create_mxfp8")
            else:
                w = _lib.CtxKVWeights(*[t.data_ptr() for t in self._weights])
                check(_lib.lib().dflash_ctxkv_create(C.byref(cfg), C.byref(w), C.byref(handle)),
                      "dflash_ctxkv_create")
        self._h = handle
        self.device = self._weights[0].device
        self._ws: Optional[torch.Tensor] = None

    def workspace(self, total_ctx: int) -> torch.Tensor:
        need = int(_lib.lib().dflash_ctxkv_workspace_bytes(self._h, int(total_ctx)))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def append(self, context_states: torch.Tensor, ctx_offsets, positions: torch.Tensor,
               caches: Sequence[KVCache], workspace: Optional[torch.Tensor] = None, stream=None) -> None:
        """Append every sequence's new context rows to every layer's cache."""
        s = self.shape
        if len(caches) != s.n_layers:
            raise ValueError("one cache per layer")
        B = caches[0].batch
        for c in caches:
            _check_cache(c, LayerShape(s.hidden, 1, s.n_kv_heads, s.head_dim, 1, s.dtype), self.device,
                         s.n_kv_heads, s.head_dim)
            if c.batch != B:
                raise ValueError("every layer's cache must hold the same sequences")
        offs = _ctx_offsets(ctx_offsets, B)
        mc = int(offs[-1])
        _check_tensor(context_states, "context_states", s.dtype, (mc, s.hidden), self.device)
        if positions is not None:  # None: contiguous positions len_b, len_b + 1, ...
            _check_tensor(positions, "positions", torch.int32, (mc,), self.device)
        if workspace is not None:
            _check_workspace(workspace, self.device)
        offs = (C.c_int32 * (B + 1))(*offs.tolist())
        descs = (C.POINTER(_lib.KVCacheDesc) * s.n_layers)(*[C.pointer(c.desc) for c in caches])
        if workspace is None:
            workspace = self.workspace(int(ctx_offsets[-1]))
        st = _lib.lib().dflash_ctxkv_append(self._h, _ptr(context_states), offs, _ptr(positions), descs,
                                            _ptr(workspace), workspace.numel(), _stream_handle(stream))
        check(st, "dflash_ctxkv_append")

    def workspace_region(self, workspace: torch.Tensor, total_ctx: int, region: str) -> torch.Tensor:
        """A view into ``workspace`` (as passed to ``append``) of the
        hidden_norm-ed rows the append left there: ``"normed"`` ``[rows, H]``
        (the dtype, or uint8 E4M3 codes with MXFP8 weights) or
        ``"normed_mx_scales"`` (``[H/128, rows, 4]`` E8M0 bytes)."""
        off = C.c_size_t()
        check(_lib.lib().dflash_ctxkv_workspace_offset(self._h, int(total_ctx), _lib.CTX_WS_REGIONS[region],
                                                       C.byref(off)), "dflash_ctxkv_workspace_offset")
        s, rows = self.shape, int(total_ctx)
        if region == "normed_mx_scales":
            return workspace[off.value:off.value + rows * s.hidden // 32].view(s.hidden // 128, rows, 4)
        if self.mxfp8:
            return workspace[off.value:off.value + rows * s.hidden].view(rows, s.hidden)
        es = 2 if s.dtype == torch.bfloat16 else 4
        return workspace[off.value:off.value + rows * s.hidden * es].view(s.dtype).view(rows, s.hidden)

    def set_fc(self, w_fc: Optional[torch.Tensor]) -> None:
        """Register the fc weight ``[H, fc_in]`` (the dtype, device) used by
        ``combine``; None removes it."""
        if w_fc is None:
            self._fc = None
            check(_lib.lib().dflash_ctxkv_set_fc(self._h, None, 0), "dflash_ctxkv_set_fc")
            return
        w = w_fc.contiguous()
        if w.dtype != self.shape.dtype or not w.is_cuda or w.dim() != 2 or w.shape[0] != self.shape.hidden:
            raise ValueError("fc weight must be a [hidden, fc_in] device tensor of the dtype")
        check(_lib.lib().dflash_ctxkv_set_fc(self._h, w.data_ptr(), w.shape[1]), "dflash_ctxkv_set_fc")
        self._fc = w

    def combine(self, aux_states: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """The fc projection of concatenated target-layer features
        ``[rows, fc_in]`` -> context states ``[rows, H]`` for ``append``."""
        if getattr(self, "_fc", None) is None:
            raise ValueError("no fc weight set")
        a = aux_states.contiguous()
        if a.dim() != 2:
            raise ValueError("aux_states must be [rows, fc_in] in the dtype")
        _check_tensor(a, "aux_states", self.shape.dtype, (a.shape[0], self._fc.shape[1]), self.device)
        if out is None:
            out = torch.empty((a.shape[0], self.shape.hidden), dtype=a.dtype, device=a.device)
        _check_tensor(out, "out", self.shape.dtype, (a.shape[0], self.shape.hidden), self.device)
        need = int(_lib.lib().dflash_ctxkv_combine_workspace_bytes(self._h, a.shape[0]))
        if getattr(self, "_fc_ws", None) is None or self._fc_ws.numel() < need:
            self._fc_ws = torch.empty(need, dtype=torch.uint8, device=a.device)
        check(_lib.lib().dflash_ctxkv_combine(self._h, _ptr(a), a.shape[0], _ptr(out), _ptr(self._fc_ws),
                                              self._fc_ws.numel(), _stream_handle(stream)),
              "dflash_ctxkv_combine")
        return out

    def set_append_mode(self, mode: str) -> None:
        """``"auto"`` (default), ``"fused"`` (projection epilogue) or ``"separate"``."""
        check(_lib.lib().dflash_ctxkv_set_append_mode(self._h, _lib.APPEND_MODES[mode]), "set_append_mode")

    def poll_error(self, stream=None) -> int:
        return int(_lib.lib().dflash_ctxkv_poll_error(self._h, _stream_handle(stream)))

    def close(self) -> None:
        if getattr(self, "_h", None):
            _lib.lib().dflash_ctxkv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mxfp8_quantize(x: torch.Tensor, stream=None):
    """MXFP8 codes ``[rows, cols]`` and E8M0 scales ``[rows, cols / 32]``
    (uint8 device tensors) of a bf16 device matrix, by the rule the MXFP8
    precompute applies to its activations."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 2:
        raise ValueError("x must be a 2-D bf16 device tensor")
    x = x.contiguous()
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    check(_lib.lib().dflash_mxfp8_quantize(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream_handle(stream)),
          "dflash_mxfp8_quantize")
    return codes, scales


class _BorrowedLayer(DFlashLayer):
    """The attention layer a decoder owns (no destroy of its own)."""

    def __init__(self, shape: LayerShape, handle, device: torch.device):
        self.shape = shape
        self._h = handle
        self._weights = []
        self.device = device
        self._ws = None

    def close(self) -> None:
        self._h = None


class DFlashDecoder:
    """One draft decoder layer: input_layernorm, the attention layer step,
    residual add, post_attention_layernorm, SwiGLU MLP, residual add.
    ``w_gate_up`` is ``[2 I, H]`` (gate rows, then up rows), ``w_down``
    ``[H, I]``; the attention weights are those of ``DFlashLayer``."""

    def __init__(self, shape: LayerShape, intermediate: int, w_qkv, w_o, q_norm, k_norm, input_norm, post_norm,
                 w_gate_up, w_down):
        self.shape, self.intermediate = shape, int(intermediate)
        self._weights = [t.contiguous() for t in (w_qkv, w_o, q_norm, k_norm, input_norm, post_norm, w_gate_up,
                                                  w_down)]
        for t in self._weights:
            if t.dtype != shape.dtype or not t.is_cuda:
                raise ValueError("weights must be device tensors of the layer dtype")
        acfg = _lib.Config(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.block_size,
                           shape.sliding_window, shape.max_position, _DTYPES[shape.dtype], float(shape.rope_theta),
                           float(shape.rms_eps))
        cfg = _lib.DecoderConfig(acfg, self.intermediate)
        p = [t.data_ptr() for t in self._weights]
        w = _lib.DecoderWeights(_lib.Weights(*p[:4]), *p[4:])
        handle = C.c_void_p()
        with torch.cuda.device(self._weights[0].device):
            check(_lib.lib().dflash_decoder_create(C.byref(cfg), C.byref(w), C.byref(handle)),
                  "dflash_decoder_create")
        self._h = handle
        self.device = self._weights[0].device
        self._ws: Optional[torch.Tensor] = None
        self.attention = _BorrowedLayer(shape, C.c_void_p(_lib.lib().dflash_decoder_attention(handle)),
                                        self.device)

    def workspace(self, batch: int, total_ctx: int) -> torch.Tensor:
        need = int(_lib.lib().dflash_decoder_workspace_bytes(self._h, int(batch), int(total_ctx)))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def step(self, x: torch.Tensor, target_hidden: Optional[torch.Tensor], ctx_offsets, positions: torch.Tensor,
             cache: KVCache, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
        s = self.shape
        offs, target_hidden = _check_step_args(s, self.device, s.dtype, x, target_hidden, ctx_offsets, positions,
                                               cache, out, workspace, "x")
        c_offs = (C.c_int32 * (cache.batch + 1))(*offs.tolist())
        if out is None:
            out = torch.empty_like(x)
        if workspace is None:
            workspace = self.workspace(cache.batch, int(offs[-1]))
        st = _lib.lib().dflash_decoder_step(self._h, _ptr(x), _ptr(target_hidden), c_offs, _ptr(positions),
                                            C.byref(cache.desc), _ptr(out), _ptr(workspace), workspace.numel(),
                                            _stream_handle(stream))
        check(st, "dflash_decoder_step")
        return out

    def workspace_region(self, workspace: torch.Tensor, batch: int, total_ctx: int, region: str) -> torch.Tensor:
        """A view into ``workspace`` (as passed to ``step``) of an intermediate
        the step left there, in the dtype: ``"a"``, ``"att"``, ``"h"``, ``"m"``
        (``[B*bs, H]``) or ``"act"`` (``[B*bs, I]``)."""
        off = C.c_size_t()
        check(_lib.lib().dflash_decoder_workspace_offset(self._h, int(batch), int(total_ctx),
                                                         _lib.DEC_WS_REGIONS[region], C.byref(off)),
              "dflash_decoder_workspace_offset")
        s = self.shape
        rows = batch * s.block_size
        cols = self.intermediate if region == "act" else s.hidden
        es = 2 if s.dtype == torch.bfloat16 else 4
        return workspace[off.value:off.value + rows * cols * es].view(s.dtype).view(rows, cols)

    def poll_error(self, stream=None) -> int:
        return self.attention.poll_error(stream)

    def close(self) -> None:
        if getattr(self, "_h", None):
            _lib.lib().dflash_decoder_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def rms_norm(x: torch.Tensor, gain: torch.Tensor, eps: float, out: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
    """Row RMSNorm (the draft model's final norm) of a contiguous [rows, H] tensor."""
    if x.dtype not in _DTYPES or x.dim() not in (1, 2):
        raise ValueError("x must be a contiguous [rows, H] (or [H]) fp32 or bf16 tensor")
    rows, h = (x.shape[0], x.shape[1]) if x.dim() == 2 else (1, x.shape[0])
    _check_tensor(x, "x", x.dtype, tuple(x.shape), x.device)
    _check_tensor(gain, "gain", x.dtype, (h,), x.device)
    if out is None:
        out = torch.empty_like(x)
    _check_tensor(out, "out", x.dtype, tuple(x.shape), x.device)
    st = _lib.lib().dflash_rms_norm(_ptr(x), _ptr(gain), _ptr(out), int(rows), int(h), float(eps), _DTYPES[x.dtype],
                                    _stream_handle(stream))
    check(st, "dflash_rms_norm")
    return out


class PagedKVCache:
    """Draft KV cache of ``batch`` sequences in 64-row blocks (the paged layout
    of include/dflash.h): pools ``k [num_blocks, n_kv, 64, d]`` and ``v
    [num_blocks, n_kv, d, 64]``, a block table per sequence (``max_blocks``
    entries; a device copy for the kernels and the host copy the library
    checks) and the library's block pool (``dflash_block_pool``), which hands
    out and takes back physical blocks and records the table entries it
    changes until ``sync`` writes them to the device table. Blocks are
    reserved before a step writes rows and released when a crop drops them."""

    BLOCK = 64

    def __init__(self, batch: int, n_kv_heads: int, head_dim: int, num_blocks: int, max_blocks: int,
                 dtype: torch.dtype = torch.bfloat16, device="cuda"):
        self.batch, self.n_kv_heads, self.head_dim = batch, n_kv_heads, head_dim
        self.num_blocks, self.max_blocks, self.dtype = num_blocks, max_blocks, dtype
        self.capacity = max_blocks * self.BLOCK
        B = self.BLOCK
        self.k = torch.empty((num_blocks, n_kv_heads, B, head_dim), dtype=dtype, device=device)
        self.v = torch.empty((num_blocks, n_kv_heads, head_dim, B), dtype=dtype, device=device)
        self._tab = (C.c_int32 * (batch * max_blocks))(*([-1] * (batch * max_blocks)))
        self.table_host = np.ctypeslib.as_array(self._tab).reshape(batch, max_blocks)
        self.table = torch.full((batch, max_blocks), -1, dtype=torch.int32, device=device)
        self._len = (C.c_int32 * max(batch, 1))()
        self.lengths = np.ctypeslib.as_array(self._len)[:batch]
        self.desc = _lib.KVCacheDesc(self.k.data_ptr(), self.v.data_ptr(), C.cast(self._len, C.POINTER(C.c_int32)),
                                     batch, self.capacity, self.table.data_ptr(),
                                     C.cast(self._tab, C.POINTER(C.c_int32)), max_blocks, num_blocks)
        self._pool = C.c_void_p()
        check(_lib.lib().dflash_block_pool_create(int(num_blocks), C.byref(self._pool)), "dflash_block_pool_create")

    def __del__(self):
        pool = getattr(self, "_pool", None)
        if pool and _lib._lib is not None:
            _lib._lib.dflash_block_pool_destroy(pool)
            self._pool = None

    # ------------------------------------------------------------ blocks
    @property
    def free(self) -> list:
        """The free blocks, bottom of the stack first (the last is taken next);
        assigning a list (e.g. a shuffled order) replaces them."""
        n = int(_lib.lib().dflash_block_pool_free_count(self._pool))
        buf = (C.c_int32 * max(n, 1))()
        check(_lib.lib().dflash_block_pool_get_free(self._pool, buf, n), "dflash_block_pool_get_free")
        return list(buf[:n])

    @free.setter
    def free(self, blocks) -> None:
        arr = np.ascontiguousarray(blocks, dtype=np.int32)
        check(_lib.lib().dflash_block_pool_set_free(self._pool, arr.ctypes.data_as(C.POINTER(C.c_int32)),
                                                    int(arr.size)), "dflash_block_pool_set_free")

    def _pool_call(self, fn, *args) -> None:
        st = fn(C.byref(self.desc), self._pool, *args)
        if st == _lib.DFLASH_ERR_SHAPE:
            raise ValueError(f"a sequence would need more than max_blocks {self.max_blocks} blocks")
        if st == _lib.DFLASH_ERR_CAPACITY:
            raise MemoryError("no free cache block")
        check(st, fn.__name__)

    def blocks_of(self, seq: int) -> int:
        return int(np.count_nonzero(self.table_host[seq] >= 0))

    def reserve(self, seq: int, rows: int) -> None:
        """Back logical rows [0, rows) of ``seq`` with blocks (all or nothing)."""
        self._pool_call(_lib.lib().dflash_cache_reserve, int(seq), int(rows))

    def release(self, seq: int, rows: int) -> None:
        """Return the blocks of ``seq`` past logical row ``rows`` to the pool."""
        self._pool_call(_lib.lib().dflash_cache_release, int(seq), int(rows))

    def reserve_all(self, rows) -> None:
        """``reserve`` for every sequence at once (sequence 0 first)."""
        arr = np.ascontiguousarray(rows, dtype=np.int64)
        if arr.shape != (self.batch,):
            raise ValueError("one row count per sequence")
        self._pool_call(_lib.lib().dflash_cache_reserve_all, arr.ctypes.data_as(C.POINTER(C.c_int64)))

    def release_all(self, rows) -> None:
        """``release`` for every sequence at once (blocks past logical row
        rows[b] go back sequence by sequence, last block first)."""
        arr = np.ascontiguousarray(rows, dtype=np.int64)
        if arr.shape != (self.batch,):
            raise ValueError("one row count per sequence")
        self._pool_call(_lib.lib().dflash_cache_release_all, arr.ctypes.data_as(C.POINTER(C.c_int64)))

    def crop_all(self, new_lengths) -> None:
        """Crop every sequence at once (all checked before any changes) and
        release the blocks the crops drop."""
        arr = np.ascontiguousarray(new_lengths, dtype=np.int32)
        if arr.shape != (self.batch,):
            raise ValueError("one length per sequence")
        check(_lib.lib().dflash_cache_crop_all(C.byref(self.desc), arr.ctypes.data_as(C.POINTER(C.c_int32))),
              "dflash_cache_crop_all")
        self.release_all(arr)

    def sync(self, stream=None) -> None:
        """Write the table entries the pool changed to the device table, ordered
        on the stream before the steps enqueued after it (small patch kernels;
        the host table may change again at once)."""
        if int(_lib.lib().dflash_block_pool_pending(self._pool)) == 0:
            return
        if self.table.device.type != "cuda":  # a host-resident cache (block accounting only)
            self.table.copy_(torch.from_numpy(self.table_host))
            check(_lib.lib().dflash_block_pool_drop_pending(self._pool), "dflash_block_pool_drop_pending")
            return
        with torch.cuda.device(self.table.device):
            check(_lib.lib().dflash_cache_push_table(C.byref(self.desc), self._pool, _stream_handle(stream)),
                  "dflash_cache_push_table")

    # ------------------------------------------------------------ rows
    def _slots(self, seq: int, r0: int, r1: int):
        rows = np.arange(r0, r1)
        return self.table_host[seq, rows // self.BLOCK], rows % self.BLOCK

    def write_prefix(self, seq: int, k: torch.Tensor, v: torch.Tensor) -> None:
        """Place rows [0, L) of ``seq`` (``k``, ``v``: ``[n_kv, L, d]``) and set its length to L."""
        L = int(k.shape[1])
        self.reserve(seq, L)
        self.sync()
        blk, off = self._slots(seq, 0, L)
        bi = torch.from_numpy(blk.astype(np.int64)).to(self.k.device)
        oi = torch.from_numpy(off.astype(np.int64)).to(self.k.device)
        self.k[bi, :, oi, :] = k.transpose(0, 1).to(self.dtype)
        self.v.permute(0, 3, 1, 2)[bi, oi] = v.transpose(0, 1).to(self.dtype)
        self.lengths[seq] = L

    def read(self, seq: int):
        """Valid rows of ``seq`` gathered as ``(k, v)``, each ``[n_kv, len, d]``."""
        L = int(self.lengths[seq])
        blk, off = self._slots(seq, 0, L)
        bi = torch.from_numpy(blk.astype(np.int64)).to(self.k.device)
        oi = torch.from_numpy(off.astype(np.int64)).to(self.k.device)
        k = self.k[bi, :, oi, :].transpose(0, 1)
        v = self.v.permute(0, 3, 1, 2)[bi, oi].transpose(0, 1)
        return k, v

    def set_lengths(self, lengths: Sequence[int]) -> None:
        self.lengths[:] = np.asarray(lengths, dtype=np.int32)

    def crop(self, seq: int, new_len: int) -> None:
        """Rewind ``seq`` to ``new_len`` rows and release the blocks past them."""
        check(_lib.lib().dflash_cache_crop(C.byref(self.desc), int(seq), int(new_len)), "dflash_cache_crop")
        self.release(seq, new_len)


def run_round(model, cache, hidden_states: torch.Tensor, target_hidden: Optional[torch.Tensor], ctx_offsets,
              accept: Sequence[int], out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One draft round on a paged (or contiguous) cache: reserve the blocks the
    step appends to and push the table entries that changed, run the layer (or
    decoder) step at the contiguous positions len_b .. len_b + n_b + bs - 1
    (computed by the kernels), then crop each sequence to its accepted prefix
    len_b + n_b + accept[b], releasing the blocks a crop drops."""
    B, bs = cache.batch, model.shape.block_size
    L = cache.lengths.astype(np.int64)
    n = np.diff(np.asarray(ctx_offsets, dtype=np.int64))
    acc = np.asarray(accept, dtype=np.int64)
    if acc.shape != (B,) or (acc < 0).any() or (acc > bs).any():
        raise ValueError("accepted counts: one per sequence, each in [0, block_size]")
    keep = L + n + acc
    if isinstance(cache, PagedKVCache):
        cache.reserve_all(L + n + bs)
        cache.sync(stream)
    out = model.step(hidden_states, target_hidden, ctx_offsets, None, cache, out=out, stream=stream)
    cache.crop_all(keep)
    return out
