#!/usr/bin/env python3
"""Throughput of the DFlash draft-attention layer step on one MI355X.

Workload: a batched ragged decode round of the Qwen3-8B-shaped draft layer
(hidden 4096, 32 Q / 8 KV heads, head_dim 128, block 16, bf16): B=32 sequences
with cached context U{512..8192}, U{1..16} new context rows each, the step,
then the crop of every sequence to its accepted prefix (accepted count
U{0..16}). Inputs are synthetic and seeded (workload.make_case) and already
resident in HBM when timing starts. Several copies of the KV cache rotate from
step to step so the 256 MB Infinity Cache cannot serve a cache that the
previous step just streamed.

One "step" = the whole hot path: grouped QKV/context-KV GEMM, norm+RoPE+append,
split-KV attention, the merge of split pairs, o_proj, and the
crop. Between timed steps the lengths are rewound to the round's starting
lengths (host-only) so that every step sees the same workload.

Prints ONE JSON line. ``value`` is draft-block tokens/s (B*bs per step);
``roofline`` covers the attention kernel (HBM-bound): algorithmic bytes per
launch (K and V rows once, Q and O once) over its mean launch time, measured
with HIP events on the launch stream in a second pass of the same K steps
(events are kept out of the timed region that gives ``value``).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft-block tokens/s + attention HBM GB/s (% of peak), B=32 ctx 512–8K"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_merge_c3_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "projection_gemms_c3_mfma_counters.json")
# every source the attention and merge kernels are compiled and planned from
ATTN_SOURCES = [os.path.join(ROOT, "block_diffusion_draft_qkv_amd", "csrc", f)
                for f in ("attention.hip", "kernels.h", "common.h", "lds_dma.h", "dflash.cpp")]
# every source the projection GEMMs are compiled and planned from
GEMM_SOURCES = [os.path.join(ROOT, "block_diffusion_draft_qkv_amd", "csrc", f)
                for f in ("gemm.hip", "kernels.h", "common.h", "lds_dma.h", "dflash.cpp")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="C3", help="workload (C3 is the reported one)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copies", type=int, default=3, help="KV-cache copies rotated across steps")
    ap.add_argument("--cpu-sample", type=int, default=32,
                    help="sequences of the workload the oracle is timed on (0: skip)")
    ap.add_argument("--append-mode", default="auto", choices=("auto", "fused", "separate"),
                    help="where q/k norm + RoPE + cache append run (projection epilogue or own kernel)")
    ap.add_argument("--ctxkv-steps", type=int, default=50,
                    help="timed runs of the multi-layer context K/V precompute (0: skip)")
    ap.add_argument("--decoder-steps", type=int, default=30,
                    help="timed steps of the whole draft decoder layer at C3 (0: skip)")
    ap.add_argument("--paged-steps", type=int, default=50,
                    help="timed C3 steps on the paged cache, and as many driver rounds (0: skip)")
    ap.add_argument("--mxfp8-steps", type=int, default=50,
                    help="timed C3 steps of the layer with MXFP8 projections (0: skip)")
    ap.add_argument("--other-steps", type=int, default=30,
                    help="steps of the C4 and C5 layer step measurements (0 skips them)")
    ap.add_argument("--mxfp8-only", action="store_true",
                    help="only time the C3 layer step with MXFP8 projections (for profiling)")
    ap.add_argument("--decoder-only", action="store_true",
                    help="only time the draft decoder layer (for profiling)")
    ap.add_argument("--context-kv-only", default=None, choices=("P3", "P4"),
                    help="only time the context K/V precompute on this workload (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed steps before the warm-up steps, so the GPU clocks reach the "
                         "level they hold under sustained load (0: none)")
    return ap.parse_args()


SETTLE_S = 1.0  # set from --settle in main()


def settle(step, seconds: float = None) -> int:
    """Run `step(i)` for a fixed wall time, untimed, so that the GPU clocks
    reach the level they hold under sustained load (they drop during the host
    set-up of each workload); returns the number of calls."""
    import torch
    seconds = SETTLE_S if seconds is None else seconds
    n = 0
    if seconds <= 0:
        return 0
    torch.cuda.synchronize()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_per_launch(workload: str):
    """HBM bytes of one attention launch and its merge from the committed
    counter summary, or None when there is none, it covers another workload,
    or the kernels' sources changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if not rec.get("workload", "").startswith(workload):
        return None
    if rec.get("attention_source_sha256_16") != source_hash(ATTN_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


def mfma_counters(workload: str):
    """The projection GEMMs' MFMA counters (utilisation, counted flops per
    dispatch duration) from the committed counter summary, or None when there
    is none, it covers another workload, or the GEMM sources changed since."""
    try:
        rec = json.load(open(MFMA_FILE))
    except (OSError, ValueError):
        return None
    if not rec.get("workload", "").startswith(workload) or rec.get("gemm_source_sha256_16") != source_hash(GEMM_SOURCES):
        return None
    return {k: {"mfma_util": v["mfma_util"], "counted_tflops": v["tflops"], "dispatch_us": v["dispatch_us"]}
            for k, v in rec["kernels"].items()}


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def cpu_baseline(case, n_seq: int, runs: int = 5):
    """Time the float64 oracle on the first n_seq sequences of the workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    k = min(n_seq, case.batch)
    bs = case.cfg.block_size
    offs = case.ctx_offsets[:k + 1]
    npos = int(offs[-1]) + k * bs
    cache = oracle.OracleCache.from_arrays(case.cache_k[:k], case.cache_v[:k])
    args = (case.cfg, case.weights, cache, case.hidden_states[:k * bs],
            case.target_hidden[:int(offs[-1])], offs, case.positions[:npos])
    times = []
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        if ctx:
            ctx.__enter__()
        for _ in range(runs):
            t0 = time.perf_counter()
            oracle.layer_step(*args)
            times.append(time.perf_counter() - t0)
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    t = float(np.median(times))
    return {"value": k * bs / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{k} of {case.batch} sequences of the same workload "
                      f"({int(case.total_len[:k].sum())} keys), float64 numpy, median of "
                      f"{len(times)} runs of {t:.2f}s"}


def cold_weight_steps(step, layer, n: int, i0: int) -> dict:
    """The projections' weights from HBM. Back-to-back steps find part of the
    q|k|v and o_proj weights still in the 256 MB memory-side cache from the
    step before; in a serving loop the target model runs in between. So the
    same steps one by one, each timed with an event pair on the launch stream
    and preceded by GPU work that lets the host enqueue the step ahead of the
    GPU: first a short spin that touches no memory (weights as the previous
    step left them), then a 1 GiB copy that streams through that cache; and
    their kernels with per-kernel events."""
    import torch
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    res = {}
    for mode in ("warm", "cold"):
        pairs = []
        for i in range(n):
            if mode == "cold":
                dst.copy_(src)
            else:
                torch.cuda._sleep(400_000)  # ~0.2 ms, no memory traffic
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step(i0 + i)
            e1.record()
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
        layer.set_profiling(True)
        for i in range(n):
            if mode == "cold":
                dst.copy_(src)
            step(i0 + n + i)
        torch.cuda.synchronize()
        kt = layer.kernel_times()
        layer.set_profiling(False)
        res[mode] = {"step_us_median": round(t[len(t) // 2], 1),
                     "gemm_qkv_us": round(kt["gemm_qkv"][0] * 1e3 / kt["gemm_qkv"][1], 2),
                     "gemm_o_us": round(kt["gemm_o"][0] * 1e3 / kt["gemm_o"][1], 2)}
    del src, dst
    torch.cuda.empty_cache()
    res["method"] = ("per-step HIP event pairs, each step queued behind other GPU work: warm after a ~0.2 ms "
                     "spin kernel, cold after a 1 GiB device copy that evicts the weights from the "
                     "memory-side cache")
    return res


def bench_context_kv(steps: int, warmup: int, names=("P3", "P4"), formats=("bf16", "mxfp8")):
    """The multi-layer context K/V precompute on its two workloads: P3 (the
    context rows of one C3 decode round, 3 layers) and P4 (a 4096-row prefill,
    3 layers), with bf16 weights and with MXFP8 weights (entries
    "<name>_mxfp8"). Each run appends every layer's rows and the lengths are
    rewound (host-only) before the next; the time is HIP events on the launch
    stream around `steps` runs."""
    import numpy as np
    import torch

    from block_diffusion_draft_qkv_amd import ContextKV, ContextKVShape, KVCache
    from workload import make_ctxkv_case, make_mxfp8_kv_weights

    res = {}
    for name, fmt in [(n, f) for n in names for f in formats]:
        case = make_ctxkv_case(name, seed=0)
        mx = fmt == "mxfp8"
        c = case.cfg
        dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32

        def dev(x, dtype=dt):
            return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)

        w = case.weights
        shape = ContextKVShape(c.hidden, c.n_layers, c.n_kv_heads, c.head_dim, dt, c.rope_theta, c.rms_eps,
                               c.max_position)
        if mx:
            mw = make_mxfp8_kv_weights(c, 0)
            pre = ContextKV(shape, dev(w.hidden_norm), torch.from_numpy(mw.w_kv_codes.reshape(-1, c.hidden)).cuda(),
                            dev(w.k_norm),
                            w_kv_scale=torch.from_numpy(mw.w_kv_scales.reshape(-1, c.hidden // 32)).cuda())
        else:
            pre = ContextKV(shape, dev(w.hidden_norm), dev(w.w_kv.reshape(-1, c.hidden)), dev(w.k_norm))
        caches = []
        for layer in range(c.n_layers):
            kv = KVCache(case.batch, c.n_kv_heads, c.head_dim, case.capacity(), dt)
            for b in range(case.batch):
                kv.write_prefix(b, dev(case.cache_k[layer][b]), dev(case.cache_v[layer][b]))
            caches.append(kv)
        ctx, pos = dev(case.context_states), dev(case.positions, torch.int32)
        offs = [int(o) for o in case.ctx_offsets]
        ws = pre.workspace(offs[-1])
        L0 = case.cached_len.copy()

        def run():
            pre.append(ctx, offs, pos, caches, workspace=ws)
            for kv in caches:
                kv.set_lengths(L0)

        settle(lambda i: run())
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        if pre.poll_error() != 0:
            raise RuntimeError("context position outside the RoPE table")
        us = e0.elapsed_time(e1) * 1e3 / steps
        rows = offs[-1]
        es = 2 if c.dtype == "bf16" else 4
        fc = None
        if not mx:
            # the optional fc projection before it (three target layers' features)
            from workload import make_fc_inputs
            aux, w_fc = make_fc_inputs(c, rows, seed=0)
            pre.set_fc(dev(w_fc))
            aux_d = dev(aux)
            ctx_fc = torch.empty((rows, c.hidden), dtype=dt, device="cuda")
            for _ in range(warmup):
                pre.combine(aux_d, out=ctx_fc)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                pre.combine(aux_d, out=ctx_fc)
            e1.record()
            torch.cuda.synchronize()
            fc_us = e0.elapsed_time(e1) * 1e3 / steps
            fc_flops = 2.0 * rows * c.hidden * aux.shape[1]
            fc = {"us_per_run": round(fc_us, 2), "fc_in": int(aux.shape[1]),
                  "tflops": round(fc_flops / (fc_us * 1e-6) / 1e12, 1),
                  "floor_us": {"mfma": round(fc_flops / (BF16_PEAK_TFLOPS * 1e12) * 1e6, 2),
                               "hbm": round((w_fc.size + aux.size + rows * c.hidden) * es / (HBM_PEAK_GBS * 1e9) * 1e6,
                                            2)}}
        n_out = c.n_layers * 2 * c.n_kv_heads * c.head_dim
        flops = 2.0 * rows * n_out * c.hidden
        weight_bytes = n_out * c.hidden * es if not mx else n_out * c.hidden * 33 // 32   # codes + scales
        io_bytes = rows * c.hidden * es + rows * n_out * es   # states in, K/V rows out
        peak = FP8_PEAK_TFLOPS if mx else BF16_PEAK_TFLOPS
        res[name + ("_mxfp8" if mx else "")] = {
            "workload": (f"{name}: {case.batch} sequence(s), {rows} context rows, {c.n_layers} layers, "
                         f"H={c.hidden}, {c.n_kv_heads} KV heads, head_dim {c.head_dim}, {c.dtype}"
                         + (", MXFP8 weights and activations" if mx else "")),
            "us_per_run": round(us, 2),
            "context_rows_per_s": round(rows / (us * 1e-6), 1),
            "tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "hbm_gbs": round((weight_bytes + io_bytes) / (us * 1e-6) / 1e9, 1),
            "floor_us": {"mfma": round(flops / (peak * 1e12) * 1e6, 2),
                         "hbm": round((weight_bytes + io_bytes) / (HBM_PEAK_GBS * 1e9) * 1e6, 2)},
        }
        if fc is not None:
            res[name]["fc_combine"] = fc
        pre.close()
        del caches
        torch.cuda.empty_cache()
    return res


def bench_decoder(steps: int, warmup: int, seed: int = 0, copies: int = 3):
    """One draft decoder layer step at C3 (input_layernorm, the attention layer
    step, residual, post_attention_layernorm, SwiGLU MLP of width 12288,
    residual), timed with HIP events on the launch stream over `steps` steps;
    KV-cache copies rotate and lengths are rewound on the host as for the
    layer step."""
    import numpy as np
    import torch

    from block_diffusion_draft_qkv_amd import DFlashDecoder, KVCache, LayerShape
    from workload import QWEN3_8B_INTERMEDIATE, make_case, make_mlp_weights

    case = make_case("C3", seed=seed)
    cfg = case.cfg
    inter = QWEN3_8B_INTERMEDIATE
    mw = make_mlp_weights(case, inter)
    dt = torch.bfloat16

    def dev(x, dtype=dt):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)

    w = case.weights
    dec = DFlashDecoder(LayerShape(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_size, dt,
                                   cfg.rope_theta, cfg.rms_eps, cfg.sliding_window, cfg.max_position), inter,
                        dev(w.w_qkv), dev(w.w_o), dev(w.q_norm), dev(w.k_norm), dev(mw.input_norm),
                        dev(mw.post_norm), dev(mw.w_gate_up), dev(mw.w_down))
    B, bs = case.batch, cfg.block_size
    caches = []
    for i in range(copies):
        c = KVCache(B, cfg.n_kv_heads, cfg.head_dim, case.capacity(), dt)
        if i == 0:
            for b in range(B):
                c.write_prefix(b, dev(case.cache_k[b]), dev(case.cache_v[b]))
        else:
            c.k.copy_(caches[0].k)
            c.v.copy_(caches[0].v)
            c.set_lengths(case.cached_len)
        caches.append(c)
    x, th, pos = dev(case.hidden_states), dev(case.target_hidden), dev(case.positions, torch.int32)
    offs = [int(o) for o in case.ctx_offsets]
    out = torch.empty_like(x)
    ws = dec.workspace(B, offs[-1])
    L0 = case.cached_len.copy()

    def one(i):
        cache = caches[i % copies]
        dec.step(x, th, offs, pos, cache, out=out, workspace=ws)
        cache.set_lengths(L0)

    settle(one)
    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        one(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    if dec.poll_error() != 0:
        raise RuntimeError("position outside the RoPE table")
    us = e0.elapsed_time(e1) * 1e3 / steps
    H, mq = cfg.hidden, B * bs
    mlp_flops = 2.0 * mq * H * 3 * inter
    res = {
        "workload": (f"C3 decoder layer: B={B}, block {bs}, H={H}, {cfg.n_q_heads}/{cfg.n_kv_heads} heads, "
                     f"head_dim {cfg.head_dim}, MLP width {inter}, bf16"),
        "us_per_step": round(us, 2),
        "tokens_per_s": round(mq / (us * 1e-6), 1),
        "mlp_gflop": round(mlp_flops / 1e9, 1),
        "mlp_weight_mb": round(3 * inter * H * 2 / 1e6, 1),
    }
    dec.close()
    del caches
    torch.cuda.empty_cache()
    return res


def bench_other_configs(names, steps: int, warmup: int, seed: int = 0, copies: int = 2):
    """The layer step at the other full-size workloads (C4 long context, C5
    sliding window): wall-clock step time, then the same steps with HIP
    events for the attention kernel against its algorithmic bytes (in-band
    keys only under the window)."""
    import numpy as np
    import torch

    from block_diffusion_draft_qkv_amd import DFlashLayer, KVCache, LayerShape
    from workload import make_case

    res = {}
    for name in names:
        case = make_case(name, seed=seed)
        cfg = case.cfg
        B, bs, H = case.batch, cfg.block_size, cfg.hidden
        nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        es = 2 if cfg.dtype == "bf16" else 4

        def dev(x, dtype=dt):
            return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)

        w = case.weights
        layer = DFlashLayer(LayerShape(H, nq, nkv, d, bs, dt, cfg.rope_theta, cfg.rms_eps, cfg.sliding_window,
                                       cfg.max_position), dev(w.w_qkv), dev(w.w_o), dev(w.q_norm), dev(w.k_norm))
        caches = []
        for i in range(copies):
            c = KVCache(B, nkv, d, case.capacity(), dt)
            if i == 0:
                for b in range(B):
                    c.write_prefix(b, dev(case.cache_k[b]), dev(case.cache_v[b]))
            else:
                c.k.copy_(caches[0].k)
                c.v.copy_(caches[0].v)
                c.set_lengths(case.cached_len)
            caches.append(c)
        hs = dev(case.hidden_states)
        th = dev(case.target_hidden) if case.target_hidden.size else None
        pos = dev(case.positions, torch.int32)
        offs = [int(o) for o in case.ctx_offsets]
        out = torch.empty((B * bs, H), dtype=dt, device="cuda")
        ws = layer.workspace(B, offs[-1])
        L0 = case.cached_len.copy()
        accepted = (case.cached_len + case.new_ctx + case.accept).tolist()

        def one(i):
            c = caches[i % copies]
            layer.step(hs, th, offs, pos, c, out=out, workspace=ws)
            c.crop_all(accepted)
            c.set_lengths(L0)

        settle(one)
        for i in range(warmup):
            one(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            one(warmup + i)
        torch.cuda.synchronize()
        t_step = (time.perf_counter() - t0) / steps
        layer.set_profiling(True)
        for i in range(steps):
            one(i)
        torch.cuda.synchronize()
        kt = layer.kernel_times()
        layer.set_profiling("attn_span")
        for i in range(steps):
            one(i)
        torch.cuda.synchronize()
        span_ms, span_n = layer.kernel_times()["attn_merge"]
        layer.set_profiling(False)
        if layer.poll_error() != 0:
            raise RuntimeError(f"{name}: device-side error")
        T = case.total_len.astype(np.int64)
        keys = np.minimum(T, cfg.sliding_window + bs - 1) if cfg.sliding_window else T
        attn_bytes = int(keys.sum()) * nkv * d * 2 * es + 2 * B * bs * nq * d * es
        ms, n = kt["attn"]
        t_attn = ms * 1e3 / n
        t_merge = kt["merge"][0] * 1e3 / steps
        res[name] = {
            "workload": (f"B={B}, cached ctx {cfg.cached_len}, new ctx {cfg.new_ctx}, block {bs}, "
                         f"window {cfg.sliding_window or 'none'}"),
            "ms_per_step": round(t_step * 1e3, 4),
            "tokens_per_s": round(B * bs / t_step, 1),
            "attn_us": round(t_attn, 2),
            "attn_algorithmic_bytes": attn_bytes,
            "attn_hbm_frac": round(attn_bytes / (t_attn * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "attn_merge_us": round(span_ms * 1e3 / span_n, 2),
            "attn_merge_hbm_frac": round(attn_bytes / (span_ms * 1e-3 / span_n) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_mean_us": {k: round(v[0] * 1e3 / v[1], 2) for k, v in kt.items() if v[1]},
        }
        layer.close()
        del caches
        torch.cuda.empty_cache()
    return res


def bench_mxfp8_layer(steps: int, warmup: int, seed: int = 0, copies: int = 3):
    """The C3 layer step with MXFP8 projections (E4M3 weights with E8M0 block
    scales, activations quantised on the fly): `steps` steps with the crops,
    lengths rewound on the host, on `copies` rotating cache copies; then the
    same steps with per-kernel HIP events (the q|k|v and o_proj figures
    include their activation quantisation)."""
    import numpy as np
    import torch

    from block_diffusion_draft_qkv_amd import DFlashLayer, KVCache, LayerShape
    from workload import make_case, make_mxfp8_layer_weights

    case = make_case("C3", seed=seed)
    cfg = case.cfg
    dt = torch.bfloat16
    B, bs, H = case.batch, cfg.block_size, cfg.hidden

    def dev(x, dtype=dt):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)

    def u8(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    mw = make_mxfp8_layer_weights(cfg, 0)
    layer = DFlashLayer(LayerShape(H, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, bs, dt, cfg.rope_theta,
                                   cfg.rms_eps, cfg.sliding_window, cfg.max_position),
                        u8(mw.w_qkv_codes), u8(mw.w_o_codes), dev(case.weights.q_norm), dev(case.weights.k_norm),
                        w_qkv_scale=u8(mw.w_qkv_scales), w_o_scale=u8(mw.w_o_scales))
    caches = []
    for i in range(copies):
        c = KVCache(B, cfg.n_kv_heads, cfg.head_dim, case.capacity(), dt)
        for b in range(B):
            c.write_prefix(b, dev(case.cache_k[b]), dev(case.cache_v[b]))
        caches.append(c)
    hs, th, pos = dev(case.hidden_states), dev(case.target_hidden), dev(case.positions, torch.int32)
    offs = [int(o) for o in case.ctx_offsets]
    out = torch.empty((B * bs, H), dtype=dt, device="cuda")
    ws = layer.workspace(B, offs[-1])
    L0 = case.cached_len.copy()
    accepted = (case.cached_len + case.new_ctx + case.accept).tolist()

    def one(i):
        c = caches[i % copies]
        layer.step(hs, th, offs, pos, c, out=out, workspace=ws)
        c.crop_all(accepted)
        c.set_lengths(L0)

    settle(one)
    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one(warmup + i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / steps
    layer.set_profiling(True)
    for i in range(steps):
        one(i)
    torch.cuda.synchronize()
    kt = layer.kernel_times()
    layer.set_profiling(False)
    if layer.poll_error() != 0:
        raise RuntimeError("position outside the RoPE table")
    return {
        "workload": "C3 layer step with MXFP8 q|k|v and o_proj (E4M3, E8M0 scale per 32), B=32, block 16",
        "ms_per_step": round(t_step * 1e3, 4),
        "tokens_per_s": round(B * bs / t_step, 1),
        "kernel_mean_us": {k: round(v[0] * 1e3 / v[1], 2) if v[1] else 0.0 for k, v in kt.items()},
    }


def bench_paged(steps: int, warmup: int, seed: int = 0, copies: int = 3):
    """The C3 layer step on the paged cache (64-row blocks handed out in a
    shuffled order): `steps` steps with lengths rewound on the host, HIP
    events on the launch stream, then the attention kernel's mean from a
    profiled pass; and `steps` rounds of the draft-round driver (reserve the
    appended blocks, copy the table, step, crop to the accepted prefix and
    release the dropped blocks), host work included."""
    import numpy as np
    import torch

    from block_diffusion_draft_qkv_amd import DFlashLayer, LayerShape, PagedKVCache, run_round
    from workload import make_case

    case = make_case("C3", seed=seed)
    cfg = case.cfg
    dt = torch.bfloat16
    B, bs, H = case.batch, cfg.block_size, cfg.hidden

    def dev(x, dtype=dt):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)

    w = case.weights
    layer = DFlashLayer(LayerShape(H, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, bs, dt, cfg.rope_theta,
                                   cfg.rms_eps, cfg.sliding_window, cfg.max_position),
                        dev(w.w_qkv), dev(w.w_o), dev(w.q_norm), dev(w.k_norm))
    need = [-(-int(t) // 64) for t in case.total_len]
    caches = []
    for i in range(copies):
        c = PagedKVCache(B, cfg.n_kv_heads, cfg.head_dim, sum(need) + 4 * B, max(need) + 4, dt)
        order = c.free
        np.random.default_rng(seed + i).shuffle(order)
        c.free = order
        for b in range(B):
            c.write_prefix(b, dev(case.cache_k[b]), dev(case.cache_v[b]))
            c.reserve(b, int(case.total_len[b]))
        c.sync()
        caches.append(c)
    hs, th, pos = dev(case.hidden_states), dev(case.target_hidden), dev(case.positions, torch.int32)
    offs = [int(o) for o in case.ctx_offsets]
    out = torch.empty((B * bs, H), dtype=dt, device="cuda")
    ws = layer.workspace(B, offs[-1])
    L0 = case.cached_len.copy()

    def one(i):
        c = caches[i % copies]
        layer.step(hs, th, offs, pos, c, out=out, workspace=ws)
        c.set_lengths(L0)

    settle(one)
    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one(warmup + i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / steps
    layer.set_profiling(True)
    for i in range(steps):
        one(i)
    torch.cuda.synchronize()
    ms, n = layer.kernel_times()["attn"]
    layer.set_profiling(False)
    attn_us = ms * 1e3 / n
    T = case.total_len.astype(np.int64)
    attn_bytes = int(T.sum()) * cfg.n_kv_heads * cfg.head_dim * 2 * 2 + 2 * B * bs * cfg.n_q_heads * cfg.head_dim * 2

    # Driver rounds with simulated accepted counts; after each round the
    # sequences are cropped back to their starting lengths (a rewind, host
    # work included), so every round has C3's lengths and reserves its blocks
    # anew.
    c = caches[0]
    c.crop_all(L0)
    rng = np.random.default_rng(seed + 7)
    accepts = rng.integers(0, bs + 1, size=(steps, B))
    for r in range(min(warmup, steps)):
        run_round(layer, c, hs, th, offs, accepts[r], out=out)
        c.crop_all(L0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(steps):
        run_round(layer, c, hs, th, offs, accepts[r], out=out)
        c.crop_all(L0)
    torch.cuda.synchronize()
    t_round = (time.perf_counter() - t0) / steps
    res = {
        "workload": f"C3 layer step on a paged cache (64-row blocks, shuffled), B={B}, block {bs}",
        "ms_per_step": round(t_step * 1e3, 4),
        "tokens_per_s": round(B * bs / t_step, 1),
        "attn_mean_us": round(attn_us, 2),
        "attn_hbm_frac": round(attn_bytes / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "driver_round_ms": round(t_round * 1e3, 4),
        "driver_tokens_per_s": round(B * bs / t_round, 1),
    }
    layer.close()
    del caches
    torch.cuda.empty_cache()
    return res


def main():
    global SETTLE_S
    a = parse()
    SETTLE_S = a.settle
    if a.gpus != 1:
        print("bench.py measures one GPU only: the multi-GPU path of this layer is a design "
              "(sequence/head sharding) that is not built; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return
    if a.decoder_only:
        print(json.dumps({"decoder_layer": bench_decoder(a.decoder_steps, 5)}), flush=True)
        return
    if a.mxfp8_only:
        print(json.dumps({"mxfp8_layer_step": bench_mxfp8_layer(a.mxfp8_steps, 10)}), flush=True)
        return
    if a.context_kv_only:
        print(json.dumps({"context_kv_precompute": bench_context_kv(a.ctxkv_steps, 5, (a.context_kv_only,))}),
              flush=True)
        return

    import numpy as np
    import torch

    from block_diffusion_draft_qkv_amd import DFlashLayer, KVCache, LayerShape
    from workload import make_case

    case = make_case(a.config, seed=a.seed)
    cfg = case.cfg
    B, bs, H = case.batch, cfg.block_size, cfg.hidden
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    es = 2 if cfg.dtype == "bf16" else 4

    def dev(x, dtype=dt):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)

    w = case.weights
    layer = DFlashLayer(LayerShape(H, nq, nkv, d, bs, dt, cfg.rope_theta, cfg.rms_eps,
                                   cfg.sliding_window, cfg.max_position),
                        dev(w.w_qkv), dev(w.w_o), dev(w.q_norm), dev(w.k_norm))
    layer.set_append_mode(a.append_mode)
    cap = case.capacity()
    caches = []
    for i in range(a.copies):
        c = KVCache(B, nkv, d, cap, dt)
        if i == 0:
            for b in range(B):
                c.write_prefix(b, dev(case.cache_k[b]), dev(case.cache_v[b]))
        else:
            c.k.copy_(caches[0].k)
            c.v.copy_(caches[0].v)
            c.set_lengths(case.cached_len)
        caches.append(c)
    hs = dev(case.hidden_states)
    th = dev(case.target_hidden) if case.target_hidden.size else None
    pos = dev(case.positions, torch.int32)
    offs = [int(o) for o in case.ctx_offsets]
    out = torch.empty((B * bs, H), dtype=dt, device="cuda")
    ws = layer.workspace(B, offs[-1])
    L0 = case.cached_len.copy()
    accepted = (case.cached_len + case.new_ctx + case.accept).tolist()
    torch.cuda.synchronize()

    def one_step(i):
        cache = caches[i % a.copies]
        layer.step(hs, th, offs, pos, cache, out=out, workspace=ws)
        cache.crop_all(accepted)
        cache.set_lengths(L0)  # rewind for the next use of this copy (not part of the step)

    # Clock settle: the GPU raises its clocks only after some milliseconds of
    # sustained load, and the first tens of steps of a cold run (a few ms) run
    # the projections ~20 % slower. Untimed steps for a fixed wall time first,
    # then the W warm-up steps, then the K timed ones.
    settle_steps = settle(one_step, a.settle)
    for i in range(a.warmup):
        one_step(i)
    torch.cuda.synchronize()
    if layer.poll_error() != 0:
        raise RuntimeError("position outside the RoPE table during warm-up")

    # Timed region: K steps with nothing but the steps themselves enqueued.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        one_step(a.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Per-kernel durations: the same K steps again with HIP events recorded
    # around every launch on the launch stream (kept out of the timed region).
    layer.set_profiling(True)
    for i in range(a.steps):
        one_step(a.warmup + a.steps + i)
    torch.cuda.synchronize()
    kt = layer.kernel_times()
    # The attention and its merge as one span: a single event pair on the
    # launch stream, none between the two kernels (every event packet adds its
    # own time, so the per-kernel pairs above overstate the span).
    layer.set_profiling("attn_span")
    for i in range(a.steps):
        one_step(a.warmup + 2 * a.steps + i)
    torch.cuda.synchronize()
    span_ms, span_n = layer.kernel_times()["attn_merge"]
    layer.set_profiling(False)
    weights = cold_weight_steps(one_step, layer, min(a.steps, 50), a.warmup + 3 * a.steps)

    ms_per_step = elapsed * 1e3 / a.steps
    tokens_per_s = B * bs / (elapsed / a.steps)

    # Algorithmic bytes and flops of one step.
    T = case.total_len.astype(np.int64)
    keys = np.minimum(T, cfg.sliding_window + bs - 1) if cfg.sliding_window else T
    attn_bytes = int(keys.sum()) * nkv * d * 2 * es + 2 * B * bs * nq * d * es
    mc = int(offs[-1])
    proj_flops = 2 * H * (B * bs * (nq + 2 * nkv) * d + mc * 2 * nkv * d + B * bs * nq * d)

    def mean_us(name):
        ms, n = kt[name]
        return ms * 1e3 / n if n else 0.0

    t_attn = mean_us("attn")
    # the merge runs only when some pair was split; its mean is per step
    t_merge = kt["merge"][0] * 1e3 / a.steps
    t_span = span_ms * 1e3 / span_n
    t_proj = mean_us("gemm_qkv") + mean_us("gemm_o")
    achieved = attn_bytes / (t_span * 1e-6) / 1e9
    traffic = traffic_per_launch(f"{cfg.name}: ") if a.seed == 0 else None

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: one draft-attention layer step + crop, B={B}, cached ctx "
                         f"{cfg.cached_len}, new ctx {cfg.new_ctx}, block {bs}, H={H}, "
                         f"{nq}/{nkv} heads, head_dim {d}, window {cfg.sliding_window or 'none'}"),
            "batch": B, "block_size": bs, "total_keys": int(T.sum()), "new_ctx_rows": mc,
            "seed": a.seed, "kv_cache_copies": a.copies, "append_mode": a.append_mode,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": f"attn_splitkv_kernel<{cfg.dtype},{d}> + attn_merge_kernel",
            "algorithmic_bytes_per_launch": attn_bytes,
            "mean_launch_us": round(t_span, 2),
            "timing": "one HIP event pair on the launch stream around the attention and its merge",
            "attention_us": round(t_attn, 2),
            "merge_us": round(t_merge, 2),
            "per_kernel_events_sum_us": round(t_attn + t_merge, 2),
        },
        "attention_kernel_alone": {
            "achieved_gbs": round(attn_bytes / (t_attn * 1e-6) / 1e9, 1),
            "frac": round(attn_bytes / (t_attn * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "clock_settle": {"seconds": a.settle, "steps": settle_steps},
        "projections": {
            "bound": "mfma", "flops_per_step": proj_flops,
            "achieved_tflops": round(proj_flops / (t_proj * 1e-6) / 1e12, 1) if t_proj else None,
            "peak_tflops": BF16_PEAK_TFLOPS,
            "counters": mfma_counters(f"{cfg.name}: ") if a.seed == 0 else None,
        },
        "kernel_mean_us": {k: round(mean_us(k), 2) for k in kt if k != "attn_merge"},
        "kernel_sum_us_per_step": round(sum(v[0] for v in kt.values()) * 1e3 / a.steps, 2),
        "projection_weights_from_hbm": weights,
    }
    if a.cpu_sample > 0:
        line["cpu_baseline"] = cpu_baseline(case, a.cpu_sample)
    layer.close()
    del caches
    torch.cuda.empty_cache()
    if a.ctxkv_steps > 0:
        line["context_kv_precompute"] = bench_context_kv(a.ctxkv_steps, 5)
    if a.decoder_steps > 0:
        line["decoder_layer"] = bench_decoder(a.decoder_steps, 5)
    if a.paged_steps > 0:
        line["paged"] = bench_paged(a.paged_steps, 10)
    if a.mxfp8_steps > 0:
        line["mxfp8_layer_step"] = bench_mxfp8_layer(a.mxfp8_steps, 10)
    if a.other_steps > 0:
        line["other_configs"] = bench_other_configs(("C4", "C5"), a.other_steps, 5)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
