"""A layer step captured into a HIP graph (torch.cuda.CUDAGraph on the launch
stream) replays bit-identically to the eager step. The step enqueues only
kernels: no allocation (the workspace is the caller's, or the library's
static scratch for the no-allocation entry point), no memset, no
synchronisation. Lengths and the attention's split plan are baked into the
kernel arguments at capture, so a replay repeats the captured step exactly:
the test restores the cache between replays (eager copies and a
synchronisation between them) and checks every replay. Contiguous and paged
caches, with the workspace and the no-allocation entry points."""
import pytest
import torch

from harness import make_cache, make_layer, step_inputs
from test_gpu_parity import small
from workload import make_case

pytestmark = pytest.mark.gpu

REPLAYS = 3


def snapshot(cache):
    tabs = (cache.table.clone(),) if hasattr(cache, "table") else ()
    return cache.k.clone(), cache.v.clone(), cache.lengths.copy(), tabs


def restore(cache, snap):
    k, v, lens, _ = snap
    cache.k.copy_(k)
    cache.v.copy_(v)
    cache.lengths[:] = lens


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_captured_step_replays_bit_identically(layout, entry):
    case = make_case(small(config_id=51), seed=9)
    layer = make_layer(case)
    if layout == "paged":
        from test_gpu_paged import make_paged
        cache = make_paged(case, seed=2)
        for b in range(case.batch):
            cache.reserve(b, int(case.total_len[b]))
        cache.sync()
    else:
        cache = make_cache(case)
    hs, th, pos = step_inputs(case)
    B, Mc = case.batch, int(case.ctx_offsets[-1])
    ws = layer.workspace(B, Mc)
    out = torch.empty((B * case.cfg.block_size, case.cfg.hidden), dtype=hs.dtype, device="cuda")

    def step():
        if entry == "noalloc":
            layer.step_noalloc(hs, th, case.ctx_offsets, pos, cache, out)
        else:
            layer.step(hs, th, case.ctx_offsets, pos, cache, out=out, workspace=ws)

    snap = snapshot(cache)
    step()                                     # eager reference
    torch.cuda.synchronize()
    ref_out, ref_k, ref_v, ref_len = out.clone(), cache.k.clone(), cache.v.clone(), cache.lengths.copy()

    restore(cache, snap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()                                 # captured, not run
    assert cache.lengths.tolist() == ref_len.tolist()  # the host side ran once at capture
    for r in range(REPLAYS):
        restore(cache, snap)                   # eager work between replays
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), ref_out.view(torch.uint8)), f"replay {r}: output"
        # bit patterns: the dead rows hold a NaN canary
        assert torch.equal(cache.k.view(torch.uint8), ref_k.view(torch.uint8)), f"replay {r}: cache K"
        assert torch.equal(cache.v.view(torch.uint8), ref_v.view(torch.uint8)), f"replay {r}: cache V"
    assert layer.poll_error() == 0
