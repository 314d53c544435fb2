"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (same library, same step call), against the float64 oracle
run over every output and every appended cache row.

C1 tiny fp32 | C2 single bf16 | C3 ragged B=32 | C4 long 32K | C5 window 4096,
each in the default append mode and, where that mode picks a path by size,
also in the other one.
After the step each sequence is cropped to its accepted prefix and the
lengths and surviving rows are checked bit-exactly.
"""
import numpy as np
import pytest
import torch

from harness import (assert_close, cache_bits, check_cache_after_step, make_cache, make_layer, raw_bits,
                     run_oracle, step_inputs, to64)
from workload import make_case

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


# Each workload in the default append mode, plus the other path where the
# default picks one by size: C2 and C4 (few rows, deep k) append in the
# separate kernel by default, C3 in the projection's epilogue.
FULL_CASES = [("C1", "auto"), ("C2", "auto"), ("C3", "auto"), ("C4", "auto"), ("C5", "auto"),
              ("C2", "fused"), ("C4", "fused"), ("C3", "separate")]


@pytest.mark.parametrize("name,mode", FULL_CASES)
def test_full_config_step_and_crop(name, mode):
    case = make_case(name, seed=0)
    print(f"[{name} {mode}] batch {case.batch}, keys {int(case.total_len.sum())}", flush=True)
    layer = make_layer(case)
    layer.set_append_mode(mode)
    cache = make_cache(case)
    bk, bv = cache_bits(cache)
    hs, th, pos = step_inputs(case)
    out = layer.step(hs, th, case.ctx_offsets, pos, cache)
    torch.cuda.synchronize()
    assert layer.poll_error() == 0
    ref, new = run_oracle(case)
    max_abs, rel = assert_close(to64(out), ref, case.cfg.dtype, f"{name} out")
    print(f"[{name} {mode}] out max abs {max_abs:.3e} rel-RMS {rel:.3e}", flush=True)
    check_cache_after_step(case, cache, bk, bv, new)

    # crop to the accepted prefix: lengths exact, rows below untouched
    k_after, v_after = raw_bits(cache.k), raw_bits(cache.v)
    accepted = case.cached_len + case.new_ctx + case.accept
    for b in range(case.batch):
        cache.crop(b, int(accepted[b]))
    assert cache.lengths.tolist() == accepted.tolist()
    np.testing.assert_array_equal(raw_bits(cache.k), k_after)
    np.testing.assert_array_equal(raw_bits(cache.v), v_after)
    layer.close()
