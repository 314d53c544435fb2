"""Host logic of the paged KV cache (no GPU): the block allocator, the
scatter of a prefix into 64-row blocks and its gather back, and the blocks
a crop releases. Runs on CPU tensors."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_qkv_amd import PagedKVCache


def test_prefix_scatter_gather_roundtrip_and_block_accounting():
    rng = np.random.default_rng(0)
    c = PagedKVCache(batch=3, n_kv_heads=2, head_dim=8, num_blocks=12, max_blocks=5, dtype=torch.float32,
                     device="cpu")
    lens = [130, 0, 64]
    data = {}
    for b, L in enumerate(lens):
        k = torch.from_numpy(rng.standard_normal((2, L, 8)).astype(np.float32))
        v = torch.from_numpy(rng.standard_normal((2, L, 8)).astype(np.float32))
        c.write_prefix(b, k, v)
        data[b] = (k, v)
    assert c.lengths.tolist() == lens
    assert [c.blocks_of(b) for b in range(3)] == [3, 0, 1]
    assert len(c.free) == 12 - 4
    used = c.table_host[c.table_host >= 0]
    assert len(set(used.tolist())) == len(used)          # no block given twice
    assert torch.equal(c.table, torch.from_numpy(c.table_host))  # device copy in sync
    for b in range(3):
        k, v = c.read(b)
        assert torch.equal(k, data[b][0]) and torch.equal(v, data[b][1])
    # a physical block holds 64 consecutive rows of one sequence, V transposed
    blk = int(c.table_host[0, 1])
    assert torch.equal(c.k[blk, :, 5, :], data[0][0][:, 64 + 5, :])
    assert torch.equal(c.v[blk, :, :, 5], data[0][1][:, 64 + 5, :])


def test_reserve_release_and_limits():
    c = PagedKVCache(batch=2, n_kv_heads=1, head_dim=4, num_blocks=4, max_blocks=3, dtype=torch.float32,
                     device="cpu")
    c.reserve(0, 129)                # 3 blocks
    assert c.blocks_of(0) == 3 and len(c.free) == 1
    with pytest.raises(ValueError):
        c.reserve(1, 3 * 64 + 1)     # more than max_blocks
    c.reserve(1, 10)
    with pytest.raises(MemoryError):
        c.reserve(1, 100)            # pool exhausted
    c.release(0, 64)                 # keep one block
    assert c.blocks_of(0) == 1 and len(c.free) == 2
    c.release(0, 0)
    assert c.blocks_of(0) == 0 and len(c.free) == 3
    c.sync()
    assert torch.equal(c.table, torch.from_numpy(c.table_host))
