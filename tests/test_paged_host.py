"""Host logic of the paged KV cache (no GPU): the block allocator, the
scatter of a prefix into 64-row blocks and its gather back, and the blocks
a crop releases. Runs on CPU tensors."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_qkv_amd import DFlashError, PagedKVCache


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


def test_batched_reserve_and_crop_match_the_per_sequence_calls():
    """reserve_all / crop_all (one C call for every crop) leave the same table,
    free list and lengths as the per-sequence reserve / crop, round after round."""
    import numpy as np
    rng = np.random.default_rng(3)
    B = 6
    a = PagedKVCache(B, 2, 16, 200, 12, torch.float32, device="cpu")
    b = PagedKVCache(B, 2, 16, 200, 12, torch.float32, device="cpu")
    order = list(range(200))
    rng.shuffle(order)
    a.free, b.free = list(order), list(order)
    lens = rng.integers(0, 300, B)
    a.set_lengths(lens)
    b.set_lengths(lens)
    for _ in range(25):
        grow = a.lengths.astype(np.int64) + rng.integers(0, 90, B)
        for s in range(B):
            a.reserve(s, int(grow[s]))
        b.reserve_all(grow)
        assert np.array_equal(a.table_host, b.table_host) and a.free == b.free
        a.set_lengths(grow)
        b.set_lengths(grow)
        new = (grow * rng.uniform(0.2, 1.0, B)).astype(np.int64)
        for s in range(B):
            a.crop(s, int(new[s]))
        b.crop_all(new)
        assert np.array_equal(a.table_host, b.table_host) and a.free == b.free
        assert a.lengths.tolist() == b.lengths.tolist() == new.tolist()
    # a crop that would grow one sequence changes nothing
    bad = b.lengths.astype(np.int64).copy()
    bad[2] += 1
    before = (b.table_host.copy(), list(b.free), b.lengths.copy())
    with pytest.raises(DFlashError):
        b.crop_all(bad)
    assert np.array_equal(b.table_host, before[0]) and b.free == before[1]
    assert b.lengths.tolist() == before[2].tolist()
