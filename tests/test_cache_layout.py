"""The contiguous KV cache's memory layout as the kernels address it (no GPU).

The kernels take element (sequence b, head j, row t, dim e) of K at
((b * (cap/64) + t // 64) * nkv + j) * 64 * d + (t % 64) * d + e and of V at
((b * (cap/64) + t // 64) * nkv + j) * d * 64 + e * 64 + t % 64. The binding
writes and reads CPU tensors here, and every element is checked at that
offset of the flat storage: the binding, the header's layout and the
kernels' address arithmetic must agree."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_qkv_amd import KVCache


@pytest.mark.parametrize("lens", [(0, 5), (64, 130), (191, 192)])
def test_prefix_lands_at_the_block_major_offsets(lens):
    B, nkv, d, cap = 2, 3, 8, 192
    rng = np.random.default_rng(sum(lens))
    c = KVCache(B, nkv, d, cap, torch.float32, device="cpu")
    c.k.fill_(float("nan"))
    c.v.fill_(float("nan"))
    data = []
    for b, L in enumerate(lens):
        k = torch.from_numpy(rng.standard_normal((nkv, L, d)).astype(np.float32))
        v = torch.from_numpy(rng.standard_normal((nkv, L, d)).astype(np.float32))
        c.write_prefix(b, k, v)
        data.append((k, v))
    assert c.lengths.tolist() == list(lens)
    fk, fv = c.k.reshape(-1).numpy(), c.v.reshape(-1).numpy()
    written_k = np.zeros(fk.size, dtype=bool)
    written_v = np.zeros(fv.size, dtype=bool)
    nb = cap // 64
    for b, (k, v) in enumerate(data):
        for j in range(nkv):
            for t in range(k.shape[1]):
                blk = (b * nb + t // 64) * nkv + j
                ko = blk * 64 * d + (t % 64) * d
                np.testing.assert_array_equal(fk[ko:ko + d], k[j, t].numpy())
                written_k[ko:ko + d] = True
                vo = blk * d * 64 + np.arange(d) * 64 + t % 64
                np.testing.assert_array_equal(fv[vo], v[j, t].numpy())
                written_v[vo] = True
        rk, rv = c.read(b)
        assert torch.equal(rk, k) and torch.equal(rv, v)
        assert torch.equal(c.k_rows()[b, :, :k.shape[1]], k)
        assert torch.equal(c.vt_rows()[b, :, :, :k.shape[1]], v.transpose(1, 2))
    assert np.isnan(fk[~written_k]).all() and np.isnan(fv[~written_v]).all()


def test_capacity_must_be_whole_blocks():
    for cap in (0, 100, -64):
        with pytest.raises(ValueError):
            KVCache(1, 1, 8, cap, torch.float32, device="cpu")
    c = KVCache(1, 1, 8, 64, torch.float32, device="cpu")
    with pytest.raises(ValueError):
        c.write_prefix(0, torch.zeros(1, 65, 8), torch.zeros(1, 65, 8))
