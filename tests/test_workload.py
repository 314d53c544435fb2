"""The seeded input generator: determinism, shapes and bf16 rounding."""
import numpy as np
import pytest

from workload import CONFIGS, make_case, round_bf16


def test_round_bf16_matches_torch_round_to_nearest_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3e38, -3e38, 1e-40])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_bf16(x).view(np.uint32), ref.view(np.uint32))


def test_case_is_deterministic_and_shaped():
    a = make_case("C1", seed=3)
    b = make_case("C1", seed=3)
    np.testing.assert_array_equal(a.hidden_states, b.hidden_states)
    np.testing.assert_array_equal(a.weights.w_q, b.weights.w_q)
    cfg = CONFIGS["C1"]
    assert a.hidden_states.shape == (cfg.batch * cfg.block_size, cfg.hidden)
    assert a.target_hidden.shape == (128, cfg.hidden)
    assert a.positions.tolist() == list(range(0, 136))
    c = make_case("C1", seed=4)
    assert not np.array_equal(a.hidden_states, c.hidden_states)


def test_ragged_case_ranges():
    cfg = CONFIGS["C3"].replace(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64)
    c = make_case(cfg, seed=0, cached_len=(512, 8192))
    assert c.batch == 32
    assert np.all((c.cached_len >= 512) & (c.cached_len <= 8192))
    assert np.all((c.new_ctx >= 1) & (c.new_ctx <= 16))
    assert np.all((c.accept >= 0) & (c.accept <= 16))
    assert c.capacity() % 64 == 0 and c.capacity() >= c.total_len.max()
    off = 0
    for b in range(c.batch):
        n = int(c.new_ctx[b]) + cfg.block_size
        assert c.positions[off:off + n].tolist() == list(range(c.cached_len[b], c.cached_len[b] + n))
        off += n
    w = c.weights
    assert np.all(round_bf16(w.w_q) == w.w_q)
