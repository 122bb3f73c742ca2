"""The seeded input generators: deterministic, well-formed CSR, and the
degree statistics the named workloads are meant to have."""
import numpy as np
import pytest

from graph_transformer_sparse_amd import inputs as I


def _well_formed(ip, ix, R, M, self_loops=True):
    assert ip.dtype == np.int32 and ix.dtype == np.int32
    assert ip.size == R + 1 and ip[0] == 0 and ip[-1] == ix.size
    assert np.all(np.diff(ip) >= 0)
    assert ix.min() >= 0 and ix.max() < M
    rows = np.repeat(np.arange(R), np.diff(ip))
    # strictly ascending columns inside each row
    same = rows[1:] == rows[:-1]
    assert np.all(ix[1:][same] > ix[:-1][same])
    if self_loops:
        key = rows.astype(np.int64) * M + ix
        loops = np.arange(min(R, M), dtype=np.int64)
        assert np.isin(loops * M + loops, key).all()


def test_tiny_graph():
    cfg = I.CONFIGS["tiny"]
    ip, ix = I.graph_for(cfg)
    _well_formed(ip, ix, cfg.n_rows, cfg.n_cols)
    deg = np.diff(ip)
    assert 8.5 < ix.size / cfg.n_rows < 9.5        # mean out-degree 8 plus the self-loop
    assert deg.min() >= 1 and deg.max() < 30
    ip2, ix2 = I.graph_for(cfg)
    np.testing.assert_array_equal(ip, ip2)
    np.testing.assert_array_equal(ix, ix2)


def test_mid_graph():
    cfg = I.CONFIGS["mid"]
    ip, ix = I.graph_for(cfg)
    _well_formed(ip, ix, cfg.n_rows, cfg.n_cols)
    deg = np.diff(ip)
    assert 13 < ix.size / cfg.n_rows < 15.5
    assert 4000 < deg.max() < 20000                 # R-MAT skew
    assert 0.25 < deg[deg > 256].sum() / ix.size < 0.45


def test_features_and_bias():
    x = I.features(3, I.S_Q, 100, 4, 32, "bf16")
    y = I.features(3, I.S_Q, 100, 4, 32, "bf16")
    np.testing.assert_array_equal(x, y)
    assert x.dtype == np.float32 and x.shape == (100, 4, 32)
    # bf16 values: low 16 bits of every float32 are zero
    assert not np.any(x.view(np.uint32) & 0xFFFF)
    f = I.features(3, I.S_Q, 100, 4, 32, "f32")
    # rounding to nearest bf16 is within half an ulp (2^-8 relative)
    assert np.all(np.abs(f - x) <= np.abs(f) * 2.0 ** -8 + 1e-30)
    b = I.edge_bias(3, 200000, 4)
    assert abs(b.var() - 0.5) < 0.01 and abs(b.mean()) < 0.01


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -(1.0 + 2.0 ** -8)], np.float32)
    got = I.to_bf16_values(vals)
    # ties go to the even mantissa; below-half rounds down
    np.testing.assert_array_equal(got, np.array([1.0, 1.0 + 2.0 ** -6, 1.0, -1.0], np.float32))
    import torch
    t = torch.tensor(np.random.default_rng(0).standard_normal(10000, dtype=np.float32))
    np.testing.assert_array_equal(I.to_bf16_values(t.numpy()), t.to(torch.bfloat16).float().numpy())


def test_random_graph_degrees():
    degs = [0, 1, 2, 63, 64, 65, 5]
    ip, ix = I.random_graph(1, len(degs), 100, degs)
    np.testing.assert_array_equal(np.diff(ip), degs)
    _well_formed(ip, ix, len(degs), 100, self_loops=False)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["large", "shard"])
def test_big_graphs(name):
    cfg = I.CONFIGS[name]
    ip, ix = I.graph_for(cfg)
    _well_formed(ip, ix, cfg.n_rows, cfg.n_cols)
