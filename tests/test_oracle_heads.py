"""Pins of the head-repack oracle (oracle/heads.py) against the exchange it
stands for (the paper's Section 3.2 / Algorithm 2, as an index map over p
workers' blocks, with blocks of unequal size), brute force on small arrays,
and the property GP-A2A rests on: attention heads are computed
independently."""
import numpy as np
import pytest

from graph_transformer_sparse_amd import inputs as I
from oracle import heads as Hd
from oracle import oracle as O


def _x(rows, heads, dh, seed=0):
    return np.random.default_rng(seed).standard_normal((rows, heads, dh))


@pytest.mark.parametrize("parts", [1, 2, 4, 8])
def test_split_brute_force(parts):
    x = _x(5, 8, 3)
    s = Hd.head_split(x, parts)
    hp = 8 // parts
    assert s.shape == (parts, 5, hp, 3)
    for r in range(parts):
        for i in range(5):
            for hh in range(hp):
                for k in range(3):
                    assert s[r, i, hh, k] == x[i, r * hp + hh, k]


@pytest.mark.parametrize("parts", [1, 2, 4, 8])
def test_split_equals_the_exchange(parts):
    n_per = 6
    x = _x(parts * n_per, 8, 4, seed=parts)
    blocks = [x[k * n_per:(k + 1) * n_per] for k in range(parts)]
    got = Hd.all_to_all_node_to_head(blocks)
    s = Hd.head_split(x, parts)
    for r in range(parts):
        assert np.array_equal(got[r], s[r])
    # and back: the return exchange of the slices gives every worker its block
    back = Hd.all_to_all_head_to_node([s[r] for r in range(parts)], [n_per] * parts)
    for k in range(parts):
        assert np.array_equal(back[k], blocks[k])
    assert np.array_equal(np.concatenate(back, axis=0), Hd.head_merge(s))


def test_exchange_with_unequal_blocks():
    """Workers holding different numbers of nodes (one holding none): the
    head-partitioned tensors are still head_split of the concatenated nodes,
    and the reverse exchange gives every worker its own block back."""
    counts = [3, 0, 5, 2]
    x = _x(sum(counts), 8, 2, seed=9)
    starts = np.concatenate([[0], np.cumsum(counts)])
    blocks = [x[starts[k]:starts[k + 1]] for k in range(4)]
    got = Hd.all_to_all_node_to_head(blocks)
    s = Hd.head_split(x, 4)
    for r in range(4):
        assert np.array_equal(got[r], s[r])
    back = Hd.all_to_all_head_to_node(got, counts)
    for k in range(4):
        assert np.array_equal(back[k], blocks[k])


def test_round_trip_identity_and_per_head():
    x = _x(7, 4, 2, seed=3)
    assert np.array_equal(Hd.head_merge(Hd.head_split(x, 2)), x)
    assert np.array_equal(Hd.head_split(x, 1)[0], x)
    per = Hd.head_split(x, 4)
    for h in range(4):
        assert np.array_equal(per[h][:, 0], x[:, h])
    b = np.arange(12, dtype=np.float32).reshape(6, 2)     # [E, heads] per-edge bias
    assert np.array_equal(Hd.head_split(b, 2)[1], b[:, 1:2])


def test_heads_attend_independently():
    """Attention on each head slice over the whole graph equals the same
    heads of the attention on all heads (forward and backward)."""
    H, dh, n = 4, 8, 60
    ip, ix = I.random_graph(5, n, n, np.random.default_rng(1).integers(0, 9, n))
    rng = np.random.default_rng(2)
    Q, K, V, dY = (rng.standard_normal((n, H, dh)) for _ in range(4))
    B = rng.standard_normal((ix.size, H))
    Y, lse = O.fwd(ip, ix, n, Q, K, V, B)
    dQ, dK, dV, dB = O.bwd(ip, ix, n, Q, K, V, dY, B)
    parts = 2
    sl = lambda t: Hd.head_split(t, parts)
    q, k, v, dy, b = sl(Q), sl(K), sl(V), sl(dY), sl(B)
    outs = [O.fwd(ip, ix, n, q[r], k[r], v[r], b[r]) for r in range(parts)]
    grads = [O.bwd(ip, ix, n, q[r], k[r], v[r], dy[r], b[r]) for r in range(parts)]
    np.testing.assert_allclose(Hd.head_merge(np.stack([o[0] for o in outs])), Y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Hd.head_merge(np.stack([o[1] for o in outs])), lse, rtol=1e-12, atol=1e-12)
    for i, ref in enumerate((dQ, dK, dV, dB)):
        got = Hd.head_merge(np.stack([gr[i] for gr in grads]))
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
