"""Pins of the layer oracle (oracle/layer.py): the dense projections around
sparse graph attention (Scalable and Adaptive Parallel Training of Graph
Transformer on Large Graphs, Section 2.1, Eq. 3-5) and their gradients.

* PyTorch float64 autograd of the dense masked layer (linear maps, SDPA with
  the adjacency as a mask, residual) -- a path independent of the oracle;
* central finite differences of <Z, dZ>;
* identity / zero weights reduce the layer to bare attention.
"""
import numpy as np
import pytest
import torch

from graph_transformer_sparse_amd import inputs as I
from oracle import layer as L
from oracle import oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _problem(seed, n, H, dh, bias):
    degs = np.random.default_rng(seed).integers(1, 12, n)
    ip, ix = I.random_graph(400 + seed, n, n, degs)
    X, W, dZ = I.layer_inputs(500 + seed, n, H * dh, "f32")
    b = I.edge_bias(600 + seed, ix.size, H) if bias else None
    return ip, ix, X, W, dZ, b


def _close(a, b, tol):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert np.max(np.abs(a - b)) <= tol * max(1.0, np.max(np.abs(b))), np.max(np.abs(a - b))


@pytest.mark.parametrize("bias", [False, True])
def test_layer_against_torch_autograd(bias):
    n, H, dh = 30, 2, 8
    ip, ix, X, W, dZ, b = _problem(1 + bias, n, H, dh, bias)
    d = H * dh
    f = L.layer_fwd(ip, ix, X, W, H, b)
    g = L.layer_bwd(ip, ix, X, W, H, dZ, b)
    t = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    x, wq, wk, wv, wo = t(X), t(W["q"]), t(W["k"]), t(W["v"]), t(W["o"])
    rows = np.repeat(np.arange(n), np.diff(ip))
    mask = torch.full((H, n, n), float("-inf"), dtype=torch.float64)
    mask[:, rows, ix] = 0.0
    if b is not None:
        mask[:, rows, ix] = torch.tensor(b.T, dtype=torch.float64)
    heads = lambda m: m.reshape(n, H, dh).permute(1, 0, 2)
    q, k, v = heads(x @ wq), heads(x @ wk), heads(x @ wv)
    y = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=dh ** -0.5)
    z = x @ wo + y.permute(1, 0, 2).reshape(n, d)
    (z * torch.tensor(dZ, dtype=torch.float64)).sum().backward()
    _close(f["Z"], z.detach().numpy(), 1e-12)
    _close(g["dX"], x.grad.numpy(), 1e-11)
    for key, w in (("dWq", wq), ("dWk", wk), ("dWv", wv), ("dWo", wo)):
        _close(g[key], w.grad.numpy(), 1e-11)


def test_layer_finite_differences():
    n, H, dh = 12, 2, 4
    ip, ix, X, W, dZ, _ = _problem(3, n, H, dh, False)
    X, dZ = X.astype(np.float64), dZ.astype(np.float64)
    W = {k: v.astype(np.float64) for k, v in W.items()}
    g = L.layer_bwd(ip, ix, X, W, H, dZ)
    loss = lambda X_, W_: float((L.layer_fwd(ip, ix, X_, W_, H)["Z"] * dZ).sum())
    rng = np.random.default_rng(4)
    h = 1e-5
    for _ in range(10):
        i, j = int(rng.integers(n)), int(rng.integers(H * dh))
        Xp, Xm = X.copy(), X.copy()
        Xp[i, j] += h
        Xm[i, j] -= h
        fd = (loss(Xp, W) - loss(Xm, W)) / (2 * h)
        assert abs(fd - g["dX"][i, j]) <= 1e-7 * max(1, abs(fd))
        for key in "qkvo":
            a, c = int(rng.integers(H * dh)), int(rng.integers(H * dh))
            Wp = {k: v.copy() for k, v in W.items()}
            Wm = {k: v.copy() for k, v in W.items()}
            Wp[key][a, c] += h
            Wm[key][a, c] -= h
            fd = (loss(X, Wp) - loss(X, Wm)) / (2 * h)
            assert abs(fd - g["dW" + key][a, c]) <= 1e-7 * max(1, abs(fd)), (key, fd)


def test_identity_and_zero_weights():
    """W_q = W_k = W_v = I and W_o = 0: Q = K = V = X and Z = attention(X)."""
    n, H, dh = 25, 2, 8
    ip, ix, X, W, dZ, _ = _problem(5, n, H, dh, False)
    d = H * dh
    I_ = np.eye(d)
    W = {"q": I_, "k": I_, "v": I_, "o": np.zeros((d, d))}
    f = L.layer_fwd(ip, ix, X, W, H)
    Y, _ = O.fwd(ip, ix, n, X.reshape(n, H, dh), X.reshape(n, H, dh), X.reshape(n, H, dh))
    np.testing.assert_array_equal(f["Q"], X.astype(np.float64))
    np.testing.assert_array_equal(f["Z"], Y.reshape(n, d))


def test_bf16_rounding_matches_torch():
    """The oracle's own bf16 rounding agrees with torch's float32 -> bfloat16
    conversion (round to nearest even), including exact ties."""
    x = np.random.default_rng(9).standard_normal(100000) * 10.0 ** np.random.default_rng(10).integers(-8, 8, 100000)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2.0 ** -130])
    for a in (x, ties):
        t = torch.tensor(a.astype(np.float32)).to(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(L.round_bf16(a), t)


def test_store_none_is_unrounded():
    n, H, dh = 20, 2, 8
    ip, ix, X, W, dZ, _ = _problem(7, n, H, dh, False)
    a = L.layer_fwd(ip, ix, X, W, H)
    b = L.layer_fwd(ip, ix, X, W, H, store=None)
    np.testing.assert_array_equal(a["Z"], b["Z"])
    c = L.layer_fwd(ip, ix, X, W, H, store="bf16")
    np.testing.assert_array_equal(c["Q"], L.round_bf16(a["Q"]))
    assert np.max(np.abs(c["Z"] - a["Z"])) < 0.05 * np.max(np.abs(a["Z"]))
