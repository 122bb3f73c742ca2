"""Parity of the MFMA projection kernels (include/gt_proj.h) and of a whole
sparse graph attention layer with the fp64 layer oracle (oracle/layer.py;
the paper's Section 2.1, Eq. 3-5).

Tolerance as for attention (gpu_util): per tensor relative L2 <= rtol and
elementwise rtol*|r| + rtol*rms(r) + 8u*mag, mag = the sum of the absolute
values of each output's terms (|A| |B| for a product A B).  Weight
gradients are float32 for either input dtype and sum exact products of the
inputs, so they are held to the float32 bound (1e-5) in both cases.  bf16
outputs are also pinned to round-to-nearest-even where the float32 result
decides the rounding.
"""
import numpy as np
import pytest
import torch

from graph_transformer_sparse_amd import gtattn as T
from graph_transformer_sparse_amd import inputs as I
from oracle import layer as L
from oracle import oracle as O

from gpu_util import RTOL, TDT, assert_close, assert_rounded_to_nearest_even, dev, to_np

pytestmark = pytest.mark.gpu


def _abs(x):
    return np.abs(np.asarray(x, np.float64))


CASES = [(n, d, dt) for dt in ("f32", "bf16") for n, d in
         ((1, 64), (1, 128), (1, 256), (33, 256), (100, 128), (128, 256), (257, 128),
          (1000, 64), (4097, 128), (20000, 256), (70001, 128), (50003, 256))]


@pytest.mark.parametrize("case", CASES, ids=[f"n{n}-d{d}-{dt}" for n, d, dt in CASES])
def test_projection_kernels(case):
    n, d, dt = case
    print(f"proj n={n} d={d} {dt}", flush=True)
    X, W, dZ = I.layer_inputs(700 + n % 97, n, d, dt)
    G = [I.layer_inputs(800 + k, n, d, dt)[2] for k in range(3)]    # stand-in dQ, dK, dV
    Y = I.layer_inputs(900, n, d, dt)[2]
    t = lambda a: dev(a, TDT[dt])
    Xd, Wd = t(X), {k: t(v) for k, v in W.items()}
    rt = RTOL[dt]
    Q, K, V = T.gt_proj_qkv(Xd, Wd["q"], Wd["k"], Wd["v"])
    rq = L.proj_qkv(X, W["q"], W["k"], W["v"])
    for got, ref, k in zip((Q, K, V), rq, "qkv"):
        assert_close(got, ref, rt, "XW" + k, _abs(X) @ _abs(W[k]))
    Z = T.gt_proj_out(Xd, Wd["o"], t(Y))
    assert_close(Z, L.proj_out(X, W["o"], Y), rt, "Z", _abs(X) @ _abs(W["o"]) + _abs(Y))
    dX = T.gt_proj_bwd_data(t(dZ), t(G[0]), t(G[1]), t(G[2]), Wd["o"], Wd["q"], Wd["k"], Wd["v"])
    rdx = L.proj_bwd_data(dZ, G[0], G[1], G[2], W["o"], W["q"], W["k"], W["v"])
    mag = sum(_abs(a) @ _abs(W[k]).T for a, k in zip((dZ, *G), "oqkv"))
    assert_close(dX, rdx, rt, "dX", mag)
    dW = T.gt_proj_bwd_weight(Xd, t(dZ), t(G[0]), t(G[1]), t(G[2]))
    rdw = L.proj_bwd_weight(X, dZ, G[0], G[1], G[2])
    for got, ref, a, k in zip(dW, rdw, (dZ, *G), "oqkv"):
        assert_close(got, ref, 1e-5, "dW" + k, _abs(X).T @ _abs(a))
    torch.cuda.synchronize()


@pytest.mark.parametrize("n, d", [(1000, 64), (4097, 128), (20000, 256)])
def test_bf16_projections_round_to_nearest_even(n, d):
    """The bf16 results of Q/K/V, Z (its residual added in float32 before the
    one rounding) and dX are the float32 results rounded to nearest, ties to
    even, wherever the float32 result decides it (at d = 64 the resident
    kernels, at 128 and 256 the staged ones)."""
    X, W, dZ = I.layer_inputs(710 + d, n, d, "bf16")
    G = [I.layer_inputs(810 + k, n, d, "bf16")[2] for k in range(3)]
    Y = I.layer_inputs(910, n, d, "bf16")[2]
    t = lambda a: dev(a, torch.bfloat16)
    Xd, Wd = t(X), {k: t(v) for k, v in W.items()}
    Q, K, V = T.gt_proj_qkv(Xd, Wd["q"], Wd["k"], Wd["v"])
    for got, ref, k in zip((Q, K, V), L.proj_qkv(X, W["q"], W["k"], W["v"]), "qkv"):
        assert_rounded_to_nearest_even(got, ref, _abs(X) @ _abs(W[k]), "XW" + k)
    Z = T.gt_proj_out(Xd, Wd["o"], t(Y))
    assert_rounded_to_nearest_even(Z, L.proj_out(X, W["o"], Y), _abs(X) @ _abs(W["o"]) + _abs(Y), "Z")
    dX = T.gt_proj_bwd_data(t(dZ), t(G[0]), t(G[1]), t(G[2]), Wd["o"], Wd["q"], Wd["k"], Wd["v"])
    mag = sum(_abs(a) @ _abs(W[k]).T for a, k in zip((dZ, *G), "oqkv"))
    assert_rounded_to_nearest_even(dX, L.proj_bwd_data(dZ, G[0], G[1], G[2], W["o"], W["q"], W["k"], W["v"]),
                                   mag, "dX")


def test_weight_gradient_is_deterministic():
    n, d = 30000, 128
    X, W, dZ = I.layer_inputs(11, n, d, "bf16")
    t = lambda a: dev(a, torch.bfloat16)
    a = T.gt_proj_bwd_weight(t(X), t(dZ), t(dZ), t(X), t(dZ))
    b = T.gt_proj_bwd_weight(t(X), t(dZ), t(dZ), t(X), t(dZ))
    for x, y in zip(a, b):
        assert torch.equal(x, y)


LAYER = [("f32", 2, 32, False), ("bf16", 4, 32, True), ("f32", 1, 64, True), ("bf16", 8, 32, False),
         ("bf16", 8, 8, True)]   # the last: hidden 64 over 8 heads (Figure 7)


@pytest.mark.parametrize("case", LAYER, ids=[f"{a}-h{b}-d{c}-{'bias' if e else 'nobias'}" for a, b, c, e in LAYER])
def test_layer(case):
    dt, H, dh, bias = case
    d = H * dh
    n = 700
    degs = np.random.default_rng(d).integers(0, 90, n)
    ip, ix = I.random_graph(123 + d, n, n, degs)
    X, W, dZ = I.layer_inputs(31 + d, n, d, dt)
    b = I.edge_bias(41, ix.size, H) if bias else None
    t = lambda a: dev(a, TDT[dt])
    g = T.gt_graph_prepare(dev(ip), dev(ix), n, 4, 16, 16)
    Xd = t(X).requires_grad_()
    Wd = {k: t(v).requires_grad_() for k, v in W.items()}
    bd = dev(b, torch.float32).requires_grad_() if bias else None
    Z = T.sga_layer(g, H, Xd, Wd["q"], Wd["k"], Wd["v"], Wd["o"], bd)
    Z.backward(t(dZ))
    store = "bf16" if dt == "bf16" else None     # the intermediates the bf16 path stores
    rf = L.layer_fwd(ip, ix, X, W, H, b, store=store)
    rb = L.layer_bwd(ip, ix, X, W, H, dZ, b, store=store)
    rt = RTOL[dt]
    assert_close(Z, rf["Z"], rt, "Z")
    assert_close(Xd.grad, rb["dX"], rt, "dX")
    for k in "qkvo":
        assert_close(Wd[k].grad, rb["dW" + k], rt, "dW" + k)
    if bias:
        assert_close(bd.grad, rb["dbias"], rt, "dbias", head_axis=1)


def test_empty_node_set():
    """n = 0: the products are empty, the weight gradients exactly zero."""
    d = 128
    X = torch.empty((0, d), dtype=torch.float32, device="cuda")
    W = torch.ones((d, d), dtype=torch.float32, device="cuda")
    Q, K, V = T.gt_proj_qkv(X, W, W, W)
    assert Q.shape == (0, d)
    dX = T.gt_proj_bwd_data(X, X, X, X, W, W, W, W)
    assert dX.shape == (0, d)
    for dw in T.gt_proj_bwd_weight(X, X, X, X, X):
        assert dw.shape == (d, d) and torch.count_nonzero(dw).item() == 0


def test_layer_at_mid_size():
    """The whole layer at the Mid workload's size (131,072 nodes, 1.8M
    nonzeros, d = 128, fp32), forward and backward, every output against
    the fp64 oracle.  Magnitudes compose through the layer: a product's is
    |A| |B| with the attention oracle's magnitudes standing in for |dQ|,
    |dK|, |dV| and |Y| where those enter."""
    cfg = I.CONFIGS["mid"]
    P = I.make_problem(cfg)
    n, H, dh = cfg.n_rows, cfg.heads, cfg.head_dim
    d = H * dh
    X, W, dZ = I.layer_inputs(cfg.idx, n, d, "f32")
    t = lambda a: dev(a, torch.float32)
    g = T.gt_graph_prepare(dev(P.indptr), dev(P.indices), n)
    Xd = t(X).requires_grad_()
    Wd = {k: t(v).requires_grad_() for k, v in W.items()}
    print("layer mid: gpu", flush=True)
    Z = T.sga_layer(g, H, Xd, Wd["q"], Wd["k"], Wd["v"], Wd["o"])
    Z.backward(t(dZ))
    torch.cuda.synchronize()
    print("layer mid: oracle", flush=True)
    r3 = lambda a: np.asarray(a).reshape(n, H, dh)
    Q, K, V = L.proj_qkv(X, W["q"], W["k"], W["v"])
    m = {}
    Y, _ = O.fwd(P.indptr, P.indices, n, r3(Q), r3(K), r3(V), None, P.scale, mag=m)
    dQ, dK, dV, _ = O.bwd(P.indptr, P.indices, n, r3(Q), r3(K), r3(V), r3(dZ), None, P.scale, mag=m)
    f = lambda a: np.asarray(a).reshape(n, d)
    Y, dQ, dK, dV = f(Y), f(dQ), f(dK), f(dV)
    mY, mQ, mK, mV = (f(m[k]) for k in ("Y", "dQ", "dK", "dV"))
    aW = {k: _abs(v) for k, v in W.items()}
    aX, adZ = _abs(X), _abs(dZ)
    rt = RTOL["f32"]
    assert_close(Z, L.proj_out(X, W["o"], Y), rt, "Z", aX @ aW["o"] + mY)
    rdX = L.proj_bwd_data(dZ, dQ, dK, dV, W["o"], W["q"], W["k"], W["v"])
    mdX = adZ @ aW["o"].T + mQ @ aW["q"].T + mK @ aW["k"].T + mV @ aW["v"].T
    assert_close(Xd.grad, rdX, rt, "dX", mdX)
    rW = L.proj_bwd_weight(X, dZ, dQ, dK, dV)
    for k, ref, mg in zip("oqkv", rW, (aX.T @ adZ, aX.T @ mQ, aX.T @ mK, aX.T @ mV)):
        assert_close(Wd[k].grad, ref, rt, "dW" + k, mg)


@pytest.mark.parametrize("name", ["large", "hub"])
def test_projections_at_full_size(name):
    """The projection kernels at the Large (1,048,576 x 256) and Hub
    (2,400,000 x 128) node counts in bf16, as the layer benchmark runs them:
    sampled rows of Q, K, V, Z and dX against the oracle on those rows, and
    one weight gradient (a sum over every node) in full."""
    cfg = I.CONFIGS[name]
    n, d = cfg.n_rows, cfg.heads * cfg.head_dim
    X, W, dZ = I.layer_inputs(cfg.idx, n, d, "bf16")
    t = lambda a: dev(a, torch.bfloat16)
    Xd, dZd, Wd = t(X), t(dZ), {k: t(v) for k, v in W.items()}
    print(f"projections {name}: gpu", flush=True)
    Q, K, V = T.gt_proj_qkv(Xd, Wd["q"], Wd["k"], Wd["v"])
    Z = T.gt_proj_out(Xd, Wd["o"], dZd)                      # dZ stands in for Y
    dX = T.gt_proj_bwd_data(dZd, Xd, dZd, Xd, Wd["o"], Wd["q"], Wd["k"], Wd["v"])
    dW = T.gt_proj_bwd_weight(Xd, dZd, Xd, dZd, Xd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n), rng.integers(0, n, 4000)]))
    idx = torch.from_numpy(rows).cuda()
    x, z = X[rows], dZ[rows]
    rt = RTOL["bf16"]
    print(f"projections {name}: oracle on {rows.size} rows", flush=True)
    for got, k in zip((Q, K, V), "qkv"):
        assert_close(got[idx], L.proj_qkv(x, W[k], W[k], W[k])[0], rt, "XW" + k, _abs(x) @ _abs(W[k]))
    assert_close(Z[idx], L.proj_out(x, W["o"], z), rt, "Z", _abs(x) @ _abs(W["o"]) + _abs(z))
    rdx = L.proj_bwd_data(z, x, z, x, W["o"], W["q"], W["k"], W["v"])
    mag = _abs(z) @ _abs(W["o"]).T + _abs(x) @ _abs(W["q"]).T + _abs(z) @ _abs(W["k"]).T + _abs(x) @ _abs(W["v"]).T
    assert_close(dX[idx], rdx, rt, "dX", mag)
    print(f"projections {name}: oracle weight gradient", flush=True)
    Xf, Zf = X.astype(np.float64), dZ.astype(np.float64)
    assert_close(dW[0], Xf.T @ Zf, 1e-5, "dWo", np.abs(Xf).T @ np.abs(Zf))
    assert_close(dW[1], Xf.T @ Xf, 1e-5, "dWq", np.abs(Xf).T @ np.abs(Xf))
