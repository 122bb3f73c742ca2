"""fp64 CPU oracle of one sparse graph attention layer, dense parts included.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use this module; the GPU path never does.

The layer ("Scalable and Adaptive Parallel Training of Graph Transformer on
Large Graphs", Section 2.1, Eq. 3-5):
    Q = X W_Q,  K = X W_K,  V = X W_V        (Eq. 3, dense projections)
    Y = sparse graph attention of (A, Q, K, V) (Eq. 4-5; oracle.fwd)
    Z = X W_o + Y                             (Eq. 5, the layer output X')
and its gradients, given dZ:
    dY = dZ,  (dQ, dK, dV) = attention backward (oracle.bwd),
    dX = dZ W_o^T + dQ W_Q^T + dK W_K^T + dV W_V^T,
    dW_o = X^T dZ,  dW_Q = X^T dQ,  dW_K = X^T dK,  dW_V = X^T dV.
Readings: weights are [d, d] row-major and act as X W (the projection maps
node features of width d to the H * dh channels of the heads, here d = H dh);
the layer is square (every node is both a query and a key/value node).
With ``store="bf16"`` the tensors a bf16 layer keeps in memory between its
steps -- Q, K, V and Y in the forward, dQ, dK and dV in the backward -- are
rounded to bf16 (nearest, ties to even) where they are stored; everything
else stays float64.
numpy's float64 matmul is the one library step; nothing else is fused.
"""
from __future__ import annotations

import numpy as np

from . import oracle as O


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def round_bf16(x):
    """Round to the nearest bfloat16 value, ties to even (finite inputs):
    round to float32 first, then keep the top 16 bits of the float32 pattern
    after adding half an ulp of bf16 (plus one if the kept part is odd)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(np.shape(x))


def _store(x, store):
    return round_bf16(x) if store == "bf16" else x


def proj_qkv(X, Wq, Wk, Wv):
    X = _f64(X)
    return X @ _f64(Wq), X @ _f64(Wk), X @ _f64(Wv)


def proj_out(X, Wo, Y):
    return _f64(X) @ _f64(Wo) + _f64(Y)


def proj_bwd_data(dZ, dQ, dK, dV, Wo, Wq, Wk, Wv):
    return (_f64(dZ) @ _f64(Wo).T + _f64(dQ) @ _f64(Wq).T + _f64(dK) @ _f64(Wk).T
            + _f64(dV) @ _f64(Wv).T)


def proj_bwd_weight(X, dZ, dQ, dK, dV):
    Xt = _f64(X).T
    return Xt @ _f64(dZ), Xt @ _f64(dQ), Xt @ _f64(dK), Xt @ _f64(dV)


def layer_fwd(indptr, indices, X, W, heads, bias=None, scale=None, store=None):
    """W = dict(q, k, v, o) of [d, d].  Returns dict(Q, K, V, Y, lse, Z)."""
    X = _f64(X)
    n, d = X.shape
    dh = d // heads
    Q, K, V = (_store(t, store) for t in proj_qkv(X, W["q"], W["k"], W["v"]))
    r = lambda t: t.reshape(n, heads, dh)
    Y, lse = O.fwd(indptr, indices, n, r(Q), r(K), r(V), bias, scale)
    Y = _store(Y.reshape(n, d), store)
    Z = proj_out(X, W["o"], Y)
    return dict(Q=Q, K=K, V=V, Y=Y, lse=lse, Z=Z)


def layer_bwd(indptr, indices, X, W, heads, dZ, bias=None, scale=None, store=None):
    """Gradients of <Z, dZ>: dict(dX, dWq, dWk, dWv, dWo, dQ, dK, dV, dbias)."""
    X = _f64(X)
    n, d = X.shape
    dh = d // heads
    Q, K, V = (_store(t, store) for t in proj_qkv(X, W["q"], W["k"], W["v"]))
    r = lambda t: t.reshape(n, heads, dh)
    dQ, dK, dV, dB = O.bwd(indptr, indices, n, r(Q), r(K), r(V), r(_f64(dZ)), bias, scale)
    dQ, dK, dV = (_store(t.reshape(n, d), store) for t in (dQ, dK, dV))
    dX = proj_bwd_data(dZ, dQ, dK, dV, W["o"], W["q"], W["k"], W["v"])
    dWo, dWq, dWk, dWv = proj_bwd_weight(X, dZ, dQ, dK, dV)
    return dict(dX=dX, dWq=dWq, dWk=dWk, dWv=dWv, dWo=dWo, dQ=dQ, dK=dK, dV=dV, dbias=dB)
