"""The Python binding checks tensor shapes, dtypes and devices against the
prepared graph before any pointer reaches the C ABI (which gets only
pointers and would read or write a wrongly sized array out of bounds).
Runs without a GPU: every call here fails its checks before the library is
touched."""
import pytest
import torch

from graph_transformer_sparse_amd import gtattn as T

R, M, E, H, DH = 10, 8, 20, 2, 16


def _graph():
    st = T.GtGraph()
    st.n_rows, st.n_cols, st.nnz = R, M, E
    return T.Graph(st, torch.empty(0, dtype=torch.uint8), torch.zeros(R + 1, dtype=torch.int32),
                   torch.zeros(E, dtype=torch.int32))


def _qkv(dt=torch.float32):
    return (torch.zeros(R, H, DH, dtype=dt), torch.zeros(M, H, DH, dtype=dt),
            torch.zeros(M, H, DH, dtype=dt))


@pytest.mark.parametrize("bad, msg", [
    (dict(Q=torch.zeros(R + 1, H, DH)), "Q has shape"),
    (dict(K=torch.zeros(M - 1, H, DH)), "K has shape"),
    (dict(V=torch.zeros(M, H, DH + 1)), "V has shape"),
    (dict(K=torch.zeros(M, H, DH, dtype=torch.bfloat16)), "K has dtype"),
    (dict(Q=torch.zeros(R, H, DH, dtype=torch.float16)), "unsupported dtype"),
    (dict(bias=torch.zeros(E + 1, H)), "bias has shape"),
    (dict(bias=torch.zeros(E, H, dtype=torch.float64)), "bias has dtype"),
    (dict(V=torch.zeros(M, DH, H).transpose(1, 2)), "V must be contiguous"),
    (dict(Q=torch.zeros(R, H * DH)), "Q must be a"),
])
def test_fwd_rejects_wrong_tensors(bad, msg):
    Q, K, V = _qkv()
    args = dict(Q=Q, K=K, V=V, bias=None)
    args.update(bad)
    with pytest.raises(ValueError, match=msg):
        T.gt_attn_fwd(_graph(), **args)


def test_fwd_rejects_wrong_outputs():
    Q, K, V = _qkv()
    with pytest.raises(ValueError, match="Y has shape"):
        T.gt_attn_fwd(_graph(), Q, K, V, Y=torch.zeros(R, H, DH + 1))
    with pytest.raises(ValueError, match="lse has dtype"):
        T.gt_attn_fwd(_graph(), Q, K, V, lse=torch.zeros(R, H, dtype=torch.float64))


def test_bwd_rejects_wrong_tensors():
    Q, K, V = _qkv()
    Y, lse, dY = torch.zeros(R, H, DH), torch.zeros(R, H), torch.zeros(R, H, DH)
    g = _graph()
    with pytest.raises(ValueError, match="Y has shape"):
        T.gt_attn_bwd(g, Q, K, V, torch.zeros(R, H, DH - 1), lse, dY)
    with pytest.raises(ValueError, match="lse has shape"):
        T.gt_attn_bwd(g, Q, K, V, Y, torch.zeros(R, H + 1), dY)
    with pytest.raises(ValueError, match="dY has shape"):
        T.gt_attn_bwd(g, Q, K, V, Y, lse, torch.zeros(R - 1, H, DH))
    with pytest.raises(ValueError, match="dK has shape"):
        T.gt_attn_bwd(g, Q, K, V, Y, lse, dY, dK=torch.zeros(R, H, DH))
    with pytest.raises(ValueError, match="bias and dbias"):
        T.gt_attn_bwd(g, Q, K, V, Y, lse, dY, dbias=torch.zeros(E, H))
    with pytest.raises(ValueError, match="dbias has shape"):
        T.gt_attn_bwd(g, Q, K, V, Y, lse, dY, bias=torch.zeros(E, H), dbias=torch.zeros(E, H + 1))


def test_host_tensors_are_refused():
    """Correctly shaped tensors in host memory: refused, never handed to the library."""
    Q, K, V = _qkv()
    with pytest.raises(ValueError, match="must be on a GPU"):
        T.gt_attn_fwd(_graph(), Q, K, V)
    with pytest.raises(ValueError, match="must be on a GPU"):
        T.gt_attn_bwd(_graph(), Q, K, V, torch.zeros(R, H, DH), torch.zeros(R, H),
                      torch.zeros(R, H, DH))
    with pytest.raises(ValueError, match="must be on a GPU"):
        T.gt_proj_qkv(torch.zeros(4, 64), *(torch.zeros(64, 64) for _ in range(3)))
    with pytest.raises(ValueError, match="must be on a GPU"):
        T.gt_head_split(torch.zeros(4, 8, 16), 2)
    with pytest.raises(ValueError, match="same GPU"):
        T.gt_graph_prepare(torch.zeros(R + 1, dtype=torch.int32), torch.zeros(E, dtype=torch.int32), M)


def test_projection_shapes():
    X = torch.zeros(4, 64)
    W = torch.zeros(64, 64)
    with pytest.raises(ValueError, match="Wk has shape"):
        T.gt_proj_qkv(X, W, torch.zeros(64, 32), W)
    with pytest.raises(ValueError, match="Y has shape"):
        T.gt_proj_out(X, W, torch.zeros(5, 64))
    with pytest.raises(ValueError, match="dV has dtype"):
        T.gt_proj_bwd_data(X, X, X, X.to(torch.bfloat16), W, W, W, W)
    with pytest.raises(ValueError, match="dZ has shape"):
        T.gt_proj_bwd_weight(X, torch.zeros(4, 32), X, X, X)


def test_prepare_rejects_wrong_index_types():
    with pytest.raises(ValueError, match="indptr must be int32"):
        T.gt_graph_prepare(torch.zeros(R + 1, dtype=torch.int64), torch.zeros(E, dtype=torch.int32), M)
    with pytest.raises(ValueError, match="indices must be a 1-D"):
        T.gt_graph_prepare(torch.zeros(R + 1, dtype=torch.int32), torch.zeros(2, E, dtype=torch.int32), M)
