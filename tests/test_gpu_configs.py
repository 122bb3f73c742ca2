"""Parity at the full workload sizes, in the launch configuration the
benchmark times (default thresholds):

* Mid (131K nodes, 1.8M nnz, fp32): every output against the full oracle;
* Large (1M nodes, 16.5M nnz, bf16), Hub-heavy (2.4M nodes, 62M nnz, bf16 +
  bias), Shard (524K rows x 4.2M columns, 16.8M nnz, bf16): every output
  against the full oracle, and, in a second test, sampled rows (the
  highest-degree ones, which are split across wavefronts, plus random and
  lowest-degree rows) and sampled columns (likewise, plus empty ones)
  against the oracle's per-row / per-column entry points together with the
  exact invariants of the backward over all outputs.

Set GT_INPUT_CACHE to a directory to reuse generated graphs across runs.
"""
import dataclasses

import numpy as np
import pytest
import torch

from graph_transformer_sparse_amd import gtattn as T
from graph_transformer_sparse_amd import inputs as I
from oracle import oracle as O

from gpu_util import RTOL, U32, assert_close, assert_lse, device_problem, to_np

pytestmark = pytest.mark.gpu


def _run(P):
    d = device_problem(P)
    g = T.gt_graph_prepare(d["indptr"], d["indices"], P.cfg.n_cols)
    Y, lse = T.gt_attn_fwd(g, d["Q"], d["K"], d["V"], d["bias"], P.scale)
    dQ, dK, dV, dB = T.gt_attn_bwd(g, d["Q"], d["K"], d["V"], Y, lse, d["dY"], d["bias"], P.scale)
    torch.cuda.synchronize()
    out = dict(Y=to_np(Y), lse=lse.cpu().numpy().astype(np.float64), dQ=to_np(dQ),
               dK=to_np(dK), dV=to_np(dV), dB=None if dB is None else dB.cpu().numpy().astype(np.float64),
               n_split_rows=g.st.rows.n_merges, n_split_cols=g.st.cols.n_merges)
    del d, g, Y, lse, dQ, dK, dV, dB
    torch.cuda.empty_cache()
    return out


def _sample(deg, rng, n_top=12, n_rand=150, n_low=8):
    order = np.argsort(-deg, kind="stable")
    pick = list(order[:n_top]) + list(rng.choice(deg.size, n_rand, replace=False))
    pick += list(order[-n_low:])
    empty = np.nonzero(deg == 0)[0]
    if empty.size:
        pick += list(empty[:4])
    return np.unique(np.asarray(pick, np.int32))


def _invariants(P, o, rtol):
    """Exact identities of the backward, checked over every output:
    sum_j dV_j = sum of dY over rows with edges (rows of U sum to 1);
    <dV, V>_h = <dY, Y>_h; <dQ, Q>_h = <dK, K>_h (the score is bilinear);
    with bias, sum_e dbias_e = 0 over every row.  The last one is a sum with
    cancellation.  Its terms are U_e (dU_e - D_i), computed around the shift
    c_i = <dY_i, Y_i> as (w_e - p_e (D_i - c_i)) / L with w_e = p_e (dU_e - c_i):
    in float32 each is good to about u (|dS_e| + 2 U_e m_i), m_i =
    sum_c |dY_i,c| |Y_i,c| (which bounds |c_i| and |D_i|), so the bound
    allows 64 u (sum |dS| + 2 m_i).  With bf16 storage, w_e and p_e are
    staged as bf16 (relative rounding 2^-9 each), which adds up to
    2^-9 (|dS_e| + 2 U_e |D_i - c_i|) per term, and |D_i - c_i| <= 2^-9 m_i
    (the rounding of the stored Y): the bound adds 2^-8 sum |dS| + 2^-15 m_i
    (twice those)."""
    Q, K, V, dY = (x.astype(np.float64) for x in (P.Q, P.K, P.V, P.dY))
    has = np.diff(P.indptr) > 0
    lhs = o["dV"].sum(axis=0)
    rhs = dY[has].sum(axis=0)
    scale = np.sqrt(np.sum(np.abs(o["dV"]) ** 2, axis=0)) + np.abs(rhs)
    assert np.all(np.abs(lhs - rhs) <= 4 * rtol * scale + 1e-6), "sum dV != sum dY"
    for a, b, c, d, name in ((o["dV"], V, dY, o["Y"], "<dV,V> != <dY,Y>"),
                             (o["dQ"], Q, o["dK"], K, "<dQ,Q> != <dK,K>")):
        x = np.einsum("nhc,nhc->h", a, b)
        y = np.einsum("nhc,nhc->h", c, d)
        mag = np.einsum("nhc,nhc->h", np.abs(a), np.abs(b)) + np.einsum("nhc,nhc->h", np.abs(c), np.abs(d))
        assert np.all(np.abs(x - y) <= 4 * rtol * mag), (name, x, y)
    if o["dB"] is not None:
        rows = np.repeat(np.arange(P.cfg.n_rows), np.diff(P.indptr))
        Dh = np.einsum("ihc,ihc->ih", np.abs(dY), np.abs(o["Y"]))
        bf16 = P.cfg.dtype == "bf16"
        for h in range(P.cfg.heads):
            s = np.bincount(rows, weights=o["dB"][:, h], minlength=P.cfg.n_rows)
            a = np.bincount(rows, weights=np.abs(o["dB"][:, h]), minlength=P.cfg.n_rows)
            tol = 4 * rtol * a + 64 * U32 * (a + 2 * Dh[:, h])
            if bf16:
                tol = tol + 2.0 ** -8 * a + 2.0 ** -15 * Dh[:, h]
            bad = np.abs(s) > tol
            if bad.any():
                i = int(np.argmax(np.where(bad, np.abs(s) / np.maximum(tol, 1e-300), 0)))
                raise AssertionError(f"dbias of row {i} head {h} sums to {s[i]!r}; sum |dbias| "
                                     f"{a[i]!r}, sum |dY Y| {Dh[i, h]!r}, "
                                     f"degree {P.indptr[i + 1] - P.indptr[i]}")


@pytest.mark.parametrize("hidden, nodes", [(128, 1 << 17), (64, 1 << 17), (256, 1 << 17),
                                           (128, 1 << 16), (128, 1 << 18)])
def test_mid_full(hidden, nodes):
    """The Mid workload (hidden 128 over 8 heads, 2^17 nodes), the same graph
    at the pages' other hidden sizes, 64 and 256 (Figure 7: head_dim 8 and
    32), and the same recipe at 2^16 and 2^18 nodes (Figure 6's axis), every
    output against the oracle."""
    cfg = I.CONFIGS["mid"]
    if hidden != cfg.heads * cfg.head_dim or nodes != cfg.n_rows:
        cfg = dataclasses.replace(cfg, head_dim=hidden // cfg.heads, n_rows=nodes, n_cols=nodes)
    P = I.make_problem(cfg)
    print(f"mid hidden {hidden} nodes {nodes}: gpu", flush=True)
    o = _run(P)
    assert o["n_split_rows"] > 0 and o["n_split_cols"] > 0
    print("mid: oracle", flush=True)
    M = P.cfg.n_cols
    m = {}
    rY, rl = O.fwd(P.indptr, P.indices, M, P.Q, P.K, P.V, None, P.scale, mag=m)
    rQ, rK, rV, _ = O.bwd(P.indptr, P.indices, M, P.Q, P.K, P.V, P.dY, None, P.scale, mag=m)
    rt = RTOL["f32"]
    assert_close(o["Y"], rY, rt, "Y", m["Y"])
    assert_lse(o["lse"], rl, 1e-5)
    assert_close(o["dQ"], rQ, rt, "dQ", m["dQ"])
    assert_close(o["dK"], rK, rt, "dK", m["dK"])
    assert_close(o["dV"], rV, rt, "dV", m["dV"])
    _invariants(P, o, rt)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["large", "hub", "shard"])
def test_big_config_sampled(name):
    cfg = I.CONFIGS[name]
    print(f"{name}: generating", flush=True)
    P = I.make_problem(cfg)
    print(f"{name}: gpu (nnz {P.nnz})", flush=True)
    o = _run(P)
    assert o["n_split_rows"] > 0
    rng = np.random.default_rng(cfg.idx)
    rows = _sample(np.diff(P.indptr), rng)
    ptr_t = np.zeros(cfg.n_cols + 1, np.int64)
    np.cumsum(np.bincount(P.indices, minlength=cfg.n_cols), out=ptr_t[1:])
    cols = _sample(np.diff(ptr_t), rng)
    print(f"{name}: oracle on {rows.size} rows, {cols.size} columns", flush=True)
    M = cfg.n_cols
    m = {}
    rY, rl, rQ, rB = O.rows(P.indptr, P.indices, M, P.Q, P.K, P.V, P.dY, rows, P.bias, P.scale,
                            mag=m)
    rK, rV = O.cols(P.indptr, P.indices, M, P.Q, P.K, P.V, P.dY, cols, P.bias, P.scale, mag=m)
    rt = RTOL[cfg.dtype]
    assert_close(o["Y"][rows], rY, rt, "Y", m["Y"])
    assert_lse(o["lse"][rows], rl, 1e-4)
    assert_close(o["dQ"][rows], rQ, rt, "dQ", m["dQ"])
    assert_close(o["dK"][cols], rK, rt, "dK", m["dK"])
    assert_close(o["dV"][cols], rV, rt, "dV", m["dV"])
    if P.bias is not None:
        eb = np.concatenate([np.arange(P.indptr[i], P.indptr[i + 1]) for i in rows])
        assert_close(o["dB"][eb], rB, rt, "dbias", head_axis=1)
    print(f"{name}: invariants", flush=True)
    _invariants(P, o, rt)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["large", "hub", "shard"])
def test_big_config_full(name):
    """Every output of the large workloads against the oracle on the whole
    graph: every row of Y, lse, dQ (and dbias), every column of dK and dV,
    at the tolerance above, in the launch configuration the benchmark times
    (default thresholds; split rows and columns present)."""
    cfg = I.CONFIGS[name]
    print(f"{name}: generating", flush=True)
    P = I.make_problem(cfg)
    print(f"{name}: gpu (nnz {P.nnz})", flush=True)
    o = _run(P)
    assert o["n_split_rows"] > 0
    print(f"{name}: oracle forward", flush=True)
    M = cfg.n_cols
    rt = RTOL[cfg.dtype]
    m = {}
    rY, rl = O.fwd(P.indptr, P.indices, M, P.Q, P.K, P.V, P.bias, P.scale, mag=m)
    assert_close(o["Y"], rY, rt, "Y", m.pop("Y"))
    assert_lse(o["lse"], rl, 1e-4)
    del rY, rl
    print(f"{name}: oracle backward", flush=True)
    rQ, rK, rV, rB = O.bwd(P.indptr, P.indices, M, P.Q, P.K, P.V, P.dY, P.bias, P.scale, mag=m)
    assert_close(o["dQ"], rQ, rt, "dQ", m.pop("dQ"))
    assert_close(o["dK"], rK, rt, "dK", m.pop("dK"))
    assert_close(o["dV"], rV, rt, "dV", m.pop("dV"))
    if P.bias is not None:
        assert_close(o["dB"], rB, rt, "dbias", head_axis=1)
    print(f"{name}: done", flush=True)


@pytest.mark.parametrize("name", ["mid", "large", "hub", "shard"])
def test_prep_full_configs(name):
    """Graph preparation at the full workload sizes, default thresholds:
    the CSR transpose and both degree-ordered schedules bit-exact with the
    oracle."""
    cfg = I.CONFIGS[name]
    ip, ix = I.named_graph(cfg)
    print(f"prep {name}: gpu", flush=True)
    g = T.gt_graph_prepare(torch.from_numpy(ip).cuda(), torch.from_numpy(ix).cuda(), cfg.n_cols)
    torch.cuda.synchronize()
    print(f"prep {name}: oracle transpose", flush=True)
    pt, it, pm = O.transpose(ip, ix, cfg.n_cols)
    assert np.array_equal(g.indptr_t.cpu().numpy(), pt)
    assert np.array_equal(g.indices_t.cpu().numpy(), it)
    assert np.array_equal(g.perm.cpu().numpy(), pm)
    ts, tm, ch = g.st.t_small, g.st.t_mid, g.st.chunk   # what prepare chose for this size
    assert (ts, tm, ch) == T.gt_graph_thresholds(ix.size)
    print(f"prep {name}: oracle schedules", flush=True)
    for which, ptr in (("rows", ip), ("cols", pt)):
        got, want = g.schedule(which), O.schedule(ptr, ts, tm, ch, 4 if which == "rows" else 1)
        assert np.array_equal(got["order"].cpu().numpy(), want["order"]), which
        assert tuple(got["counts"]) == tuple(int(c) for c in want["counts"]), which
        assert np.array_equal(got["items"].cpu().numpy(), want["items"]), which
        assert np.array_equal(got["merges"].cpu().numpy(), want["merges"]), which
        o = np.asarray(want["order"], np.int64)
        assert np.array_equal(got["spans"].cpu().numpy(),
                              np.stack([ptr[o], ptr[o + 1]], axis=1).reshape(-1, 2)), which
