"""Parity of the HIP path with the fp64 oracle: forward (Y, lse) and backward
(dQ, dK, dV, dbias), through the C ABI, on seeded inputs.

* a sweep of small graphs whose degrees sit on and around the schedule's
  thresholds (empty rows, rows of 1, 2, 63, 64, 65 nonzeros, split rows and
  columns with ragged last pieces), rectangular adjacencies, every supported
  head count / head size / dtype, with and without bias;
* the 2,000-node config in full, under several thresholds;
* -inf-masked edges, and scores spread over hundreds (running maxima that
  move in most rounds, weights that underflow), against bounds derived from
  the float32 rounding of the scores;
* bf16 outputs rounded to nearest even wherever the float32 result decides it;
* bitwise determinism.
The large configurations are in test_gpu_configs.py.
"""
import numpy as np
import pytest
import torch

from graph_transformer_sparse_amd import gtattn as T
from graph_transformer_sparse_amd import inputs as I
from oracle import oracle as O

from gpu_util import (RTOL, U32, assert_close, assert_lse, assert_rounded_to_nearest_even,
                      device_problem)

pytestmark = pytest.mark.gpu


def run_gpu(P, th=None):
    d = device_problem(P)
    g = T.gt_graph_prepare(d["indptr"], d["indices"], P.cfg.n_cols, *(th or ()))
    Y, lse = T.gt_attn_fwd(g, d["Q"], d["K"], d["V"], d["bias"], P.scale)
    dQ, dK, dV, dB = T.gt_attn_bwd(g, d["Q"], d["K"], d["V"], Y, lse, d["dY"], d["bias"], P.scale)
    torch.cuda.synchronize()
    return Y, lse, dQ, dK, dV, dB


def check_full(P, out, rtol=None):
    rtol = RTOL[P.cfg.dtype] if rtol is None else rtol
    Y, lse, dQ, dK, dV, dB = out
    M = P.cfg.n_cols
    m = {}
    rY, rl = O.fwd(P.indptr, P.indices, M, P.Q, P.K, P.V, P.bias, P.scale, mag=m)
    rQ, rK, rV, rB = O.bwd(P.indptr, P.indices, M, P.Q, P.K, P.V, P.dY, P.bias, P.scale, mag=m)
    assert_close(Y, rY, rtol, "Y", m["Y"])
    assert_lse(lse, rl, 1e-5 if P.cfg.dtype == "f32" else 1e-4)
    assert_close(dQ, rQ, rtol, "dQ", m["dQ"])
    assert_close(dK, rK, rtol, "dK", m["dK"])
    assert_close(dV, rV, rtol, "dV", m["dV"])
    if P.bias is not None:
        assert_close(dB, rB, rtol, "dbias", head_axis=1)
    else:
        assert dB is None


def _degrees(rng, R, M):
    base = [0, 1, 2, 3, 7, 8, 9, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200]
    d = np.array([min(x, M) for x in base] + list(rng.integers(0, min(M, 70), R - len(base))))
    rng.shuffle(d)
    return d


SHAPES = [  # dtype, heads, head_dim
    ("f32", 1, 64), ("f32", 8, 16), ("f32", 2, 32), ("f32", 4, 64), ("f32", 8, 32),
    ("bf16", 8, 32), ("bf16", 4, 32), ("bf16", 8, 16), ("bf16", 1, 16), ("bf16", 8, 64),
    ("bf16", 2, 64), ("f32", 1, 16),
    # hidden 64 over 8 heads (the paper's smallest hidden size, Figure 7), and head_dim 128
    ("f32", 8, 8), ("bf16", 8, 8), ("bf16", 1, 8), ("f32", 2, 128), ("bf16", 4, 128),
    ("bf16", 1, 128),
]
THRESH = [None, (2, 8, 8), (4, 16, 5), (0, 0, 3)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{a}-h{b}-d{c}" for a, b, c in SHAPES])
@pytest.mark.parametrize("bias", [False, True], ids=["nobias", "bias"])
def test_small_graphs(shape, bias):
    dt, H, dh = shape
    k = SHAPES.index(shape) * 2 + int(bias)
    rng = np.random.default_rng(k)
    R, M = (120, 260) if k % 3 == 0 else ((260, 90) if k % 3 == 1 else (220, 220))
    degs = _degrees(rng, R, M)
    ip, ix = I.random_graph(300 + k, R, M, degs, self_loops=False)
    P = I.small_problem(k, ip, ix, M, H, dh, dt, bias)
    for th in THRESH:
        print(f"small {shape} bias={bias} th={th}", flush=True)
        check_full(P, run_gpu(P, th))


def test_tiny_config():
    P = I.make_problem(I.CONFIGS["tiny"])
    for th in (None, (2, 6, 4), (16, 16, 7)):
        print(f"tiny th={th}", flush=True)
        check_full(P, run_gpu(P, th))


def test_scale_other_than_default():
    ip, ix = I.random_graph(9, 64, 64, np.full(64, 12))
    P = I.small_problem(9, ip, ix, 64, 4, 16, "f32", True)
    d = device_problem(P)
    g = T.gt_graph_prepare(d["indptr"], d["indices"], 64, 2, 8, 8)
    Y, lse = T.gt_attn_fwd(g, d["Q"], d["K"], d["V"], d["bias"], 0.3)
    dQ, dK, dV, dB = T.gt_attn_bwd(g, d["Q"], d["K"], d["V"], Y, lse, d["dY"], d["bias"], 0.3)
    rY, rl = O.fwd(ip, ix, 64, P.Q, P.K, P.V, P.bias, 0.3)
    rQ, rK, rV, rB = O.bwd(ip, ix, 64, P.Q, P.K, P.V, P.dY, P.bias, 0.3)
    for a, b, n in ((Y, rY, "Y"), (dQ, rQ, "dQ"), (dK, rK, "dK"), (dV, rV, "dV"), (dB, rB, "dB")):
        assert_close(a, b, 1e-5, n, head_axis=1 if n == "dB" else "auto")
    assert_lse(lse, rl, 1e-5)


@pytest.mark.parametrize("dt, H, dh", [("f32", 4, 16), ("bf16", 4, 32), ("f32", 1, 64)])
def test_minus_inf_bias_masks_edges(dt, H, dh):
    """A -inf bias masks its edge: rows whose first edges (a whole first
    round of a lane group, or of a wavefront's groups) are masked, rows with
    every edge masked in one head or in all heads, and split rows whose first
    pieces are masked, against the oracle (which treats a masked edge as
    absent and a fully masked row as empty).  Several thresholds, so that
    the masked edges fall in small rows, whole-wavefront rows and pieces."""
    import dataclasses
    rng = np.random.default_rng(81)
    R, M = 300, 280
    degs = _degrees(rng, R, M)
    ip, ix = I.random_graph(81, R, M, degs, self_loops=False)
    P = I.small_problem(81, ip, ix, M, H, dh, dt, True)
    b = P.bias.copy()
    deg = np.diff(ip)
    for i in np.nonzero(deg > 0)[0]:
        lo, d = ip[i], deg[i]
        kind = i % 5
        if kind == 0:      # the first few edges, every head
            b[lo:lo + min(d, 1 + i % 9)] = -np.inf
        elif kind == 1:    # the whole row in head 0
            b[lo:lo + d, 0] = -np.inf
        elif kind == 2 and i % 3 == 0:   # the whole row, every head
            b[lo:lo + d] = -np.inf
        elif kind == 3:    # the first half of the row (whole leading pieces of split rows)
            b[lo:lo + d // 2, H - 1] = -np.inf
    P = dataclasses.replace(P, bias=b)
    for th in (None, (2, 8, 8), (0, 0, 3)):
        print(f"minus-inf bias {dt} H={H} dh={dh} th={th}", flush=True)
        out = run_gpu(P, th)
        for t in out:
            assert not torch.isnan(t).any()
        check_full(P, out)


def _wide_problem(dt, H, dh):
    """A graph with rows of up to 600 edges and a bias ramp of 1 per edge,
    rising along even rows and falling along odd ones."""
    import dataclasses
    rng = np.random.default_rng(91)
    R, M = 150, 700
    degs = np.array([1, 2, 3, 9, 65, 130, 257, 600] + list(rng.integers(0, 300, R - 8)))
    rng.shuffle(degs)
    ip, ix = I.random_graph(91, R, M, degs, self_loops=False)
    P = I.small_problem(91, ip, ix, M, H, dh, dt, True)
    src = np.repeat(np.arange(R), np.diff(ip))
    ramp = (np.arange(ip[-1]) - ip[src]) * np.where(src % 2 == 0, 1.0, -1.0)
    return dataclasses.replace(P, bias=(P.bias + ramp[:, None]).astype(np.float32))


def score_rounding_bounds(P, lse, U, Ymag):
    """First-order bounds on what float32 rounding of the scores does to each
    output, with eps_i = u max_e [(dh + 3) S_e + 3 |b_e| + |lse_i|] over the
    edges e of row i, S_e = scale sum_c |q_c k_c|:
      weight U_e:  2 eps_i U_e (its own change and the normalisation's);
      D_i:         2 eps_i A_i,  A_i = sum_e U_e |dU_e| <= <|dY_i|, Ymag_i>;
      dS_e:        2 eps_i U_e (|dY_i|.|V_j| + 2 A_i)  (also dbias);
      Y_i:         2 eps_i Ymag_i;
      dQ, dK, dV:  the dS_e and weight bounds times |K_j|, |Q_i|, |dY_i|,
                   summed over the row or column.
    bf16 configs stage (p, w) per edge in bf16 for dbias: 2^-9 U_e
    (|dU_e| + 3 A_i) more.  Every bound is returned doubled."""
    ip, ix = P.indptr, P.indices
    R, M = ip.size - 1, P.K.shape[0]
    H, dh, sc = P.Q.shape[1], P.Q.shape[2], P.scale
    src = np.repeat(np.arange(R), np.diff(ip))
    S = sc * np.einsum("ehc,ehc->eh", np.abs(P.Q[src]), np.abs(P.K[ix]))
    lmag = np.where(np.isfinite(lse), np.abs(lse), 0.0)
    eps = np.zeros((R, H))
    np.maximum.at(eps, src, U32 * ((dh + 3) * S + 3 * np.abs(P.bias) + lmag[src]))
    A = np.einsum("rhc,rhc->rh", np.abs(P.dY), Ymag)
    dUabs = np.einsum("ehc,ehc->eh", np.abs(P.dY[src]), np.abs(P.V[ix]))
    dW = 2 * eps[src] * U
    dS = dW * (dUabs + 2 * A[src])
    b = {"Y": 2 * eps[:, :, None] * Ymag, "dbias": dS.copy(),
         "dQ": np.zeros((R, H, dh)), "dK": np.zeros((M, H, dh)), "dV": np.zeros((M, H, dh))}
    np.add.at(b["dQ"], src, sc * dS[:, :, None] * np.abs(P.K[ix]))
    np.add.at(b["dK"], ix, sc * dS[:, :, None] * np.abs(P.Q[src]))
    np.add.at(b["dV"], ix, dW[:, :, None] * np.abs(P.dY[src]))
    if P.cfg.dtype == "bf16":
        b["dbias"] += 2.0 ** -9 * U * (dUabs + 3 * A[src])
    return {k: 2 * v for k, v in b.items()}


@pytest.mark.parametrize("dt, H, dh", [("f32", 4, 16), ("bf16", 4, 32), ("f32", 1, 64)])
def test_wide_score_range(dt, H, dh):
    """Scores spread over hundreds: along the rows of a bias ramp the running
    maximum moves up in most rounds (rescaling the state each time) or stays
    at the first edge, more than half of the weights underflow to 0 in
    float32, and the pieces of split rows merge with shifts far apart.  The
    float32 rounding of the scores themselves then bounds the accuracy
    (score_rounding_bounds), which is added to the usual tolerance."""
    P = _wide_problem(dt, H, dh)
    ip, ix, M, sc = P.indptr, P.indices, P.cfg.n_cols, P.scale
    m = {}
    rY, rl, rU = O.fwd(ip, ix, M, P.Q, P.K, P.V, P.bias, sc, want_U=True, mag=m)
    rQ, rK, rV, rB = O.bwd(ip, ix, M, P.Q, P.K, P.V, P.dY, P.bias, sc, mag=m)
    assert np.ptp(P.bias) > 800 and np.mean(rU < 1e-38) > 0.5
    extra = score_rounding_bounds(P, rl, rU, m["Y"])
    rtol = RTOL[dt]
    for th in (None, (2, 8, 8), (0, 0, 3)):
        print(f"wide scores {dt} H={H} dh={dh} th={th}", flush=True)
        Y, lse, dQ, dK, dV, dB = run_gpu(P, th)
        assert_lse(lse, rl, 1e-5 if dt == "f32" else 1e-4)
        assert_close(Y, rY, rtol, "Y", m["Y"], extra=extra["Y"])
        assert_close(dQ, rQ, rtol, "dQ", m["dQ"], extra=extra["dQ"])
        assert_close(dK, rK, rtol, "dK", m["dK"], extra=extra["dK"])
        assert_close(dV, rV, rtol, "dV", m["dV"], extra=extra["dV"])
        assert_close(dB, rB, rtol, "dbias", head_axis=1, extra=extra["dbias"])


@pytest.mark.parametrize("bias", [False, True], ids=["nobias", "bias"])
def test_bf16_outputs_round_to_nearest_even(bias):
    """bf16 outputs are the float32 results rounded to nearest, ties to even,
    wherever the float32 result decides it (assert_rounded_to_nearest_even)."""
    rng = np.random.default_rng(123)
    R = M = 300
    ip, ix = I.random_graph(123, R, M, rng.integers(1, 60, R))
    P = I.small_problem(123, ip, ix, M, 4, 32, "bf16", bias)
    m = {}
    rY, _ = O.fwd(ip, ix, M, P.Q, P.K, P.V, P.bias, P.scale, mag=m)
    rQ, rK, rV, _ = O.bwd(ip, ix, M, P.Q, P.K, P.V, P.dY, P.bias, P.scale, mag=m)
    Y, _, dQ, dK, dV, _ = run_gpu(P)
    for name, got, r in (("Y", Y, rY), ("dQ", dQ, rQ), ("dK", dK, rK), ("dV", dV, rV)):
        assert_rounded_to_nearest_even(got, r, m[name], name)


def test_bitwise_determinism():
    """Two runs, and a run on another stream, give bitwise-equal outputs."""
    P = I.make_problem(I.CONFIGS["tiny"])
    a = run_gpu(P, (2, 6, 4))
    b = run_gpu(P, (2, 6, 4))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c = run_gpu(P, (2, 6, 4))
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        if x is not None:
            assert torch.equal(x, y) and torch.equal(x, z)


def test_one_graph_two_concurrent_streams():
    """One prepared graph, two streams running forward and backward at the
    same time on different inputs (each call with its own work buffer): the
    library keeps no state between calls, so each stream's results are
    bitwise those of a lone run."""
    ip, ix = I.random_graph(31, 400, 400, _degrees(np.random.default_rng(31), 400, 400))
    probs = [I.small_problem(31 + k, ip, ix, 400, 4, 32, "bf16", True) for k in range(2)]
    devs = [device_problem(P) for P in probs]
    g = T.gt_graph_prepare(devs[0]["indptr"], devs[0]["indices"], 400, 2, 8, 8)

    def step(d, P):
        Y, lse = T.gt_attn_fwd(g, d["Q"], d["K"], d["V"], d["bias"], P.scale)
        return (Y, lse) + T.gt_attn_bwd(g, d["Q"], d["K"], d["V"], Y, lse, d["dY"], d["bias"], P.scale)

    alone = [step(d, P) for d, P in zip(devs, probs)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    outs = [[], []]
    for _ in range(4):                       # interleaved, no synchronisation in between
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                outs[k].append(step(devs[k], probs[k]))
    torch.cuda.synchronize()
    for k in range(2):
        for got in outs[k]:
            for x, y in zip(got, alone[k]):
                assert torch.equal(x, y)
    assert not torch.equal(alone[0][0], alone[1][0])    # the two inputs differ


@pytest.mark.parametrize("limit", ["1", "3"])
def test_grid_in_several_launches(limit, monkeypatch):
    """Grids larger than one launch allows go out in several launches, each
    told its workgroup offset; GT_LAUNCH_BLOCKS lowers the limit so that a
    small graph takes that path (every kernel and every merge in 1- or
    3-workgroup launches).  Results are bitwise those of single launches."""
    P = I.make_problem(I.CONFIGS["tiny"])
    ip, ix = I.random_graph(21, 300, 280, _degrees(np.random.default_rng(21), 300, 280))
    Pb = I.small_problem(21, ip, ix, 280, 4, 32, "bf16", True)
    for prob, th in ((P, (2, 6, 4)), (Pb, (2, 8, 8)), (Pb, None)):
        monkeypatch.delenv("GT_LAUNCH_BLOCKS", raising=False)
        ref = run_gpu(prob, th)
        monkeypatch.setenv("GT_LAUNCH_BLOCKS", limit)
        got = run_gpu(prob, th)
        for x, y in zip(ref, got):
            if x is not None:
                assert torch.equal(x, y)
        check_full(prob, got)


def test_autograd_function_matches_abi():
    ip, ix = I.random_graph(11, 80, 80, np.random.default_rng(1).integers(1, 40, 80))
    P = I.small_problem(11, ip, ix, 80, 4, 32, "bf16", True)
    d = device_problem(P)
    g = T.gt_graph_prepare(d["indptr"], d["indices"], 80, 2, 8, 8)
    q, k, v, b = (d[n].clone().requires_grad_() for n in ("Q", "K", "V", "bias"))
    y = T.sparse_graph_attention(g, q, k, v, b)
    y.backward(d["dY"])
    ref = run_gpu(P, (2, 8, 8))
    assert torch.equal(y.detach(), ref[0])
    assert torch.equal(q.grad, ref[2]) and torch.equal(k.grad, ref[3])
    assert torch.equal(v.grad, ref[4]) and torch.equal(b.grad, ref[5])


@pytest.mark.parametrize("case", ["no_edges", "all_rows_empty_but_one", "no_columns"])
def test_degenerate_graphs(case):
    """Edge cases of the method: no edges at all (Y = 0, lse = -inf, all
    gradients 0), a single edge in a large graph, and a graph whose
    key/value side is empty (M = 0, so K, V, dK, dV have no rows)."""
    if case == "no_edges":
        R, M = 50, 40
        ip, ix = np.zeros(R + 1, np.int32), np.zeros(0, np.int32)
    elif case == "all_rows_empty_but_one":
        R, M = 300, 700
        ip, ix = I.csr_from_rows([[]] * 299 + [[123]], M)
    else:
        R, M = 20, 0
        ip, ix = np.zeros(R + 1, np.int32), np.zeros(0, np.int32)
    for dt, H, dh in (("f32", 2, 32), ("bf16", 4, 16)):
        P = I.small_problem(77, ip, ix, M, H, dh, dt, bias=(case != "no_columns"))
        out = run_gpu(P, (2, 4, 4))
        Y, lse, dQ, dK, dV, dB = out
        if case != "all_rows_empty_but_one":
            assert torch.all(Y == 0) and torch.all(dQ == 0)
            assert torch.all(torch.isneginf(lse))
            assert dK.numel() == M * H * dh and torch.all(dK == 0) and torch.all(dV == 0)
        else:
            check_full(P, out)
