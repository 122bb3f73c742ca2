"""Maximum sizes: arrays past 2^31 elements (and 4 GiB), nnz near the int32
limit of the CSR.

Inputs are periodic so that the oracle stays small while every element of
the large outputs is still checked:
  * attention: a circulant graph on n nodes, row i linking to (i + o_k) mod n
    for 24 offsets spread over the whole node range (inputs.circulant_*),
    with Q, K, V, dY periodic in the node index (period P = 64) and the bias
    periodic in (i mod P, k).  Every output is then periodic and equals the
    oracle's on the P-node circulant graph with offsets o_k mod P (the same
    edges, features and bias; only the order of each softmax sum differs).
    At n = 24 * 2^20, H = 4, dh = 32, bf16: Q, K, V, dY and the outputs hold
    3.2e9 elements (6.4 GB) each, the bias and dbias 2.4e9 (9.7 GB), and
    nnz = 604M; at n = 89.5M, H = 1, dh = 16: nnz = 2,147,483,136, just
    below the int32 limit of the CSR.  The transpose is checked bit-exactly
    against its closed form (column j's sources are (j - o_k) mod n,
    ascending).
  * projections: X and the gradients periodic in the row (period P) at
    n = 2^24 + 2^18 rows of d = 128 (2.2e9 elements); Q, K, V, Z and dX are
    periodic, and dW = (n / P) times the oracle's product on one period.
    X and the gradients take values in {-1, 0, 1} (X's last row of each
    period 0), so every partial sum of dW is an integer below 2^24 and dW
    must be exact: periodic inputs make the rounding errors of a long
    float32 sum coherent (they grow with the rows per slot instead of as a
    random walk), and an exact comparison still catches a lost or doubled
    slot of rows, which a rounding tolerance at this length would not.
  * head repack: a periodic [n, 8, 16] bf16 tensor (4.4 GB), bit-exact.
Each output is reduced on the GPU to its elementwise minimum and maximum
over the periods; the one farther from the oracle, element by element, is
held to the usual bound (gpu_util), which then bounds every period.
"""
import gc

import numpy as np
import pytest
import torch

from graph_transformer_sparse_amd import gtattn as T
from graph_transformer_sparse_amd import inputs as I
from oracle import heads as OH
from oracle import layer as L
from oracle import oracle as O

from gpu_util import RTOL, assert_close, assert_lse, dev

pytestmark = pytest.mark.gpu

P = 64
BF = torch.bfloat16


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def period_extremes(t, period=P, chunk_elems=1 << 27):
    """Elementwise min and max of t [n, ...] over its n / period periods
    (float32, on t's device), as numpy float64 arrays [period, ...]."""
    v = t.reshape(t.shape[0] // period, period, *t.shape[1:])
    per = max(1, chunk_elems // max(1, v[0].numel()))
    mn = mx = None
    for c in v.split(per, 0):
        c = c.float()
        a, b = c.amin(0), c.amax(0)
        mn = a if mn is None else torch.minimum(mn, a)
        mx = b if mx is None else torch.maximum(mx, b)
    f = lambda x: x.cpu().numpy().astype(np.float64)
    return f(mn), f(mx)


def worst_of(t, ref, period=P):
    """Per element, whichever of the min and max over the periods is farther
    from ref: |x - ref| <= |worst - ref| for every period x."""
    mn, mx = period_extremes(t, period)
    ref = np.asarray(ref, np.float64)
    return np.where(np.abs(mn - ref) > np.abs(mx - ref), mn, mx)


def by_offset(dbias, slot, deg, row_block=1 << 20):
    """dbias [n*deg, H] in CSR order -> [n, deg, H] ordered by offset index
    k (slot gives k of every stored edge), on the device, in row blocks."""
    n = slot.numel() // deg
    H = dbias.shape[1]
    out = torch.empty((n, deg, H), dtype=dbias.dtype, device=dbias.device)
    d3 = dbias.view(n, deg, H)
    s2 = slot.view(n, deg)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        k = s2[r0:r1].long()[:, :, None].expand(-1, -1, H)
        out[r0:r1].scatter_(1, k, d3[r0:r1])
    return out


def check_transpose(g, indices, offsets, n, deg, col_block=1 << 20):
    """indptr_t, indices_t and perm of the circulant graph, bit-exact:
    column j has deg sources (j - o_k) mod n in ascending order, and perm[t]
    is the CSR id of the edge (indices_t[t], j), i.e. it lies in row
    indices_t[t] (ids i*deg .. i*deg + deg - 1) and its column is j."""
    dev_ = indices.device
    ipt = g.indptr_t
    assert torch.equal(ipt.long(), torch.arange(0, n + 1, device=dev_, dtype=torch.int64) * deg)
    o = torch.as_tensor(np.asarray(offsets, np.int64), device=dev_)
    it = g.indices_t.view(n, deg)
    pm = g.perm.view(n, deg)
    for c0 in range(0, n, col_block):
        c1 = min(n, c0 + col_block)
        j = torch.arange(c0, c1, device=dev_, dtype=torch.int64)
        src, _ = torch.sort((j[:, None] - o[None, :]) % n, dim=1)
        assert torch.equal(it[c0:c1].long(), src), f"indices_t differs in columns {c0}..{c1}"
        p = pm[c0:c1].long()
        assert torch.equal(p // deg, src), f"perm rows differ in columns {c0}..{c1}"
        assert torch.equal(indices[p.reshape(-1)].long().view(-1, deg), j[:, None].expand(-1, deg)), \
            f"perm columns differ in columns {c0}..{c1}"


def attention_case(n, deg, H, dh, seed, thresholds=None, device="cuda"):
    """Runs the periodic circulant problem through the library and checks
    every output against the oracle on one period."""
    D = H * dh
    o = I.circulant_offsets(seed, n, P, deg)
    Bt = I.edge_bias(seed, P * deg, H).reshape(P, deg, H)
    Qb, Kb, Vb, dYb = (I.features(seed, s, P, H, dh, "bf16") for s in (I.S_Q, I.S_K, I.S_V, I.S_DY))
    scale = dh ** -0.5

    # the oracle on one period
    ip_s, ix_s, sl_s, b_s = I.circulant_csr(P, o % P, Bt)
    ip_s, ix_s, sl_s, b_s = ip_s.numpy(), ix_s.numpy(), sl_s.numpy(), b_s.numpy()
    m = {}
    rY, rl = O.fwd(ip_s, ix_s, P, Qb, Kb, Vb, b_s, scale, mag=m)
    rQ, rK, rV, rB = O.bwd(ip_s, ix_s, P, Qb, Kb, Vb, dYb, b_s, scale, mag=m)
    rB_k = np.empty((P, deg, H))
    rB_k[np.repeat(np.arange(P), deg), sl_s.astype(np.int64)] = rB

    # the full problem on the device
    print(f"maxsize attention n={n} deg={deg} H={H} dh={dh} th={thresholds}: building", flush=True)
    indptr, indices, slot, bias = I.circulant_csr(n, o, Bt, device=device)
    rep = lambda a: dev(a, BF, device).repeat(n // P, 1, 1)
    Q, K, V, dY = rep(Qb), rep(Kb), rep(Vb), rep(dYb)
    g = T.gt_graph_prepare(indptr, indices, n, *(thresholds or ()))
    print("  prepared; checking the transpose", flush=True)
    check_transpose(g, indices, o, n, deg)
    Y, lse = T.gt_attn_fwd(g, Q, K, V, bias, scale)
    dQ, dK, dV, dB = T.gt_attn_bwd(g, Q, K, V, Y, lse, dY, bias, scale)
    torch.cuda.synchronize()
    print("  ran fwd + bwd; comparing", flush=True)
    rt = RTOL["bf16"]
    assert_close(worst_of(Y, rY), rY, rt, "Y", m["Y"])
    assert_lse(worst_of(lse, rl), rl, 1e-4)
    assert_close(worst_of(dQ, rQ), rQ, rt, "dQ", m["dQ"])
    assert_close(worst_of(dK, rK), rK, rt, "dK", m["dK"])
    assert_close(worst_of(dV, rV), rV, rt, "dV", m["dV"])
    dBk = by_offset(dB, slot, deg)
    assert_close(worst_of(dBk, rB_k).reshape(P * deg, H), rB_k.reshape(P * deg, H), rt,
                 "dbias", head_axis=1)
    return n * D


ATTN = {
    # node arrays of 3.2e9 elements, bias of 2.4e9, nnz 604M
    "elements": dict(n=24 << 20, deg=24, H=4, dh=32, gb=120),
    # nnz = 2,147,483,136, just below the int32 limit of the CSR
    "nnz": dict(n=1398101 * P, deg=24, H=1, dh=16, gb=140),
}


@pytest.mark.parametrize("th", [None, (8, 64, 64)], ids=["default", "wave_rows"])
@pytest.mark.parametrize("case", list(ATTN))
def test_attention_at_maximum_sizes(case, th):
    """wave_rows makes every row a wavefront item: on the nnz case that is
    89M wavefronts, a grid that has to go out in several launches."""
    c = ATTN[case]
    n, deg, H, dh = c["n"], c["deg"], c["H"], c["dh"]
    assert n * deg < 2 ** 31 - 1
    if case == "elements":
        assert n * H * dh > 2 ** 31 and n * deg * H > 2 ** 31
    else:
        assert n * deg > 2 ** 31 - 2 ** 20
    free, _ = torch.cuda.mem_get_info()
    if free < c["gb"] << 30:
        pytest.skip(f"needs about {c['gb']} GB of device memory, {free >> 30} GB free")
    try:
        attention_case(n, deg, H, dh, seed=31, thresholds=th)
    finally:
        _free()


def projection_case(n, d, seed, device="cuda"):
    """Q, K, V, Z, dX and dW of periodic rows against the oracle on one period."""
    W = I.layer_inputs(seed, P, d, "bf16")[1]
    Xb, dZb, *Gb = (I.ternary(seed, s, (P, d)) for s in (I.S_X, I.S_DZ, I.S_Q, I.S_K, I.S_V))
    Xb[-1] = 0.0            # |sum over a period of x * g| <= P - 1 < 2^24 / (n / P)
    assert (n // P) * (P - 1) < 2 ** 24
    Yb = I.layer_inputs(seed + 4, P, d, "bf16")[2]
    rep = lambda a: dev(a, BF, device).repeat(n // P, 1)
    Wd = {k: dev(v, BF, device) for k, v in W.items()}
    rt = RTOL["bf16"]
    A = lambda x: np.abs(np.asarray(x, np.float64))
    X = rep(Xb)
    Q, K, V = T.gt_proj_qkv(X, Wd["q"], Wd["k"], Wd["v"])
    for got, ref, k in zip((Q, K, V), L.proj_qkv(Xb, W["q"], W["k"], W["v"]), "qkv"):
        assert_close(worst_of(got, ref), ref, rt, "XW" + k, A(Xb) @ A(W[k]))
    del Q, K, V
    Z = T.gt_proj_out(X, Wd["o"], rep(Yb))
    ref = L.proj_out(Xb, W["o"], Yb)
    assert_close(worst_of(Z, ref), ref, rt, "Z", A(Xb) @ A(W["o"]) + A(Yb))
    del Z
    dZ, G = rep(dZb), [rep(x) for x in Gb]
    dX = T.gt_proj_bwd_data(dZ, *G, Wd["o"], Wd["q"], Wd["k"], Wd["v"])
    ref = L.proj_bwd_data(dZb, *Gb, W["o"], W["q"], W["k"], W["v"])
    mag = sum(A(a) @ A(W[k]).T for a, k in zip((dZb, *Gb), "oqkv"))
    assert_close(worst_of(dX, ref), ref, rt, "dX", mag)
    del dX
    dW = T.gt_proj_bwd_weight(X, dZ, *G)
    reps = n // P
    for got, r, k in zip(dW, L.proj_bwd_weight(Xb, dZb, *Gb), "oqkv"):
        ref = reps * r
        assert np.all(np.abs(ref) < 2 ** 24) and np.array_equal(ref, np.round(ref))
        g = got.cpu().numpy().astype(np.float64)
        assert np.array_equal(g, ref), f"dW{k}: {int((g != ref).sum())} entries differ, " \
            f"max |diff| {np.abs(g - ref).max()}"


def test_projections_past_2_31_elements():
    n, d = (1 << 24) + (1 << 18), 128
    assert n * d > 2 ** 31 and n % P == 0
    free, _ = torch.cuda.mem_get_info()
    if free < 64 << 30:
        pytest.skip(f"needs about 64 GB of device memory, {free >> 30} GB free")
    print(f"maxsize projections n={n} d={d}", flush=True)
    try:
        projection_case(n, d, seed=41)
    finally:
        _free()


def repack_case(n, H, dh, parts, seed, device="cuda"):
    """Split and merge of a periodic bf16 tensor, bit-exact against the oracle."""
    xb = I.features(seed, I.S_Q, P, H, dh, "bf16")
    ref = OH.head_split(I.bf16_bits(xb).view(np.int16), parts)        # [parts, P, H/p, dh]
    x = dev(xb, BF, device).repeat(n // P, 1, 1)
    s = T.gt_head_split(x, parts)
    r = torch.from_numpy(np.ascontiguousarray(ref)).to(device)
    sv = s.view(torch.int16).view(parts, n // P, P, H // parts, dh)
    for c in sv.split(1 << 16, 1):
        assert torch.equal(c, r[:, None].expand_as(c))
    back = T.gt_head_merge(s)
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))


def test_head_repack_past_4_gib():
    n, H, dh, parts = (1 << 24) + (1 << 18), 8, 16, 2
    assert n * H * dh * 2 > 2 ** 32
    free, _ = torch.cuda.mem_get_info()
    if free < 24 << 30:
        pytest.skip(f"needs about 24 GB of device memory, {free >> 30} GB free")
    print(f"maxsize head repack n={n} H={H} dh={dh} parts={parts}", flush=True)
    try:
        repack_case(n, H, dh, parts, seed=51)
    finally:
        _free()
