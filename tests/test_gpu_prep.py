"""Graph preparation on the GPU is bit-exact with the oracle: the stable CSR
transpose (indptr_t, indices_t, perm), both degree-ordered schedules, and
the CSR validator's codes."""
import numpy as np
import pytest
import torch

from graph_transformer_sparse_amd import gtattn as T
from graph_transformer_sparse_amd import inputs as I
from oracle import oracle as O

from gpu_util import dev

pytestmark = pytest.mark.gpu


def _graphs():
    out = []
    rng = np.random.default_rng(0)
    for seed, (R, M, dmax, loops) in enumerate([(50, 50, 20, True), (200, 31, 31, False),
                                                (31, 300, 60, False), (1, 1, 1, True),
                                                (300, 300, 150, True)]):
        degs = rng.integers(0, dmax + 1, R)
        degs = np.minimum(degs, M)
        if loops:
            degs = np.maximum(degs, 1)
        out.append((f"rand{seed}", *I.random_graph(100 + seed, R, M, degs, self_loops=loops), M))
    # one hub row, one hub column, empty rows and columns
    rows = [[5]] * 40 + [list(range(0, 3000, 2))] + [[]] * 7 + [list(range(1500, 1510))]
    ip, ix = I.csr_from_rows(rows, 3000)
    out.append(("hubs", ip, ix, 3000))
    ip, ix = I.graph_for(I.CONFIGS["tiny"])
    out.append(("tiny", ip, ix, 2000))
    # edges only every 7000th row (thousands of empty rows between), one row
    # long enough to fill several 4096-edge tiles of the row-of-edge pass
    rows = [[] for _ in range(60000)]
    for r in range(0, 60000, 7000):
        rows[r] = [r % 900, 1000 + r % 7]
    rows[14000] = list(range(0, 9000))
    ip, ix = I.csr_from_rows(rows, 9000)
    out.append(("sparse_rows", ip, ix, 9000))
    return out


GRAPHS = _graphs()
THRESH = [(32, 2048, 2048), (2, 8, 8), (0, 0, 1), (4, 16, 5), (3, 3, 1000)]


ROW_CLASS = 4   # small rows of A are ordered by degree rounded down to a multiple of 4


def _check_sched(got, ptr, ts, tm, ch, cls=1):
    want = O.schedule(ptr, ts, tm, ch, cls)
    np.testing.assert_array_equal(got["order"].cpu().numpy(), want["order"])
    assert tuple(got["counts"]) == tuple(int(c) for c in want["counts"])
    np.testing.assert_array_equal(got["items"].cpu().numpy(), want["items"])
    np.testing.assert_array_equal(got["merges"].cpu().numpy(), want["merges"])
    # extents of the ordered segments, from the oracle's order and the CSR pointer
    o = np.asarray(want["order"], np.int64)
    np.testing.assert_array_equal(got["spans"].cpu().numpy(),
                                  np.stack([ptr[o], ptr[o + 1]], axis=1).reshape(-1, 2))
    assert got["max_degree"] == (int(np.max(np.diff(ptr))) if ptr.size > 1 else 0)


@pytest.mark.parametrize("gi", range(len(GRAPHS)), ids=[g[0] for g in GRAPHS])
@pytest.mark.parametrize("th", THRESH, ids=[str(t) for t in THRESH])
def test_transpose_and_schedules(gi, th):
    name, ip, ix, M = GRAPHS[gi]
    print(f"prep {name} {th}", flush=True)
    g = T.gt_graph_prepare(dev(ip), dev(ix), M, *th)
    torch.cuda.synchronize()
    pt, it, pm = O.transpose(ip, ix, M)
    np.testing.assert_array_equal(g.indptr_t.cpu().numpy(), pt)
    np.testing.assert_array_equal(g.indices_t.cpu().numpy(), it)
    np.testing.assert_array_equal(g.perm.cpu().numpy(), pm)
    _check_sched(g.schedule("rows"), ip, *th, ROW_CLASS)
    _check_sched(g.schedule("cols"), pt, *th)


def test_mid_config_prep():
    ip, ix = I.graph_for(I.CONFIGS["mid"])
    M = I.CONFIGS["mid"].n_cols
    print("prep mid", flush=True)
    g = T.gt_graph_prepare(dev(ip), dev(ix), M)
    pt, it, pm = O.transpose(ip, ix, M)
    np.testing.assert_array_equal(g.indptr_t.cpu().numpy(), pt)
    np.testing.assert_array_equal(g.indices_t.cpu().numpy(), it)
    np.testing.assert_array_equal(g.perm.cpu().numpy(), pm)
    ts, tm, ch = g.st.t_small, g.st.t_mid, g.st.chunk   # what prepare chose for this size
    assert (ts, tm, ch) == T.gt_graph_thresholds(ix.size)
    _check_sched(g.schedule("rows"), ip, ts, tm, ch, ROW_CLASS)
    _check_sched(g.schedule("cols"), pt, ts, tm, ch)


def test_empty_graph():
    ip = np.zeros(6, np.int32)
    ix = np.zeros(0, np.int32)
    g = T.gt_graph_prepare(dev(ip), dev(ix), 4, 2, 8, 8)
    np.testing.assert_array_equal(g.indptr_t.cpu().numpy(), np.zeros(5, np.int32))
    s = g.schedule("rows")
    assert s["counts"] == (0, 0, 5)
    np.testing.assert_array_equal(s["order"].cpu().numpy(), np.arange(5))


def test_validator_codes():
    ip, ix = I.csr_from_rows([[0, 2], [1], [], [0, 1, 3]], 4)
    cases = [
        (ip, ix),
        (ip, np.array([0, 2, 1, 0, 1, 4], np.int32)),          # out of range (3)
        (ip, np.array([0, 2, 1, 0, 3, 1], np.int32)),          # not ascending (4)
        (ip, np.array([2, 0, 1, 0, 9, 3], np.int32)),          # 4 at e=1 before 3 at e=4
        (ip, np.array([0, 7, 1, 1, 1, 3], np.int32)),          # 3 at e=1 before 4 at e=4
        (np.array([0, 2, 1, 3, 6], np.int32), ix),             # decreasing (2)
        (np.array([1, 2, 3, 3, 6], np.int32), ix),             # indptr[0] != 0 (1)
        (np.array([0, 2, 3, 3, 5], np.int32), ix),             # indptr[R] != nnz (1)
    ]
    for a, b in cases:
        want = O.csr_check(a, b, 4)
        got = T.gt_csr_validate(dev(a), dev(b), 4)
        assert got == want, (a, b, got, want)
    big_ip, big_ix = I.graph_for(I.CONFIGS["tiny"])
    assert T.gt_csr_validate(dev(big_ip), dev(big_ix), 2000) == 0


def test_prepare_validates_by_default():
    """The binding's prepare checks the CSR (unless validate=False) before any prep kernel
    runs and raises on a malformed graph; a valid one prepares as usual."""
    ip, ix = I.csr_from_rows([[0, 2], [1], [], [0, 1, 3]], 4)
    bad = np.array([0, 2, 1, 0, 1, 4], np.int32)           # a column out of range
    with pytest.raises(T.GTError):
        T.gt_graph_prepare(dev(ip), dev(bad), 4)
    g = T.gt_graph_prepare(dev(ip), dev(ix), 4, validate=True)
    assert g.nnz == ix.size


def test_tier_env_overrides(monkeypatch):
    """GT_TIER_SMALL / GT_TIER_MID / GT_TIER_CHUNK replace the schedule's
    defaults; explicit arguments still win."""
    ip, ix = I.csr_from_rows([[0, 2], [1], [], [0, 1, 3]], 4)
    monkeypatch.setenv("GT_TIER_SMALL", "1")
    monkeypatch.setenv("GT_TIER_MID", "2")
    monkeypatch.setenv("GT_TIER_CHUNK", "2")
    g = T.gt_graph_prepare(dev(ip), dev(ix), 4)
    assert (g.st.t_small, g.st.t_mid, g.st.chunk) == (1, 2, 2)
    _check_sched(g.schedule("rows"), ip, 1, 2, 2, ROW_CLASS)
    g = T.gt_graph_prepare(dev(ip), dev(ix), 4, 0, 8, 8)
    assert (g.st.t_small, g.st.t_mid, g.st.chunk) == (0, 8, 8)
