"""Seeded synthetic inputs: CSR graphs and dense node features.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds none of the attention arithmetic: it only draws random graphs and
random feature matrices and lays them out.

Stand-ins.  The pages measure on ogbn-arxiv/proteins/products and Reddit
(Scalable and Adaptive Parallel Training of Graph Transformer on Large
Graphs, Table 2 and Section 5.2).  Those datasets are not available, so
power-law and R-MAT generators of similar size and skew stand in for them.

Every array comes from ``np.random.default_rng([cfg, stream])`` (PCG64):
stream 0 draws the graph, 1 Q, 2 K, 3 V, 4 dY and 5 the per-edge bias.

Graph conventions (the adjacency A of the SGA definition, Section 2.1 of
the paper): row i is the query / destination node, column j the key/value
source node, A is a 0/1 pattern stored as CSR (int32 indptr and indices),
the columns of every row strictly ascending, and every row r < n_rows has
the self-loop (r, r).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# stream ids of the seeded generators
S_GRAPH, S_Q, S_K, S_V, S_DY, S_BIAS = 0, 1, 2, 3, 4, 5
S_X, S_WQ, S_WK, S_WV, S_WO, S_DZ = 6, 7, 8, 9, 10, 11


@dataclass(frozen=True)
class Config:
    name: str
    idx: int           # seed component
    n_rows: int        # R: query rows (destination nodes)
    n_cols: int        # M: key/value rows (source nodes)
    heads: int
    head_dim: int
    dtype: str         # "f32" or "bf16"
    bias: bool
    desc: str = field(default="", compare=False)


CONFIGS = {
    "tiny": Config("tiny", 0, 2000, 2000, 1, 64, "f32", False,
                   "Erdos-Renyi directed, mean out-degree 8, self-loops"),
    "mid": Config("mid", 1, 131072, 131072, 8, 16, "f32", False,
                  "R-MAT (0.57,0.19,0.19,0.05), 14 draws per node, self-loops"),
    "large": Config("large", 2, 1 << 20, 1 << 20, 8, 32, "bf16", False,
                    "Chung-Lu exponent 2.1, mean 16, max weight 50000, self-loops"),
    "hub": Config("hub", 3, 2_400_000, 2_400_000, 4, 32, "bf16", True,
                  "Chung-Lu exponent 1.9, 62M nnz, per-edge bias"),
    "shard": Config("shard", 4, 524288, 4194304, 8, 16, "bf16", False,
                    "rank-0 row block of a relabelled R-MAT graph on 2^22 nodes"),
}
CONFIG_ORDER = ["tiny", "mid", "large", "hub", "shard"]


def rng_for(cfg_idx: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([cfg_idx, stream])


# ----------------------------------------------------------------------------
# CSR assembly
# ----------------------------------------------------------------------------

def csr_from_pairs(rows, cols, n_rows: int, n_cols: int, self_loops: bool = True):
    """Deduplicate (row, col) pairs, add self-loops, and return int32 CSR.

    The result has strictly ascending columns within every row.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    keys = rows * n_cols + cols
    if self_loops:
        loops = np.arange(min(n_rows, n_cols), dtype=np.int64)
        keys = np.concatenate([keys, loops * n_cols + loops])
    keys = np.unique(keys)
    r = keys // n_cols
    c = keys - r * n_cols
    counts = np.bincount(r, minlength=n_rows)
    indptr = np.zeros(n_rows + 1, dtype=np.int64)
    np.cumsum(counts, out=indptr[1:])
    assert indptr[-1] < 2**31
    return indptr.astype(np.int32), c.astype(np.int32)


def csr_from_rows(row_lists, n_cols: int):
    """CSR from explicit per-row column lists (sorted, deduplicated here)."""
    indptr = [0]
    idx = []
    for cols in row_lists:
        u = sorted(set(int(c) for c in cols))
        assert all(0 <= c < n_cols for c in u)
        idx.extend(u)
        indptr.append(len(idx))
    return np.asarray(indptr, dtype=np.int32), np.asarray(idx, dtype=np.int32)


# ----------------------------------------------------------------------------
# graph families
# ----------------------------------------------------------------------------

def gnp_directed(n: int, mean_deg: float, rng) -> tuple:
    """Directed G(n, p) over ordered pairs i != j with p = mean_deg / (n - 1)."""
    p = mean_deg / (n - 1)
    rows, cols = [], []
    step = max(1, (1 << 22) // n)
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        hit = rng.random((r1 - r0, n)) < p
        rr, cc = np.nonzero(hit)
        rr = rr + r0
        keep = rr != cc
        rows.append(rr[keep])
        cols.append(cc[keep])
    return np.concatenate(rows), np.concatenate(cols)


RMAT_ABCD = (0.57, 0.19, 0.19, 0.05)


def rmat_pairs(levels: int, n_draws: int, rng, batch: int = 1 << 22):
    """R-MAT draws: per level one uniform u picks quadrant a/b/c/d for
    (row bit, col bit), most significant bit first."""
    a, b, c, _ = RMAT_ABCD
    t_ab, t_abc = a + b, a + b + c
    rows = np.empty(n_draws, dtype=np.int64)
    cols = np.empty(n_draws, dtype=np.int64)
    for s in range(0, n_draws, batch):
        m = min(batch, n_draws - s)
        r = np.zeros(m, dtype=np.int64)
        cc = np.zeros(m, dtype=np.int64)
        for _ in range(levels):
            u = rng.random(m, dtype=np.float32)
            rb = u >= np.float32(t_ab)                    # quadrants c, d
            cb = ((u >= np.float32(a)) & ~rb) | (u >= np.float32(t_abc))  # b, d
            r = (r << 1) | rb
            cc = (cc << 1) | cb
        rows[s:s + m] = r
        cols[s:s + m] = cc
    return rows, cols


def chung_lu_weights(n: int, alpha: float, x_min: float, w_max: float, rng):
    u = 1.0 - rng.random(n)            # (0, 1]
    return np.minimum(x_min * u ** (-1.0 / alpha), w_max)


def _bisect_xmin(u, alpha, w_max, mean):
    lo, hi = 1e-3, float(mean)
    for _ in range(100):
        mid = 0.5 * (lo + hi)
        m = np.minimum(mid * u ** (-1.0 / alpha), w_max).mean()
        if m < mean:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw_by_weight(cdf, m, rng):
    """m indices drawn with probability proportional to the weights whose
    running sum is cdf (inverse-CDF sampling).  Each slice of the queries is
    searched in sorted order (same indices as searching them as drawn, with
    cache-friendly access), slices in parallel threads."""
    q = rng.random(m) * cdf[-1]
    out = np.empty(m, dtype=np.int64)
    nt = _workers()
    cuts = np.linspace(0, m, 4 * nt + 1).astype(np.int64)

    def one(k):
        sl = slice(int(cuts[k]), int(cuts[k + 1]))
        qq = q[sl]
        o = np.argsort(qq)
        r = np.empty(qq.size, dtype=np.int64)
        r[o] = np.searchsorted(cdf, qq[o], side="right")
        out[sl] = r

    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(one, range(4 * nt)))
    return out


def _chung_lu_distinct(cdf, n_cols, need, rng, batch=20_000_000):
    """The first `need` distinct directed edges (i != j) in draw order, with
    row and column both drawn proportional to the weights, in batches; returned
    as int64 keys i * n_cols + j (as a set: all but the last batch sorted).

    Draw order only decides which edges of the last batch are cut at `need`,
    so earlier batches are merged as sorted sets and only the last one is
    put in first-draw order."""
    kept = np.empty(0, dtype=np.int64)          # sorted set of the edges kept so far
    tail = np.empty(0, dtype=np.int64)
    while kept.size + tail.size < need:
        rows = _draw_by_weight(cdf, batch, rng)
        cols = _draw_by_weight(cdf, batch, rng)
        keys = rows * n_cols + cols
        keys = keys[rows != cols]
        new = np.unique(keys)
        if kept.size:
            pos = np.searchsorted(kept, new)
            pos[pos == kept.size] = 0
            new = new[kept[pos] != new]
        if kept.size + new.size <= need:
            kept = np.sort(np.concatenate([kept, new]))
            continue
        # last batch: distinct new edges in first-draw order, cut at `need`
        _, first = np.unique(keys, return_index=True)
        keys = keys[np.sort(first)]
        pos = np.searchsorted(kept, keys)
        pos[pos == kept.size] = 0
        keys = keys[kept[pos] != keys] if kept.size else keys
        tail = keys[: need - kept.size]
    return np.concatenate([kept, tail])


def hub_graph(n: int, target: int, rng, batch: int = 20_000_000):
    """Chung-Lu, exponent 1.9 (weights u^(-1/0.9), capped at n - 1), with
    exactly `target` stored nonzeros: target - n distinct non-loop edges in
    first-draw order, then a self-loop on every node."""
    w = chung_lu_weights(n, 0.9, 1.0, float(n - 1), rng)
    kept = _chung_lu_distinct(np.cumsum(w), n, target - n, rng, batch)
    r = kept // n
    c = kept - r * n
    ip, ix = csr_from_pairs(r, c, n, n)
    assert ix.size == target, ix.size
    return ip, ix


def graph_for(cfg: Config):
    """(indptr, indices) int32 for one of the named configurations."""
    rng = rng_for(cfg.idx, S_GRAPH)
    R, M = cfg.n_rows, cfg.n_cols
    if cfg.name == "tiny":
        rows, cols = gnp_directed(R, 8.0, rng)
        return csr_from_pairs(rows, cols, R, M)
    if cfg.name == "mid":
        # 2^17 nodes as configured; other powers of two give the same recipe
        # at another node count
        levels = int(R).bit_length() - 1
        assert R == M == 1 << levels, "the R-MAT recipe needs a power-of-two node count"
        rows, cols = rmat_pairs(levels, 14 * R, rng)
        return csr_from_pairs(rows, cols, R, M)
    if cfg.name == "large":
        u = 1.0 - rng.random(R)
        xmin = _bisect_xmin(u, 1.1, 50000.0, 16.0)
        w = np.minimum(xmin * u ** (-1.0 / 1.1), 50000.0)
        cdf = np.cumsum(w)
        n = int(round(cdf[-1]))
        rows = _draw_by_weight(cdf, n, rng)
        cols = _draw_by_weight(cdf, n, rng)
        keep = rows != cols
        return csr_from_pairs(rows[keep], cols[keep], R, M)
    if cfg.name == "hub":
        return hub_graph(R, 62_000_000, rng)
    if cfg.name == "shard":
        n_glob = 1 << 22
        perm = rng.permutation(n_glob)
        rows_all, cols_all = [], []
        n_draws = 32 * n_glob
        batch = 1 << 23
        for s in range(0, n_draws, batch):
            m = min(batch, n_draws - s)
            r, c = rmat_pairs(22, m, rng)
            r = perm[r]
            c = perm[c]
            keep = r < R
            rows_all.append(r[keep])
            cols_all.append(c[keep])
        return csr_from_pairs(np.concatenate(rows_all), np.concatenate(cols_all), R, M)
    raise KeyError(cfg.name)


# ----------------------------------------------------------------------------
# features
# ----------------------------------------------------------------------------

def to_bf16_values(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even) and return the bf16
    values widened back to float32, exactly.  NaN/Inf are not produced by the
    generators, so the plain rounding rule on the bit pattern applies."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).reshape(x32.shape)


def bf16_bits(x_bf16_values: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exact bf16 values."""
    u = np.ascontiguousarray(x_bf16_values, dtype=np.float32).view(np.uint32)
    assert not np.any(u & 0xFFFF)
    return (u >> 16).astype(np.uint16)


def features(cfg_idx: int, stream: int, n: int, heads: int, head_dim: int, dtype: str):
    """[n, heads, head_dim] standard normal features.  Returned as float32
    holding exactly the values of the requested dtype (bf16 is rounded)."""
    x = rng_for(cfg_idx, stream).standard_normal((n, heads, head_dim), dtype=np.float32)
    if dtype == "bf16":
        x = to_bf16_values(x)
    return x


def edge_bias(cfg_idx: int, nnz: int, heads: int):
    """[nnz, heads] float32 ~ N(0, variance 0.5), in CSR edge order."""
    return rng_for(cfg_idx, S_BIAS).normal(0.0, np.sqrt(0.5), (nnz, heads)).astype(np.float32)


@dataclass
class Problem:
    cfg: Config
    indptr: np.ndarray
    indices: np.ndarray
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    dY: np.ndarray
    bias: np.ndarray | None

    @property
    def nnz(self) -> int:
        return int(self.indices.size)

    @property
    def scale(self) -> float:
        return float(self.cfg.head_dim) ** -0.5


def _cache_dir():
    d = os.environ.get("GT_INPUT_CACHE")
    return d if d else None


_GRAPHS = {}   # the named graphs generated in this process


def named_graph(cfg: Config):
    """graph_for(cfg), generated once per process (and read from / written
    to the directory GT_INPUT_CACHE names, if set)."""
    # the graph depends on the recipe (name) and the node counts only
    named = CONFIGS.get(cfg.name)
    same = named is not None and (named.n_rows, named.n_cols) == (cfg.n_rows, cfg.n_cols)
    key = cfg.name if same else f"{cfg.name}_{cfg.n_rows}x{cfg.n_cols}"
    if key in _GRAPHS:
        return _GRAPHS[key]
    cache = _cache_dir()
    path = os.path.join(cache, f"graph_{key}.npz") if cache else None
    if path and os.path.exists(path):
        with np.load(path) as z:
            graph = (z["indptr"], z["indices"])
    else:
        graph = graph_for(cfg)
        if path:
            os.makedirs(cache, exist_ok=True)
            tmp = path + ".tmp.npz"
            np.savez(tmp, indptr=graph[0], indices=graph[1])
            os.replace(tmp, path)
    _GRAPHS[key] = graph
    return graph


def make_problem(cfg: Config, graph=None) -> Problem:
    """All inputs of one configuration.  ``graph`` overrides the graph."""
    indptr, indices = named_graph(cfg) if graph is None else graph
    H, dh = cfg.heads, cfg.head_dim
    Q = features(cfg.idx, S_Q, cfg.n_rows, H, dh, cfg.dtype)
    K = features(cfg.idx, S_K, cfg.n_cols, H, dh, cfg.dtype)
    V = features(cfg.idx, S_V, cfg.n_cols, H, dh, cfg.dtype)
    dY = features(cfg.idx, S_DY, cfg.n_rows, H, dh, cfg.dtype)
    bias = edge_bias(cfg.idx, int(indices.size), H) if cfg.bias else None
    return Problem(cfg, indptr, indices, Q, K, V, dY, bias)


def small_problem(seed: int, indptr, indices, n_cols: int, heads: int, head_dim: int,
                  dtype: str = "f32", bias: bool = False, name: str = "small") -> Problem:
    """Inputs for an explicit small graph (tests)."""
    R = int(indptr.size - 1)
    cfg = Config(name, 1000 + seed, R, n_cols, heads, head_dim, dtype, bias)
    return make_problem(cfg, graph=(np.asarray(indptr, np.int32), np.asarray(indices, np.int32)))


def random_graph(seed: int, n_rows: int, n_cols: int, degrees, self_loops: bool = True):
    """CSR whose row r has exactly degrees[r] distinct columns (including the
    self-loop when self_loops and r < n_cols).  Columns are uniform without
    replacement."""
    rng = np.random.default_rng([2000 + seed, S_GRAPH])
    rows = []
    for r in range(n_rows):
        d = int(degrees[r])
        assert d <= n_cols
        if self_loops and r < n_cols and d > 0:
            others = np.delete(np.arange(n_cols), r)
            pick = rng.choice(others, size=d - 1, replace=False)
            cols = np.concatenate([[r], pick])
        else:
            cols = rng.choice(n_cols, size=d, replace=False)
        rows.append(cols)
    return csr_from_rows(rows, n_cols)


# ----------------------------------------------------------------------------
# inputs of a whole layer (node features, projection weights, output gradient)
# ----------------------------------------------------------------------------

def layer_inputs(cfg_idx: int, n: int, d: int, dtype: str):
    """X [n, d] and dZ [n, d] ~ N(0, 1); weights W_q, W_k, W_v, W_o [d, d]
    ~ N(0, 1/d) (so a projection of unit-variance features has unit
    variance).  float32 arrays holding exactly the values of ``dtype``."""
    def draw(stream, shape, std):
        x = rng_for(cfg_idx, stream).normal(0.0, std, shape).astype(np.float32)
        return to_bf16_values(x) if dtype == "bf16" else x
    X = draw(S_X, (n, d), 1.0)
    W = {k: draw(s, (d, d), d ** -0.5) for k, s in (("q", S_WQ), ("k", S_WK), ("v", S_WV), ("o", S_WO))}
    dZ = draw(S_DZ, (n, d), 1.0)
    return X, W, dZ


# ---------------------------------------------------------------------------
# periodic circulant problems (tests at the maximum sizes)
# ---------------------------------------------------------------------------
def circulant_offsets(seed: int, n: int, period: int, degree: int) -> np.ndarray:
    """Offsets o_0 = 0, o_1 .. o_{degree-1} of a circulant graph on n nodes
    (row i links to (i + o_k) mod n; n a multiple of `period`, degree <=
    period).  The residues o_k mod period are distinct (0, then degree - 1
    drawn without replacement) and each gets a multiple of the period drawn
    over [0, n), so a row's edges reach across the whole node range.  With
    features periodic in the node index, every output of the graph is then
    periodic too, and equals that of the `period`-node circulant graph with
    offsets o_k mod period."""
    assert n % period == 0 and 1 <= degree <= min(period, 255)
    rng = rng_for(seed, S_GRAPH)
    res = np.concatenate([[0], rng.choice(np.arange(1, period), degree - 1, replace=False)])
    mult = np.concatenate([[0], rng.integers(0, n // period, degree - 1)])
    return (res + period * mult).astype(np.int64)


def circulant_csr(n: int, offsets, bias_table=None, device="cpu", row_block: int = 1 << 20):
    """The circulant graph on n nodes as CSR torch tensors on `device`: row i
    holds the columns (i + o_k) mod n in ascending order.  Returns (indptr
    int32 [n+1], indices int32 [n*deg], slot uint8 [n*deg] = the offset index
    k of each stored edge, bias float32 [n*deg, H] = bias_table[i mod P, k]
    (P = bias_table.shape[0]) or None).  Built in blocks of rows."""
    import torch
    o = torch.as_tensor(np.asarray(offsets, np.int64), device=device)
    deg = int(o.numel())
    assert len(set(int(x) % n for x in np.asarray(offsets))) == deg, "offsets collide mod n"
    indptr = torch.arange(0, n + 1, dtype=torch.int64, device=device).mul_(deg).to(torch.int32)
    indices = torch.empty(n * deg, dtype=torch.int32, device=device)
    slot = torch.empty(n * deg, dtype=torch.uint8, device=device)
    bias = None
    if bias_table is not None:
        bt = torch.as_tensor(np.ascontiguousarray(bias_table, np.float32), device=device)
        per, H = bt.shape[0], bt.shape[2]
        bias = torch.empty((n * deg, H), dtype=torch.float32, device=device)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        rows = torch.arange(r0, r1, dtype=torch.int64, device=device)
        cols, k = torch.sort((rows[:, None] + o[None, :]) % n, dim=1)
        indices[r0 * deg:r1 * deg] = cols.reshape(-1).to(torch.int32)
        slot[r0 * deg:r1 * deg] = k.reshape(-1).to(torch.uint8)
        if bias is not None:
            b = bt[rows % per]                                   # [rows, deg, H] by offset
            bias[r0 * deg:r1 * deg] = torch.gather(b, 1, k[:, :, None].expand(-1, -1, H)).reshape(-1, H)
    return indptr, indices, slot, bias


def ternary(seed: int, stream: int, shape) -> np.ndarray:
    """Values drawn uniformly from {-1, 0, 1} as float32 (exact in bf16):
    products and sums of them stay integers, exact in float32 below 2^24."""
    return rng_for(seed, stream).integers(-1, 2, shape).astype(np.float32)
