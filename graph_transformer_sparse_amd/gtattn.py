"""Python binding of libgtattn (include/gt_attn.h), through ctypes.

Argument marshalling only: tensors are allocated with torch on the current
device, their pointers and the current HIP stream go to the C ABI, and every
step of the computation runs in the library's kernels.  If the library has
not been built, every entry point raises; there is no fallback.

Names follow the C ABI: gt_graph_prepare, gt_attn_fwd, gt_attn_bwd,
gt_attn_work_bytes, gt_csr_validate, gt_default_thresholds, gt_graph_thresholds, plus the
autograd wrapper GTAttnFn / sparse_graph_attention.
"""
from __future__ import annotations

import ctypes as C
import math
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_build", "libgtattn.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

GT_OK = 0
GT_F32, GT_BF16 = 0, 1
GT_VALIDATE_WORK_BYTES = 64
STATUS = {0: "GT_OK", 1: "GT_E_NULL", 2: "GT_E_ARG", 3: "GT_E_DTYPE", 4: "GT_E_SHAPE",
          5: "GT_E_ALIGN", 6: "GT_E_UNSUPPORTED", 7: "GT_E_WORKSPACE", 8: "GT_E_CSR",
          9: "GT_E_HIP"}

_i64, _i32, _P, _f32, _sz = C.c_int64, C.c_int32, C.c_void_p, C.c_float, C.c_size_t


class GtSched(C.Structure):
    _fields_ = [("order", _P), ("items", _P), ("merges", _P), ("spans", _P),
                ("n_seg", _i64), ("n_big", _i64), ("n_mid", _i64), ("n_small", _i64),
                ("n_items", _i64), ("n_merges", _i64), ("max_degree", _i64)]


class GtGraph(C.Structure):
    _fields_ = [("n_rows", _i64), ("n_cols", _i64), ("nnz", _i64),
                ("indptr", _P), ("indices", _P),
                ("indptr_t", _P), ("indices_t", _P), ("perm", _P),
                ("rows", GtSched), ("cols", GtSched),
                ("t_small", _i32), ("t_mid", _i32), ("chunk", _i32), ("reserved", _i32)]


class GTError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")
        self.status = status


_lib = None


def header_functions() -> list[str]:
    """Names of the functions the headers in include/ declare."""
    names = set()
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, f)).read(), flags=re.S)
            names.update(re.findall(r"\b(gt_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with graph_transformer_sparse_amd.build")
    L = C.CDLL(LIB_PATH)
    G = C.POINTER(GtGraph)
    sig = {
        "gt_graph_meta_bytes": (_sz, [_i64, _i64, _i64, _i32]),
        "gt_graph_prepare": (_i32, [_P, _P, _i64, _i64, _i64, _i32, _i32, _i32, _P, _sz, G, _P]),
        "gt_default_thresholds": (None, [C.POINTER(_i32)] * 3),
        "gt_graph_thresholds": (None, [_i64] + [C.POINTER(_i32)] * 3),
        "gt_csr_validate": (_i32, [_P, _P, _i64, _i64, _i64, _P, _sz, C.POINTER(_i32), _P]),
        "gt_attn_work_bytes": (_sz, [G, _i32, _i32]),
        "gt_attn_fwd": (_i32, [G, _i32, _i32, _i32, _f32, _P, _P, _P, _P, _P, _P, _P, _sz, _P]),
        "gt_attn_fwd_noalloc": (_i32, [G, _i32, _i32, _i32, _f32, _P, _P, _P, _P, _P, _P, _P]),
        "gt_attn_bwd": (_i32, [G, _i32, _i32, _i32, _f32, _P, _P, _P, _P, _P, _P, _P,
                               _P, _P, _P, _P, _P, _sz, _P]),
        "gt_prof_enable": (_i32, [_i32]),
        "gt_prof_reset": (_i32, []),
        "gt_prof_query": (_i32, [C.c_char_p, C.POINTER(C.c_double), C.POINTER(_i64)]),
        "gt_head_split": (_i32, [_i64, _i32, _i32, _i32, _P, _P, _P]),
        "gt_head_merge": (_i32, [_i64, _i32, _i32, _i32, _P, _P, _P]),
        "gt_status_str": (C.c_char_p, [_i32]),
        "gt_last_error": (C.c_char_p, []),
        "gt_version": (_i32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int, where: str):
    if status != GT_OK:
        raise GTError(status, where, lib().gt_last_error().decode())


def _ptr(t):
    # a plain int: ctypes converts it for c_void_p parameters
    return None if t is None else t.data_ptr()


def _stream(device=None):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dt(dtype) -> int:
    if dtype == torch.float32:
        return GT_F32
    if dtype == torch.bfloat16:
        return GT_BF16
    raise TypeError(f"unsupported dtype {dtype}")


def _need(cond: bool, where: str, msg):
    """Raise ValueError(where: msg) unless cond; msg may be a callable, so
    that the text is only built on failure (these checks run on every call)."""
    if not cond:
        raise ValueError(f"{where}: {msg() if callable(msg) else msg}")


def _tensor(where: str, name: str, t, shape, dtype, device):
    """Check that t is a contiguous tensor of this shape, dtype and device.
    The C ABI gets only pointers: a wrongly sized array would be read or
    written out of bounds on the GPU, so sizes are checked here."""
    if (isinstance(t, torch.Tensor) and t.shape == shape and t.dtype == dtype
            and t.device == device and t.is_contiguous()):
        return
    _need(isinstance(t, torch.Tensor), where, f"{name} must be a tensor")
    _need(tuple(t.shape) == tuple(shape), where,
          f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    _need(t.dtype == dtype, where, f"{name} has dtype {t.dtype}, expected {dtype}")
    _need(t.device == device, where, f"{name} is on {t.device}, expected {device}")
    _need(t.is_contiguous(), where, f"{name} must be contiguous")


def _attn_shapes(where: str, g: "Graph", Q, K, V, bias):
    """(R, H, dh, dtype, device) of the attention inputs, checked against the
    prepared graph."""
    _need(isinstance(Q, torch.Tensor) and Q.dim() == 3, where, "Q must be a [rows, heads, "
          "head_dim] tensor")
    R, H, dh = Q.shape
    dt, dev = Q.dtype, Q.device
    _need(dt in (torch.float32, torch.bfloat16), where, lambda: f"unsupported dtype {dt}")
    _tensor(where, "Q", Q, (g.n_rows, H, dh), dt, dev)
    _tensor(where, "K", K, (g.n_cols, H, dh), dt, dev)
    _tensor(where, "V", V, (g.n_cols, H, dh), dt, dev)
    if bias is not None:
        _tensor(where, "bias", bias, (g.nnz, H), torch.float32, dev)
    return R, H, dh, dt, dev


def _on_gpu(where: str, g: "Graph", dev):
    _need(dev.type == "cuda", where, lambda: f"tensors must be on a GPU, not {dev}")
    _need(g.meta.device == dev, where,
          lambda: f"the graph is on {g.meta.device}, the tensors on {dev}")


def gt_default_thresholds():
    a, b, c = _i32(), _i32(), _i32()
    lib().gt_default_thresholds(C.byref(a), C.byref(b), C.byref(c))
    return a.value, b.value, c.value


def gt_graph_thresholds(nnz: int):
    """(t_small, t_mid, chunk) tuned for a graph of nnz nonzeros."""
    a, b, c = _i32(), _i32(), _i32()
    lib().gt_graph_thresholds(int(nnz), C.byref(a), C.byref(b), C.byref(c))
    return a.value, b.value, c.value


class Graph:
    """A CSR adjacency prepared for attention (transpose and schedules).

    Holds the device CSR, the meta buffer and the filled gt_graph struct."""

    def __init__(self, st: GtGraph, meta: torch.Tensor, indptr: torch.Tensor,
                 indices: torch.Tensor):
        self.st = st
        self.meta = meta
        self.indptr = indptr
        self.indices = indices
        # plain copies of the sizes (read on every call) and the work sizes
        # asked for so far, per (heads, head_dim)
        self.n_rows, self.n_cols, self.nnz = int(st.n_rows), int(st.n_cols), int(st.nnz)
        self._work_bytes = {}

    def _view(self, ptr: int, n: int) -> torch.Tensor:
        base = self.meta.data_ptr()
        off = ptr - base
        if off % 4 or off < 0 or off + 4 * n > self.meta.numel():
            raise RuntimeError("graph struct points outside its meta buffer")
        return self.meta.view(torch.int32)[off // 4: off // 4 + n]

    @property
    def indptr_t(self):
        return self._view(self.st.indptr_t, self.n_cols + 1)

    @property
    def indices_t(self):
        return self._view(self.st.indices_t, self.nnz)

    @property
    def perm(self):
        return self._view(self.st.perm, self.nnz)

    def schedule(self, which: str) -> dict:
        s = self.st.rows if which == "rows" else self.st.cols
        return dict(order=self._view(s.order, s.n_seg),
                    counts=(s.n_big, s.n_mid, s.n_small),
                    items=self._view(s.items, 4 * s.n_items).view(-1, 4),
                    merges=self._view(s.merges, 3 * s.n_merges).view(-1, 3),
                    spans=self._view(s.spans, 2 * s.n_seg).view(-1, 2),
                    max_degree=s.max_degree)


def gt_graph_prepare(indptr: torch.Tensor, indices: torch.Tensor, n_cols: int,
                     t_small: int | None = None, t_mid: int | None = None,
                     chunk: int | None = None, validate: bool = True) -> Graph:
    """Prepare a device CSR (int32 indptr/indices) for attention.  The CSR
    content is checked on the GPU first (gt_csr_validate: row pointer
    monotone and consistent, every column in [0, n_cols), columns strictly
    ascending in each row), and a malformed graph raises GTError instead of
    reaching the kernels, whose gathers trust the column indices.  A caller
    that has already checked the graph may pass validate=False."""
    L = lib()
    # tuning overrides of the schedule's defaults (GT_TIER_SMALL, GT_TIER_MID,
    # GT_TIER_CHUNK); explicit arguments win
    env = lambda k: int(os.environ[k]) if os.environ.get(k) else None
    t_small = env("GT_TIER_SMALL") if t_small is None else t_small
    t_mid = env("GT_TIER_MID") if t_mid is None else t_mid
    chunk = env("GT_TIER_CHUNK") if chunk is None else chunk
    d_small, d_mid, d_chunk = gt_graph_thresholds(indices.numel())
    t_small = d_small if t_small is None else t_small
    t_mid = d_mid if t_mid is None else t_mid
    chunk = d_chunk if chunk is None else chunk
    where = "gt_graph_prepare"
    for name, t in (("indptr", indptr), ("indices", indices)):
        _need(isinstance(t, torch.Tensor) and t.dim() == 1, where, f"{name} must be a 1-D tensor")
        _need(t.dtype == torch.int32, where, f"{name} must be int32, not {t.dtype}")
        _need(t.is_contiguous(), where, f"{name} must be contiguous")
    _need(indptr.numel() >= 1, where, "indptr needs n_rows + 1 >= 1 entries")
    _need(indptr.device.type == "cuda" and indices.device == indptr.device, where,
          "indptr and indices must be on the same GPU")
    R, E = indptr.numel() - 1, indices.numel()
    if validate:
        code = gt_csr_validate(indptr, indices, n_cols)
        if code != 0:
            raise GTError(8, "gt_graph_prepare", f"malformed CSR (gt_csr_validate code {code})")
    nb = L.gt_graph_meta_bytes(R, n_cols, E, chunk)
    if nb == 0:
        raise GTError(2, "gt_graph_meta_bytes", "sizes out of range")
    meta = torch.empty(nb, dtype=torch.uint8, device=indptr.device)
    st = GtGraph()
    _check(L.gt_graph_prepare(_ptr(indptr), _ptr(indices) if E else None, R, n_cols, E,
                              t_small, t_mid, chunk, _ptr(meta), nb, C.byref(st),
                              _stream(indptr.device)), "gt_graph_prepare")
    return Graph(st, meta, indptr, indices)


def gt_csr_validate(indptr: torch.Tensor, indices: torch.Tensor, n_cols: int) -> int:
    """The CSR check code (0 valid, 1-4 as gt_attn.h)."""
    work = torch.empty(GT_VALIDATE_WORK_BYTES, dtype=torch.uint8, device=indptr.device)
    code = _i32(-1)
    st = lib().gt_csr_validate(_ptr(indptr), _ptr(indices) if indices.numel() else None,
                               indptr.numel() - 1, n_cols, indices.numel(), _ptr(work),
                               GT_VALIDATE_WORK_BYTES, C.byref(code), _stream(indptr.device))
    if st not in (GT_OK, 8):
        _check(st, "gt_csr_validate")
    return code.value


def gt_attn_work_bytes(g: Graph, heads: int, head_dim: int) -> int:
    key = (heads, head_dim)
    nb = g._work_bytes.get(key)
    if nb is None:
        nb = g._work_bytes[key] = int(lib().gt_attn_work_bytes(C.byref(g.st), heads, head_dim))
    return nb


def _work(g, heads, head_dim, device, work):
    nb = gt_attn_work_bytes(g, heads, head_dim)
    if work is not None:
        _need(work.dtype == torch.uint8 and work.device == device and work.is_contiguous(),
              "work", "work must be a contiguous uint8 tensor on the inputs' device")
    if work is None or work.numel() < nb:
        work = torch.empty(nb, dtype=torch.uint8, device=device)
    return work


def gt_attn_fwd(g: Graph, Q, K, V, bias=None, scale=None, work=None, Y=None, lse=None):
    """Forward: returns (Y, lse).  Q [R,H,dh], K/V [M,H,dh] (f32 or bf16)."""
    R, H, dh, dt, dev = _attn_shapes("gt_attn_fwd", g, Q, K, V, bias)
    scale = dh ** -0.5 if scale is None else float(scale)
    Y = torch.empty_like(Q) if Y is None else Y
    lse = torch.empty((R, H), dtype=torch.float32, device=dev) if lse is None else lse
    _tensor("gt_attn_fwd", "Y", Y, (R, H, dh), dt, dev)
    _tensor("gt_attn_fwd", "lse", lse, (R, H), torch.float32, dev)
    _on_gpu("gt_attn_fwd", g, dev)
    work = _work(g, H, dh, dev, work)
    _check(lib().gt_attn_fwd(C.byref(g.st), H, dh, _dt(Q.dtype), scale, _ptr(Q), _ptr(K),
                             _ptr(V), _ptr(bias), _ptr(Y), _ptr(lse), _ptr(work),
                             work.numel(), _stream(Q.device)), "gt_attn_fwd")
    return Y, lse


def gt_attn_fwd_noalloc(g: Graph, Q, K, V, bias=None, scale=None, Y=None, lse=None):
    """Forward with the library's static scratch (no workspace argument):
    returns (Y, lse).  Allocates Y and lse only if they are not given."""
    R, H, dh, dt, dev = _attn_shapes("gt_attn_fwd_noalloc", g, Q, K, V, bias)
    scale = dh ** -0.5 if scale is None else float(scale)
    Y = torch.empty_like(Q) if Y is None else Y
    lse = torch.empty((R, H), dtype=torch.float32, device=dev) if lse is None else lse
    _tensor("gt_attn_fwd_noalloc", "Y", Y, (R, H, dh), dt, dev)
    _tensor("gt_attn_fwd_noalloc", "lse", lse, (R, H), torch.float32, dev)
    _on_gpu("gt_attn_fwd_noalloc", g, dev)
    _check(lib().gt_attn_fwd_noalloc(C.byref(g.st), H, dh, _dt(Q.dtype), scale, _ptr(Q), _ptr(K),
                                     _ptr(V), _ptr(bias), _ptr(Y), _ptr(lse), _stream(Q.device)),
           "gt_attn_fwd_noalloc")
    return Y, lse


def gt_attn_bwd(g: Graph, Q, K, V, Y, lse, dY, bias=None, scale=None, work=None,
                dQ=None, dK=None, dV=None, dbias=None):
    """Backward: returns (dQ, dK, dV, dbias); dbias is None without bias.
    Y and lse are the forward's outputs."""
    where = "gt_attn_bwd"
    R, H, dh, dt, dev = _attn_shapes(where, g, Q, K, V, bias)
    scale = dh ** -0.5 if scale is None else float(scale)
    _tensor(where, "Y", Y, (R, H, dh), dt, dev)
    _tensor(where, "lse", lse, (R, H), torch.float32, dev)
    _tensor(where, "dY", dY, (R, H, dh), dt, dev)
    dQ = torch.empty_like(Q) if dQ is None else dQ
    dK = torch.empty_like(K) if dK is None else dK
    dV = torch.empty_like(V) if dV is None else dV
    if bias is not None and dbias is None:
        dbias = torch.empty_like(bias)
    _need((bias is None) == (dbias is None), where, "bias and dbias go together")
    _tensor(where, "dQ", dQ, (R, H, dh), dt, dev)
    _tensor(where, "dK", dK, (g.n_cols, H, dh), dt, dev)
    _tensor(where, "dV", dV, (g.n_cols, H, dh), dt, dev)
    if dbias is not None:
        _tensor(where, "dbias", dbias, (g.nnz, H), torch.float32, dev)
    _on_gpu(where, g, dev)
    work = _work(g, H, dh, dev, work)
    _check(lib().gt_attn_bwd(C.byref(g.st), H, dh, _dt(Q.dtype), scale, _ptr(Q), _ptr(K),
                             _ptr(V), _ptr(bias), _ptr(Y), _ptr(lse), _ptr(dY), _ptr(dQ),
                             _ptr(dK), _ptr(dV), _ptr(dbias), _ptr(work), work.numel(),
                             _stream(Q.device)), "gt_attn_bwd")
    return dQ, dK, dV, dbias


def bwd_reads_y(has_bias: bool) -> bool:
    """Whether gt_attn_bwd reads Y: with a bias its row pass shifts its sums
    by <dY, Y> (include/gt_attn.h)."""
    return bool(has_bias)


PROF_KERNELS = ["fwd", "fwd_merge", "bwd_rows", "bwd_rows_merge", "bwd_cols", "bwd_cols_merge",
                "bwd_dbias"]


def prof_enable(kernels=True):
    """Time the launches of ``kernels`` (a list of names; True: all; False:
    none) with HIP events."""
    if kernels is True:
        mask = (1 << len(PROF_KERNELS)) - 1
    elif not kernels:
        mask = 0
    else:
        mask = sum(1 << PROF_KERNELS.index(k) for k in kernels)
    _check(lib().gt_prof_enable(mask), "gt_prof_enable")


def prof_reset():
    _check(lib().gt_prof_reset(), "gt_prof_reset")


def prof_query(kernel: str):
    """(total milliseconds, launches) recorded for a kernel since the reset."""
    ms, n = C.c_double(), _i64()
    _check(lib().gt_prof_query(kernel.encode(), C.byref(ms), C.byref(n)), "gt_prof_query")
    return ms.value, n.value


class GTAttnFn(torch.autograd.Function):
    """Sparse graph attention as an autograd function over a prepared graph."""

    @staticmethod
    def forward(ctx, g: Graph, Q, K, V, bias=None, scale=None):
        Q, K, V = Q.contiguous(), K.contiguous(), V.contiguous()
        bias = None if bias is None else bias.contiguous()
        Y, lse = gt_attn_fwd(g, Q, K, V, bias, scale)
        ctx.g, ctx.scale = g, scale
        ctx.save_for_backward(Q, K, V, Y, lse, bias if bias is not None else torch.empty(0))
        ctx.has_bias = bias is not None
        return Y

    @staticmethod
    def backward(ctx, dY):
        Q, K, V, Y, lse, bias = ctx.saved_tensors
        bias = bias if ctx.has_bias else None
        dQ, dK, dV, db = gt_attn_bwd(ctx.g, Q, K, V, Y, lse, dY.contiguous(), bias, ctx.scale)
        return None, dQ, dK, dV, db, None


def sparse_graph_attention(g: Graph, Q, K, V, bias=None, scale=None):
    return GTAttnFn.apply(g, Q, K, V, bias, scale)


# ----------------------------------------------------------------------------
# dense parts of the layer (include/gt_proj.h)
# ----------------------------------------------------------------------------

def _proj_lib():
    L = lib()
    if not getattr(L, "_proj_sigs", False):
        sig = {
            "gt_proj_qkv": (_i32, [_i64, _i32, _i32] + [_P] * 8),
            "gt_proj_out": (_i32, [_i64, _i32, _i32] + [_P] * 5),
            "gt_proj_bwd_data": (_i32, [_i64, _i32, _i32] + [_P] * 10),
            "gt_proj_work_bytes": (_sz, [_i64, _i32]),
            "gt_proj_bwd_weight": (_i32, [_i64, _i32, _i32] + [_P] * 10 + [_sz, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        L._proj_sigs = True
    return L


def _nd(where: str, X, *others):
    """(n, d) of X [n, d]; `others` are (name, tensor, shape) to check against it."""
    _need(isinstance(X, torch.Tensor) and X.dim() == 2, where, "X must be a [n, d] tensor")
    _need(X.dtype in (torch.float32, torch.bfloat16), where, lambda: f"unsupported dtype {X.dtype}")
    _need(X.is_contiguous(), where, "X must be contiguous")
    n, d = X.shape
    for name, t, shape in others:
        _tensor(where, name, t, shape(n, d), X.dtype, X.device)
    _need(X.device.type == "cuda", where, lambda: f"tensors must be on a GPU, X is on {X.device}")
    return n, d


_W = lambda n, d: (d, d)
_ND = lambda n, d: (n, d)


def gt_proj_qkv(X, Wq, Wk, Wv):
    """Q, K, V = X W_q, X W_k, X W_v; X [n, d], W [d, d] (f32 or bf16)."""
    n, d = _nd("gt_proj_qkv", X, ("Wq", Wq, _W), ("Wk", Wk, _W), ("Wv", Wv, _W))
    Q, K, V = (torch.empty_like(X) for _ in range(3))
    _check(_proj_lib().gt_proj_qkv(n, d, _dt(X.dtype), _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                                   _ptr(Q), _ptr(K), _ptr(V), _stream(X.device)), "gt_proj_qkv")
    return Q, K, V


def gt_proj_out(X, Wo, Y):
    """Z = X W_o + Y."""
    n, d = _nd("gt_proj_out", X, ("Wo", Wo, _W), ("Y", Y, _ND))
    Z = torch.empty_like(X)
    _check(_proj_lib().gt_proj_out(n, d, _dt(X.dtype), _ptr(X), _ptr(Wo), _ptr(Y), _ptr(Z),
                                   _stream(X.device)), "gt_proj_out")
    return Z


def gt_proj_bwd_data(dZ, dQ, dK, dV, Wo, Wq, Wk, Wv):
    """dX = dZ W_o^T + dQ W_q^T + dK W_k^T + dV W_v^T."""
    n, d = _nd("gt_proj_bwd_data", dZ, ("dQ", dQ, _ND), ("dK", dK, _ND), ("dV", dV, _ND),
               ("Wo", Wo, _W), ("Wq", Wq, _W), ("Wk", Wk, _W), ("Wv", Wv, _W))
    dX = torch.empty_like(dZ)
    _check(_proj_lib().gt_proj_bwd_data(n, d, _dt(dZ.dtype), _ptr(dZ), _ptr(dQ), _ptr(dK),
                                        _ptr(dV), _ptr(Wo), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                                        _ptr(dX), _stream(dZ.device)), "gt_proj_bwd_data")
    return dX


def gt_proj_bwd_weight(X, dZ, dQ, dK, dV, work=None):
    """dW_o, dW_q, dW_k, dW_v = X^T dZ, X^T dQ, X^T dK, X^T dV (float32)."""
    n, d = _nd("gt_proj_bwd_weight", X, ("dZ", dZ, _ND), ("dQ", dQ, _ND), ("dK", dK, _ND),
               ("dV", dV, _ND))
    L = _proj_lib()
    nb = L.gt_proj_work_bytes(n, d)
    if work is not None:
        _need(work.dtype == torch.uint8 and work.device == X.device and work.is_contiguous(),
              "gt_proj_bwd_weight", "work must be a contiguous uint8 tensor on X's device")
    if work is None or work.numel() < nb:
        work = torch.empty(nb, dtype=torch.uint8, device=X.device)
    dW = [torch.empty((d, d), dtype=torch.float32, device=X.device) for _ in range(4)]
    _check(L.gt_proj_bwd_weight(n, d, _dt(X.dtype), _ptr(X), _ptr(dZ), _ptr(dQ), _ptr(dK),
                                _ptr(dV), *(_ptr(w) for w in dW), _ptr(work), work.numel(),
                                _stream(X.device)), "gt_proj_bwd_weight")
    return tuple(dW)


class SGALayerFn(torch.autograd.Function):
    """One sparse graph attention layer: Z = X W_o + attention(X W_q, X W_k,
    X W_v) over a prepared graph, with its backward through the C ABI."""

    @staticmethod
    def forward(ctx, g: Graph, heads: int, X, Wq, Wk, Wv, Wo, bias=None, scale=None):
        X = X.contiguous()
        n, d = X.shape
        Q, K, V = gt_proj_qkv(X, Wq, Wk, Wv)
        shp = (n, heads, d // heads)
        Y, lse = gt_attn_fwd(g, Q.view(shp), K.view(shp), V.view(shp), bias, scale)
        Z = gt_proj_out(X, Wo, Y.view(n, d))
        ctx.g, ctx.heads, ctx.scale, ctx.has_bias = g, heads, scale, bias is not None
        ctx.save_for_backward(X, Wq, Wk, Wv, Wo, Q, K, V, Y, lse,
                              bias if bias is not None else torch.empty(0))
        return Z

    @staticmethod
    def backward(ctx, dZ):
        X, Wq, Wk, Wv, Wo, Q, K, V, Y, lse, bias = ctx.saved_tensors
        bias = bias if ctx.has_bias else None
        dZ = dZ.contiguous()
        n, d = X.shape
        shp = (n, ctx.heads, d // ctx.heads)
        dQ, dK, dV, db = gt_attn_bwd(ctx.g, Q.view(shp), K.view(shp), V.view(shp), Y, lse,
                                     dZ.view(shp), bias, ctx.scale)
        dQ, dK, dV = (t.view(n, d) for t in (dQ, dK, dV))
        dX = gt_proj_bwd_data(dZ, dQ, dK, dV, Wo, Wq, Wk, Wv)
        dWo, dWq, dWk, dWv = gt_proj_bwd_weight(X, dZ, dQ, dK, dV)
        cast = lambda w, ref: w.to(ref.dtype)
        return (None, None, dX, cast(dWq, Wq), cast(dWk, Wk), cast(dWv, Wv), cast(dWo, Wo),
                db, None)


def sga_layer(g: Graph, heads: int, X, Wq, Wk, Wv, Wo, bias=None, scale=None):
    return SGALayerFn.apply(g, heads, X, Wq, Wk, Wv, Wo, bias, scale)


# ----------------------------------------------------------------------------
# head repack of graph parallelism with all-to-all (include/gt_heads.h)
# ----------------------------------------------------------------------------

def _heads_geometry(t: torch.Tensor):
    """(rows, heads, head_bytes) of a contiguous [rows, heads, ...] tensor."""
    _need(isinstance(t, torch.Tensor) and t.dim() >= 2 and t.is_contiguous(), "head repack",
          "expects a contiguous [rows, heads, ...] tensor")
    _need(t.device.type == "cuda", "head repack", lambda: f"tensors must be on a GPU, not {t.device}")
    rows, heads = t.shape[0], t.shape[1]
    per_head = t[0, 0].numel() if rows > 0 else math.prod(t.shape[2:])
    return rows, heads, int(per_head) * t.element_size()


def gt_head_split(x: torch.Tensor, parts: int, out=None) -> torch.Tensor:
    """[rows, heads, ...] -> [parts, rows, heads/parts, ...]: part r holds
    heads r*heads/parts .. (r+1)*heads/parts - 1 of every row."""
    rows, heads, hb = _heads_geometry(x)
    _need(parts >= 1 and heads % parts == 0, "gt_head_split",
          f"{heads} heads do not split into {parts} equal parts")
    shape = (parts, rows, heads // parts) + tuple(x.shape[2:])
    out = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else out
    _tensor("gt_head_split", "out", out, shape, x.dtype, x.device)
    _check(lib().gt_head_split(rows, heads, hb, parts, _ptr(x), _ptr(out), _stream(x.device)),
           "gt_head_split")
    return out


def gt_head_merge(p: torch.Tensor, out=None) -> torch.Tensor:
    """The inverse of gt_head_split: [parts, rows, hp, ...] -> [rows, parts*hp, ...]."""
    _need(isinstance(p, torch.Tensor) and p.dim() >= 3 and p.is_contiguous(), "gt_head_merge",
          "expects a contiguous [parts, rows, heads/parts, ...] tensor")
    _need(p.device.type == "cuda", "gt_head_merge", lambda: f"tensors must be on a GPU, not {p.device}")
    parts, rows, hp = p.shape[0], p.shape[1], p.shape[2]
    heads = parts * hp
    hb = math.prod(p.shape[3:]) * p.element_size()
    shape = (rows, heads) + tuple(p.shape[3:])
    out = torch.empty(shape, dtype=p.dtype, device=p.device) if out is None else out
    _tensor("gt_head_merge", "out", out, shape, p.dtype, p.device)
    _check(lib().gt_head_merge(rows, heads, hb, parts, _ptr(p), _ptr(out), _stream(p.device)),
           "gt_head_merge")
    return out


def attn_head_sliced(g: Graph, Q, K, V, dY=None, bias=None, scale=None, parts: int = 2):
    """The attention as graph parallelism with all-to-all computes it, with
    the `parts` workers on one GPU: the heads are split into `parts` slices
    (what each worker holds after the first all-to-all), the attention runs
    on each slice over the whole graph, and the outputs are merged back
    (the return all-to-all).  Returns (Y, lse) and, with dY, also
    (dQ, dK, dV, dbias)."""
    R, H, dh = Q.shape
    scale = dh ** -0.5 if scale is None else float(scale)
    q, k, v = (gt_head_split(t, parts) for t in (Q, K, V))
    b = gt_head_split(bias, parts) if bias is not None else None
    br = lambda r: b[r] if b is not None else None
    # per-slice outputs go straight into the packed layout the merge reads
    Yp = torch.empty_like(q)
    lsep = torch.empty((parts, R, H // parts), dtype=torch.float32, device=Q.device)
    for r in range(parts):
        gt_attn_fwd(g, q[r], k[r], v[r], br(r), scale, Y=Yp[r], lse=lsep[r])
    Y, lse = gt_head_merge(Yp), gt_head_merge(lsep)
    if dY is None:
        return Y, lse
    dy = gt_head_split(dY, parts)
    dQp, dKp, dVp = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dBp = torch.empty_like(b) if b is not None else None
    for r in range(parts):
        gt_attn_bwd(g, q[r], k[r], v[r], Yp[r], lsep[r], dy[r], br(r), scale, dQ=dQp[r], dK=dKp[r],
                    dV=dVp[r], dbias=dBp[r] if dBp is not None else None)
    dB = gt_head_merge(dBp) if dBp is not None else None
    return Y, lse, gt_head_merge(dQp), gt_head_merge(dKp), gt_head_merge(dVp), dB
