"""ctypes wrapper of the fp64 CPU oracle (gt_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the GPU path never does, and this
module imports nothing from it.

The wrapper only builds the shared library, marshals numpy arrays and
allocates outputs; every step of the computation is in gt_oracle.c.
GT_ORACLE_LIB, when set, names another build of gt_oracle.c to load instead
(the tests' check that the pins fail on planted mistakes).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gt_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_OUT_DIR, "libgtoracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gt_oracle.c with gcc (OpenMP, -O2, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    os.makedirs(_OUT_DIR, exist_ok=True)
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_i64, _i32, _int, _dbl = C.c_int64, C.c_int32, C.c_int, C.c_double
_P = C.c_void_p


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("GT_ORACLE_LIB") or build(force=False)
        L = C.CDLL(path)
        L.or_csr_check.restype = _int
        L.or_csr_check.argtypes = [_i64, _i64, _i64, _P, _P]
        L.or_transpose.restype = None
        L.or_transpose.argtypes = [_i64, _i64, _i64, _P, _P, _P, _P, _P]
        L.or_schedule.restype = _i64
        L.or_schedule.argtypes = [_i64, _P, _i32, _i32, _i32, _i32, _P, _P, _P, _i64, _P, _i64, _P]
        L.or_set_threads.argtypes = [_int]
        L.or_get_threads.restype = _int
        att = [_i64, _i64, _int, _int, _dbl, _P, _P, _P, _P, _P, _P]
        L.or_fwd.restype = None
        L.or_fwd.argtypes = att + [_P, _P, _P, _P]
        L.or_bwd.restype = None
        L.or_bwd.argtypes = att + [_P, _P, _P, _P, _P, _P, _P, _P]
        L.or_rows.restype = None
        L.or_rows.argtypes = att + [_P, _i64, _P, _P, _P, _P, _P, _P, _P]
        L.or_cols.restype = None
        L.or_cols.argtypes = att + [_P, _i64, _P, _P, _P, _P, _P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _i32a(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f64a(a):
    """Exact widening of float32 / bf16-valued inputs to float64."""
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def set_threads(n: int) -> None:
    lib().or_set_threads(int(n))


def threads() -> int:
    return int(lib().or_get_threads())


def csr_check(indptr, indices, n_cols: int) -> int:
    ip, ix = _i32a(indptr), _i32a(indices)
    return int(lib().or_csr_check(ip.size - 1, n_cols, ix.size, _p(ip), _p(ix)))


def transpose(indptr, indices, n_cols: int):
    """(indptr_t, indices_t, perm) of the stable CSR transpose."""
    ip, ix = _i32a(indptr), _i32a(indices)
    R, E = ip.size - 1, ix.size
    pt = np.empty(n_cols + 1, np.int32)
    it = np.empty(E, np.int32)
    pm = np.empty(E, np.int32)
    lib().or_transpose(R, n_cols, E, _p(ip), _p(ix), _p(pt), _p(it), _p(pm))
    return pt, it, pm


def schedule(ptr, t_small: int, t_mid: int, chunk: int, small_class: int = 1):
    """Degree-ordered schedule of the segments of ``ptr`` (rows of a CSR or
    columns of its transpose).  Segments go by descending degree, ties by id,
    a small segment's degree (at most t_small) rounded down to a multiple of
    ``small_class`` (4 in the library's schedule over the rows of A, 1 over
    its transpose).  Returns dict(order, counts, items, merges)."""
    ptr = _i32a(ptr)
    n = ptr.size - 1
    E = int(ptr[-1])
    cap = n + E // max(chunk, 1) + 1
    order = np.empty(n, np.int32)
    counts = np.zeros(3, np.int32)
    items = np.empty((cap, 4), np.int32)
    merges = np.empty((cap, 3), np.int32)
    nm = np.zeros(1, np.int64)
    ni = lib().or_schedule(n, _p(ptr), t_small, t_mid, chunk, small_class, _p(order), _p(counts),
                           _p(items), cap, _p(merges), cap, _p(nm))
    assert ni >= 0
    return dict(order=order, counts=counts, items=items[:ni].copy(),
                merges=merges[: int(nm[0])].copy())


def _args(indptr, indices, n_cols, Q, K, V, bias, dY, scale):
    ip, ix = _i32a(indptr), _i32a(indices)
    Q, K, V = _f64a(Q), _f64a(K), _f64a(V)
    R, H, dh = Q.shape
    assert K.shape == (n_cols, H, dh) and V.shape == K.shape
    bias = _f64a(bias)
    if bias is not None:
        assert bias.shape == (ix.size, H)
    dY = _f64a(dY)
    keep = (ip, ix, Q, K, V, bias, dY)
    head = [R, n_cols, H, dh, float(scale), _p(ip), _p(ix), _p(Q), _p(K), _p(V), _p(bias)]
    return keep, head, (R, H, dh, ix.size)


def _mag(mag, name, shape):
    if mag is None:
        return None
    mag[name] = np.empty(shape, np.float64)
    return mag[name]


def fwd(indptr, indices, n_cols, Q, K, V, bias=None, scale=None, want_U=False, mag=None):
    """Y [R,H,dh], lse [R,H] (and U [E,H] if want_U), all float64.

    If ``mag`` is a dict, mag["Y"] gets sum_e U_e |V_j|, the sum of the
    absolute values of the terms of Y (the conditioning of that sum)."""
    scale = Q.shape[2] ** -0.5 if scale is None else scale
    keep, head, (R, H, dh, E) = _args(indptr, indices, n_cols, Q, K, V, bias, None, scale)
    Y = np.empty((R, H, dh), np.float64)
    lse = np.empty((R, H), np.float64)
    U = np.empty((E, H), np.float64) if want_U else None
    lib().or_fwd(*head, _p(Y), _p(lse), _p(U), _p(_mag(mag, "Y", (R, H, dh))))
    return (Y, lse, U) if want_U else (Y, lse)


def bwd(indptr, indices, n_cols, Q, K, V, dY, bias=None, scale=None, mag=None):
    """dQ [R,H,dh], dK, dV [M,H,dh], dB [E,H] (None without bias), float64.

    If ``mag`` is a dict, mag["dQ"], mag["dK"], mag["dV"] get the sums of the
    absolute values of the terms of each output, with the score gradient
    U (dU - D) of a term bounded by U (|dU| + |D|)."""
    scale = Q.shape[2] ** -0.5 if scale is None else scale
    keep, head, (R, H, dh, E) = _args(indptr, indices, n_cols, Q, K, V, bias, dY, scale)
    dQ = np.empty((R, H, dh), np.float64)
    dK = np.empty((n_cols, H, dh), np.float64)
    dV = np.empty((n_cols, H, dh), np.float64)
    dB = np.empty((E, H), np.float64) if bias is not None else None
    lib().or_bwd(*head, _p(keep[6]), _p(dQ), _p(dK), _p(dV), _p(dB),
                 _p(_mag(mag, "dQ", (R, H, dh))), _p(_mag(mag, "dK", (n_cols, H, dh))),
                 _p(_mag(mag, "dV", (n_cols, H, dh))))
    return dQ, dK, dV, dB


def rows(indptr, indices, n_cols, Q, K, V, dY, sel, bias=None, scale=None, mag=None):
    """Y, lse, dQ of the rows ``sel`` and dB of their edges (packed); with a
    ``mag`` dict, mag["Y"] and mag["dQ"] of those rows."""
    scale = Q.shape[2] ** -0.5 if scale is None else scale
    keep, head, (R, H, dh, E) = _args(indptr, indices, n_cols, Q, K, V, bias, dY, scale)
    sel = _i32a(sel)
    ip = keep[0]
    n_e = int((ip[sel + 1] - ip[sel]).sum())
    Y = np.empty((sel.size, H, dh), np.float64)
    lse = np.empty((sel.size, H), np.float64)
    dQ = np.empty((sel.size, H, dh), np.float64)
    dB = np.empty((n_e, H), np.float64) if bias is not None else None
    lib().or_rows(*head, _p(keep[6]), sel.size, _p(sel), _p(Y), _p(lse), _p(dQ), _p(dB),
                  _p(_mag(mag, "Y", Y.shape)), _p(_mag(mag, "dQ", dQ.shape)))
    return Y, lse, dQ, dB


def cols(indptr, indices, n_cols, Q, K, V, dY, sel, bias=None, scale=None, mag=None):
    """dK, dV of the columns ``sel``; with a ``mag`` dict, mag["dK"] and
    mag["dV"] of those columns."""
    scale = Q.shape[2] ** -0.5 if scale is None else scale
    keep, head, (R, H, dh, E) = _args(indptr, indices, n_cols, Q, K, V, bias, dY, scale)
    sel = _i32a(sel)
    dK = np.empty((sel.size, H, dh), np.float64)
    dV = np.empty((sel.size, H, dh), np.float64)
    lib().or_cols(*head, _p(keep[6]), sel.size, _p(sel), _p(dK), _p(dV),
                  _p(_mag(mag, "dK", dK.shape)), _p(_mag(mag, "dV", dV.shape)))
    return dK, dV
