"""The C ABI library without a GPU: it loads, exports every function the
header declares, and its host-side argument checks return the documented
status codes before anything touches the device (fake device pointers are
never dereferenced on these paths)."""
import ctypes as C
import os

import pytest

from graph_transformer_sparse_amd import build as B
from graph_transformer_sparse_amd import gtattn as T


def _fresh():
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)]
    srcs += [os.path.join(B.INCLUDE, f) for f in os.listdir(B.INCLUDE)]
    return os.path.exists(B.LIB) and os.path.getmtime(B.LIB) >= max(map(os.path.getmtime, srcs))


@pytest.fixture(scope="module")
def L():
    if not _fresh():
        B.build()
    return T.lib()


def test_exports_every_declared_function(L):
    names = T.header_functions()
    assert "gt_attn_fwd" in names and "gt_attn_bwd" in names and "gt_graph_prepare" in names
    assert "gt_proj_qkv" in names and "gt_proj_bwd_weight" in names
    for n in names:
        assert hasattr(L, n), n
    assert L.gt_version() >= 100


def test_status_strings(L):
    for code in range(10):
        assert L.gt_status_str(code)
    assert L.gt_status_str(99) == b"unknown status"


def test_default_thresholds(L):
    ts, tm, ch = T.gt_default_thresholds()
    assert (ts, tm, ch) == (32, 256, 256)
    # one size serves every graph (pieces are dealt to the XCDs by position)
    for nnz in (0, 1000, 1_842_047, 8 << 20, 62_000_000, 2_147_483_000):
        assert T.gt_graph_thresholds(nnz) == (ts, tm, ch)


def _fake_graph(R=100, M=80, E=500, n_items=3):
    g = T.GtGraph()
    g.n_rows, g.n_cols, g.nnz = R, M, E
    fake = 0x10000000
    g.indptr, g.indices, g.indptr_t, g.indices_t, g.perm = fake, fake, fake, fake, fake
    for s in (g.rows, g.cols):
        s.order, s.items, s.merges, s.spans = fake, fake, fake, fake
        s.n_items = n_items
    return g


FAKE = C.c_void_p(0x20000000)      # 16-byte aligned, never dereferenced here
ODD = C.c_void_p(0x20000004)


def _fwd(L, g, heads=4, dh=32, dt=T.GT_F32, Q=FAKE, K=FAKE, V=FAKE, bias=None, Y=FAKE,
         lse=FAKE, work=FAKE, nb=1 << 30):
    return L.gt_attn_fwd(C.byref(g) if g is not None else None, heads, dh, dt, 0.1, Q, K, V,
                         bias, Y, lse, work, nb, None)


def test_fwd_argument_checks(L):
    g = _fake_graph()
    assert _fwd(L, None) == 1                       # NULL graph
    assert _fwd(L, g, dt=7) == 3                    # dtype
    assert _fwd(L, g, dh=48) == 4                   # head_dim
    assert _fwd(L, g, heads=3) == 4                 # heads
    assert _fwd(L, g, heads=8, dh=64) == 4          # 2 KiB rows in fp32
    assert _fwd(L, g, heads=4, dh=128) == 4         # 2 KiB rows in fp32
    assert _fwd(L, g, dh=256) == 4                  # head_dim
    assert _fwd(L, g, dh=4) == 4                    # head_dim
    assert _fwd(L, g, Q=None) == 1
    assert _fwd(L, g, K=ODD) == 5
    assert _fwd(L, g, lse=None) == 1
    assert _fwd(L, g, work=None) == 1
    assert _fwd(L, g, nb=16) == 7                   # workspace too small
    assert b"work has 16 bytes" in L.gt_last_error()
    ung = _fake_graph()
    ung.rows.order = None
    assert _fwd(L, ung) == 1                        # not prepared


def test_fwd_noalloc_argument_checks(L):
    """The static-scratch forward checks its arguments like gt_attn_fwd and
    refuses, before touching the device, a graph whose split rows need more
    scratch than its static array holds."""
    def call(g, Q=FAKE, Y=FAKE, lse=FAKE, dh=32):
        return L.gt_attn_fwd_noalloc(C.byref(g) if g is not None else None, 4, dh, T.GT_F32, 0.1,
                                     Q, FAKE, FAKE, None, Y, lse, None)
    g = _fake_graph()
    assert call(None) == 1
    assert call(g, dh=48) == 4
    assert call(g, Q=ODD) == 5
    assert call(g, lse=None) == 1
    # 4 heads x 32: (128 + 8) floats per piece state, so 31,000 pieces need 16.9 MB
    big = _fake_graph(n_items=31_000)
    assert call(big) == 7
    assert b"static maximum" in L.gt_last_error()


def test_bwd_argument_checks(L):
    g = _fake_graph()

    def bwd(bias=None, dbias=None, dQ=FAKE, nb=1 << 30, heads=4, Y=FAKE):
        return L.gt_attn_bwd(C.byref(g), heads, 32, T.GT_BF16, 0.1, FAKE, FAKE, FAKE, bias,
                             Y, FAKE, FAKE, dQ, FAKE, FAKE, dbias, FAKE, nb, None)

    assert bwd(bias=FAKE) == 6                      # bias without dbias
    assert bwd(dbias=FAKE) == 6
    assert bwd(dQ=ODD) == 5
    assert bwd(nb=64) == 7
    assert bwd(heads=16) == 4
    assert bwd(bias=FAKE, dbias=FAKE, Y=None) == 1  # with a bias the row pass reads Y
    assert b"Y is NULL" in L.gt_last_error()
    assert bwd(bias=FAKE, dbias=FAKE, Y=ODD) == 5


def test_work_bytes_grow_with_graph(L):
    g = _fake_graph(n_items=0)
    a = L.gt_attn_work_bytes(C.byref(g), 4, 32)
    g2 = _fake_graph(n_items=100)
    b = L.gt_attn_work_bytes(C.byref(g2), 4, 32)
    assert b > a > 0
    # backward: per-row statistics (lse, D) = 8 bytes per row and head
    assert a >= 100 * 4 * 8


def test_prepare_argument_checks(L):
    mb = L.gt_graph_meta_bytes(100, 80, 500, 64)
    assert mb > 4 * (2 * 500 + 81)
    assert L.gt_graph_meta_bytes(-1, 80, 500, 64) == 0
    assert L.gt_graph_meta_bytes(100, 80, 500, 0) == 0
    assert L.gt_graph_meta_bytes(1 << 31, 80, 500, 64) == 0
    out = T.GtGraph()

    def prep(indptr=FAKE, indices=FAKE, ts=4, tm=8, ch=8, meta=FAKE, nb=mb, o=True):
        return L.gt_graph_prepare(indptr, indices, 100, 80, 500, ts, tm, ch, meta, nb,
                                  C.byref(out) if o else None, None)

    assert prep(o=False) == 1
    assert prep(indptr=None) == 1
    assert prep(meta=None) == 1
    assert prep(ts=9) == 2                           # t_small > t_mid
    assert prep(ch=0) == 2
    assert prep(nb=mb - 1) == 7


def test_validate_argument_checks(L):
    code = C.c_int32(-1)
    assert L.gt_csr_validate(None, FAKE, 10, 10, 5, FAKE, 64, C.byref(code), None) == 1
    assert L.gt_csr_validate(FAKE, FAKE, 10, 10, 5, FAKE, 8, C.byref(code), None) == 7
    assert L.gt_csr_validate(FAKE, FAKE, -1, 10, 5, FAKE, 64, C.byref(code), None) == 2


def test_prof_query_checks(L):
    ms, n = C.c_double(), C.c_int64()
    assert L.gt_prof_query(b"nope", C.byref(ms), C.byref(n)) == 2
    assert L.gt_prof_query(b"fwd", C.byref(ms), C.byref(n)) == 0 and n.value == 0


def test_proj_argument_checks(L):
    T._proj_lib()
    assert L.gt_proj_qkv(10, 96, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 4   # d
    assert L.gt_proj_qkv(10, 128, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 3  # dtype
    assert L.gt_proj_qkv(10, 128, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.gt_proj_out(10, 128, 1, FAKE, ODD, FAKE, FAKE, None) == 5
    assert L.gt_proj_out(-1, 128, 1, FAKE, FAKE, FAKE, FAKE, None) == 2
    nb = L.gt_proj_work_bytes(100000, 128)
    assert nb >= 4 * 128 * 128 * 128 * 4         # 128 row slots, 4 gradients of [128, 128]
    assert L.gt_proj_bwd_weight(100000, 128, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, FAKE, nb - 1, None) == 7


def test_heads_argument_checks(L):
    # rows, heads, head_bytes, parts, src, dst, stream
    assert L.gt_head_split(10, 6, 64, 4, FAKE, FAKE, None) == 4     # heads % parts
    assert L.gt_head_split(10, 8, 6, 2, FAKE, FAKE, None) == 4      # head_bytes not a multiple of 4
    assert L.gt_head_split(10, 8, 64, 0, FAKE, FAKE, None) == 2     # parts
    assert L.gt_head_merge(-1, 8, 64, 2, FAKE, FAKE, None) == 2     # rows
    assert L.gt_head_merge(10, 8, 64, 2, None, FAKE, None) == 1
    assert L.gt_head_split(10, 8, 64, 2, FAKE, C.c_void_p(0x20000002), None) == 5  # alignment
    assert L.gt_head_split(0, 8, 64, 2, None, None, None) == 0      # nothing to move


def test_library_imports_no_device_allocator(L):
    """The library allocates no device or pinned memory: every buffer is the
    caller's (meta, work, inputs and outputs).  Checked on the shared
    object's imported symbols, so no code path can call an allocator."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", B.LIB], capture_output=True, text=True,
                         check=True).stdout
    names = [ln.split()[-1].split("@")[0] for ln in out.splitlines() if ln.strip()]
    assert "hipLaunchKernel" in names          # the listing is the real one
    alloc = [n for n in names if n.startswith(("hipMalloc", "hipFree", "hipHostMalloc",
                                               "hipHostAlloc", "hipExtMalloc", "hipMallocManaged",
                                               "hipMemPool"))]
    assert alloc == [], alloc
