"""The forward for callers that cannot allocate (gt_attn_fwd_noalloc: split
rows' softmax states in the library's static device array instead of a
caller workspace), called through the C ABI, against the workspace forward
(gt_attn_fwd: the same kernels, so bitwise equal) and against the oracle, on
two calls in a row, the second with a smaller input (the array keeps the
first call's contents)."""
import ctypes as C

import numpy as np
import pytest
import torch

from graph_transformer_sparse_amd import gtattn as T
from graph_transformer_sparse_amd import inputs as I
from oracle import oracle as O

from gpu_util import RTOL, assert_close, assert_lse, device_problem

pytestmark = pytest.mark.gpu


def _noalloc(g, d, P):
    Q, K, V, bias = d["Q"], d["K"], d["V"], d["bias"]
    R, H, dh = Q.shape
    Y = torch.empty_like(Q)
    lse = torch.empty((R, H), dtype=torch.float32, device=Q.device)
    dt = T.GT_F32 if Q.dtype == torch.float32 else T.GT_BF16
    L = T.lib()
    st = L.gt_attn_fwd_noalloc(C.byref(g.st), H, dh, dt, P.scale, Q.data_ptr(), K.data_ptr(),
                               V.data_ptr(), bias.data_ptr() if bias is not None else None,
                               Y.data_ptr(), lse.data_ptr(),
                               C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.gt_last_error()
    return Y, lse


@pytest.mark.parametrize("dt, H, dh, bias", [("bf16", 4, 32, True), ("f32", 8, 16, False)])
def test_noalloc_forward_two_calls(dt, H, dh, bias):
    rng = np.random.default_rng(91)
    for call, (R, M, top) in enumerate(((1500, 1400, 900), (400, 380, 300))):
        degs = rng.integers(0, 60, R)
        degs[:6] = (top, top - 1, 257, 200, 129, 65)        # split rows (chunk 16 below)
        ip, ix = I.random_graph(91 + call, R, M, np.minimum(degs, M), self_loops=False)
        P = I.small_problem(91 + call, ip, ix, M, H, dh, dt, bias)
        d = device_problem(P)
        g = T.gt_graph_prepare(d["indptr"], d["indices"], M, 4, 16, 16)
        assert g.st.rows.n_merges > 0
        print(f"noalloc call {call}: {dt} H={H} dh={dh} R={R} pieces={g.st.rows.n_items}",
              flush=True)
        Yw, lw = T.gt_attn_fwd(g, d["Q"], d["K"], d["V"], d["bias"], P.scale)
        Yn, ln = _noalloc(g, d, P)
        torch.cuda.synchronize()
        assert torch.equal(Yn, Yw) and torch.equal(ln, lw)
        m = {}
        rY, rl = O.fwd(ip, ix, M, P.Q, P.K, P.V, P.bias, P.scale, mag=m)
        assert_close(Yn, rY, RTOL[dt], "Y", m["Y"])
        assert_lse(ln, rl, 1e-5 if dt == "f32" else 1e-4)
