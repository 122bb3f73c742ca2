"""The attention forward and backward captured into a HIP graph and
replayed: every replay must give exactly the eager results.  The fwd/bwd
entry points enqueue kernels only (no memsets, copies or synchronisation),
which is what lets a caller capture a training step to cut launch overhead
on small graphs."""
import numpy as np
import pytest
import torch

from graph_transformer_sparse_amd import gtattn as T
from graph_transformer_sparse_amd import inputs as I

from gpu_util import device_problem

pytestmark = pytest.mark.gpu


def _bits(t):
    t = t.detach()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_graph_replays_match_eager(dtype):
    rng = np.random.default_rng(4)
    n = 500
    degs = rng.integers(0, 40, n)
    degs[:2] = (300, 490)                       # split rows: the merge kernels are captured too
    ip, ix = I.random_graph(44, n, n, degs)
    P = I.small_problem(44, ip, ix, n, 4, 32, dtype, True)
    d = device_problem(P)
    g = T.gt_graph_prepare(d["indptr"], d["indices"], n, 4, 16, 16)
    Q, K, V, dY, bias = d["Q"], d["K"], d["V"], d["dY"], d["bias"]
    work = torch.empty(T.gt_attn_work_bytes(g, 4, 32), dtype=torch.uint8, device="cuda")
    Y, lse = torch.empty_like(Q), torch.empty((n, 4), device="cuda")
    dQ, dK, dV, dB = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V), torch.empty_like(bias)

    def step():
        T.gt_attn_fwd(g, Q, K, V, bias, P.scale, work, Y, lse)
        T.gt_attn_bwd(g, Q, K, V, Y, lse, dY, bias, P.scale, work, dQ, dK, dV, dB)

    step()
    torch.cuda.synchronize()
    ref = [_bits(t).clone() for t in (Y, lse, dQ, dK, dV, dB)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                  # warm up on the side stream before capture
        step()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (Y, lse, dQ, dK, dV, dB):
            t.fill_(7.0)                        # eager work between replays
        print(f"graph {dtype} replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("Y", "lse", "dQ", "dK", "dV", "dbias"), (Y, lse, dQ, dK, dV, dB), ref):
            assert torch.equal(_bits(t), r), f"replay {rep}: {name} differs from eager"
        step()                                  # and an eager step between replays
        torch.cuda.synchronize()
