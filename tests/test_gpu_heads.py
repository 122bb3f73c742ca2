"""The head repack of graph parallelism with all-to-all (include/gt_heads.h)
against the oracle (oracle/heads.py, pinned to the simulated exchange in
test_oracle_heads.py): a byte permutation, so bit-exact; and the attention
run on head slices the way GP-A2A runs it (split, attend per slice over
the whole graph, merge), against the fp64 attention oracle at the usual
tolerance (the paper's Section 3.2 / Algorithm 2)."""
import numpy as np
import pytest
import torch

from graph_transformer_sparse_amd import gtattn as T
from graph_transformer_sparse_amd import inputs as I
from oracle import heads as Hd
from oracle import oracle as O

from gpu_util import RTOL, TDT, assert_close, assert_lse, dev, device_problem

pytestmark = pytest.mark.gpu


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = [  # rows, heads, trailing shape, dtype
    (1, 8, (16,), torch.float32), (7, 8, (16,), torch.float32), (1000, 4, (32,), torch.bfloat16),
    (100003, 8, (16,), torch.float32), (4097, 8, (32,), torch.bfloat16), (333, 2, (64,), torch.bfloat16),
    (5000, 8, (), torch.float32), (5000, 4, (), torch.float32), (259, 1, (64,), torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=[f"r{a}-h{b}-{len(c) and c[0]}-{str(d)[6:]}" for a, b, c, d in CASES])
def test_split_merge_bit_exact(case):
    rows, heads, tail, dt = case
    g = torch.Generator().manual_seed(rows + heads)
    x = torch.randn((rows, heads) + tail, generator=g).to(dt)
    xd = x.cuda()
    for parts in [p for p in (1, 2, 4, 8) if heads % p == 0]:
        print(f"heads rows={rows} heads={heads} tail={tail} {dt} parts={parts}", flush=True)
        s = T.gt_head_split(xd, parts)
        ref = torch.from_numpy(Hd.head_split(x.view(torch.int16 if dt == torch.bfloat16 else torch.int32).numpy(), parts))
        assert torch.equal(_bits(s), ref)
        m = T.gt_head_merge(s)
        assert torch.equal(_bits(m), _bits(x))


def test_unaligned_and_empty():
    buf = torch.randn(1 + 300 * 4 * 6, device="cuda")
    x = buf[1:].view(300, 4, 6)                  # 4-byte aligned only; 24-byte heads
    s = T.gt_head_split(x, 2)
    ref = Hd.head_split(x.cpu().numpy(), 2)
    assert np.array_equal(s.cpu().numpy(), ref)
    assert torch.equal(T.gt_head_merge(s), x)
    e = torch.empty((0, 8, 16), device="cuda")
    assert T.gt_head_split(e, 4).shape == (4, 0, 2, 16)
    assert T.gt_head_merge(T.gt_head_split(e, 4)).shape == (0, 8, 16)


def test_split_rejects_bad_shapes():
    x = torch.zeros((4, 6, 16), device="cuda")
    with pytest.raises(ValueError):
        T.gt_head_split(x, 4)                   # 6 heads do not divide among 4 workers


SLICED = [("f32", 8, 16, True, 2), ("f32", 8, 16, False, 8), ("bf16", 4, 32, True, 4),
          ("bf16", 8, 32, False, 2), ("f32", 2, 64, True, 2)]


@pytest.mark.parametrize("case", SLICED, ids=[f"{a}-h{b}-d{c}-{'bias' if d else 'nobias'}-p{e}" for a, b, c, d, e in SLICED])
def test_head_sliced_attention(case):
    dt, H, dh, bias, parts = case
    n = 400
    rng = np.random.default_rng(H * dh + parts)
    degs = rng.integers(0, 60, n)
    degs[:3] = (0, 150, 300)
    ip, ix = I.random_graph(70 + parts, n, n, degs)
    P = I.small_problem(80 + parts, ip, ix, n, H, dh, dt, bias)
    d = device_problem(P)
    g = T.gt_graph_prepare(d["indptr"], d["indices"], n, 4, 16, 16)
    print(f"sliced {case}", flush=True)
    Y, lse, dQ, dK, dV, dB = T.attn_head_sliced(g, d["Q"], d["K"], d["V"], d["dY"], d["bias"],
                                                P.scale, parts)
    torch.cuda.synchronize()
    m = {}
    rY, rl = O.fwd(ip, ix, n, P.Q, P.K, P.V, P.bias, P.scale, mag=m)
    rQ, rK, rV, rB = O.bwd(ip, ix, n, P.Q, P.K, P.V, P.dY, P.bias, P.scale, mag=m)
    rt = RTOL[dt]
    assert_close(Y, rY, rt, "Y", m["Y"])
    assert_lse(lse, rl, 1e-5 if dt == "f32" else 1e-4)
    assert_close(dQ, rQ, rt, "dQ", m["dQ"])
    assert_close(dK, rK, rt, "dK", m["dK"])
    assert_close(dV, rV, rt, "dV", m["dV"])
    if bias:
        assert_close(dB, rB, rt, "dbias", head_axis=1)
    else:
        assert dB is None


def test_split_at_large_size():
    """The repack at the Large shape (1,048,576 x 8 x 32 bf16) against the
    oracle, bit for bit, for every worker count the heads allow."""
    cfg = I.CONFIGS["large"]
    n, H, dh = cfg.n_rows, cfg.heads, cfg.head_dim
    x = torch.from_numpy(np.random.default_rng(3).integers(-2**15, 2**15, (n, H, dh), dtype=np.int16))
    xd = x.cuda().view(torch.bfloat16)
    for parts in (2, 4, 8):
        print(f"heads large parts={parts}", flush=True)
        s = T.gt_head_split(xd, parts)
        assert torch.equal(s.view(torch.int16).cpu(), torch.from_numpy(Hd.head_split(x.numpy(), parts)))
        assert torch.equal(T.gt_head_merge(s).view(torch.int16).cpu(), x)
