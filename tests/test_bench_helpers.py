"""The benchmark's host-side helpers, on the CPU: the byte models against
per-pass figures worked out by hand for the Hub workload, the compulsory-byte
count, the parity verdict of a timed run (it must pass the oracle's own
outputs and fail a perturbed one), and the stored counter records (used
only on the sources they were taken on)."""
import numpy as np
import pytest

import bench
from graph_transformer_sparse_amd import inputs as I
from oracle import oracle as O


def test_byte_model_matches_the_tabulated_figures():
    """Hub: 2.4M rows and columns (every column has its self-loop), 62M
    edges, 4 heads of 32 in bf16, with bias: 34.3 / 36.6 / 37.7 GB for the
    forward, the row pass (Y read: D = <dY, Y> needs it) and the column pass."""
    cfg = I.CONFIGS["hub"]
    m = bench.byte_model(cfg, 2_400_000, 2_400_000, 62_000_000, 2_400_000, True)
    assert round(m["fwd"] / 1e9, 1) == 34.3
    assert round(m["bwd_rows"] / 1e9, 1) == 36.6
    assert round(m["bwd_cols"] / 1e9, 1) == 37.7
    # the finishing pass of dbias is reported with its kernel, outside the model
    assert bench.aux_model(cfg, 2_400_000, 62_000_000) == {"bwd_dbias": 62_000_000 * 32 + 2_400_000 * 32}
    assert bench.aux_model(I.CONFIGS["mid"], 10, 10) == {}
    # without a bias the row pass reads no Y
    mid = I.CONFIGS["mid"]
    a = bench.byte_model(mid, 100, 100, 1000, 100, False)["bwd_rows"]
    b = bench.byte_model(mid, 100, 100, 1000, 100, True)["bwd_rows"]
    assert b - a == 100 * 128 * 4


def test_unique_bytes_counts_every_array_once():
    cfg = I.CONFIGS["hub"]
    R = M = 2_400_000
    E, H, Ds = 62_000_000, 4, 128 * 2
    got = bench.unique_bytes(cfg, R, M, E, True)
    csr, csr_t, feat, bias = 4 * (R + 1) + 4 * E, 4 * (M + 1) + 8 * E, R * Ds, 4 * E * H
    fwd = csr + 3 * feat + bias + feat + 4 * R * H                  # Q K V bias in; Y lse out
    bwd = csr + csr_t + 3 * feat + 2 * feat + 4 * R * H + bias + 3 * feat + bias + 16 * R * H
    assert got == fwd + bwd
    assert round(got / 1e9, 1) == 11.6


def test_parity_verdict_of_a_timed_run():
    P = I.make_problem(I.CONFIGS["tiny"])
    M = P.cfg.n_cols
    rY, rl = O.fwd(P.indptr, P.indices, M, P.Q, P.K, P.V, None, P.scale)
    rQ, rK, rV, _ = O.bwd(P.indptr, P.indices, M, P.Q, P.K, P.V, P.dY, None, P.scale)
    got = dict(Y=rY.copy(), lse=rl.copy(), dQ=rQ.copy(), dK=rK.copy(), dV=rV.copy(), dbias=None)
    rep = bench.parity_full(P, got)
    assert rep["verdict"] == "pass" and set(rep["tensors"]) == {"Y", "lse", "dQ", "dK", "dV"}
    got["dK"] = rK * (1 + 1e-4)                  # ten times the float32 tolerance
    assert bench.parity_full(P, got)["verdict"] == "FAIL"
    got["dK"] = rK.copy()
    got["lse"] = rl + 1e-3
    assert bench.parity_full(P, got)["verdict"] == "FAIL"


def test_counter_records_are_gated_by_the_source_hash(tmp_path, monkeypatch):
    rec = bench.counter_record("hub", True)
    if rec is not None:                          # taken on the current sources
        assert set(rec["per_kernel"]) == {"fwd", "bwd_rows", "bwd_cols", "bwd_dbias"}
        assert rec["bytes_per_step"] == pytest.approx(sum(rec["per_kernel"].values()))
    # a record whose hash differs is not used
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_fwd_x.txt").write_text(
        "source_hash: 0000000000000000\nhbm_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_record("fwd", "x") is None
    (tmp_path / "profiles" / "traffic_fwd_x.txt").write_text(
        f"source_hash: {bench.kernel_source_hash()}\nhbm_bytes_per_launch: 123\n")
    assert bench.traffic_record("fwd", "x") == 123.0


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and a
    message, before anything touches a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
