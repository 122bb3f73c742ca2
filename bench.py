"""Benchmark: fused sparse graph attention forward + backward on one MI355X.

One step = gt_attn_fwd + gt_attn_bwd over one synthetic graph and feature
set (every kernel of the hot path: the fused forward, the backward row pass,
the backward column pass over the transpose, and the merges of split rows and
columns).  The graph is prepared once, outside the timed region (its time is
reported separately); inputs, outputs and workspaces are resident in HBM and
allocated before timing.

With no --config, all five workloads run one after another; the last, the
hub workload (2.4M nodes, 62M edges, per-edge bias: the pages' ogbn-products
scale), is the headline and the other four go into detail.configs.  For each
workload the outputs of the timed run are checked against the fp64 oracle
on the whole graph (every output element, the tests' tolerance), and for the
headline the oracle is also timed on this host's cores on a bounded sample.

Prints ONE JSON line (rank 0) with the throughput in GEdges/s (edges =
stored nonzeros, self-loops included) and, for the dominant kernel, the
achieved fraction of the HBM roofline from the byte model below, timed with
HIP events inside the library on the stream the kernels run on (only the
dominant kernel, picked in three profiled steps after the warm-up, carries
events in the timed region; the other kernels' times in "detail" come from
those three steps).  roofline.unique_frac divides the step's compulsory
bytes (every array once) by the step time, and roofline.counter_frac the
step's counter-measured bytes (a stored rocprofv3 record in profiles/, used
only while the kernel sources hash the same).

Byte model (algorithmic bytes: what each kernel must move between HBM and
the ALUs; s = bytes per element, D = H*dh, b = 1 with a per-edge bias, y = 1
when the row pass reads Y, which it does with a bias):
  fwd       R (4 + 2Ds + 4H)                     + E (4 + 2Ds + 4Hb)
  bwd_rows  R (4 + (3 + y)Ds + 12H)              + E (4 + 2Ds + 8Hb)
  bwd_cols  M (4 + 2Ds) + M_nz 2Ds               + E (4 + 2Ds + 8H + (4 + 4H)b)
With a bias the row pass stages each edge's score gradient in dbias and a
streaming pass (bwd_dbias, E 8H + R 8H bytes) finishes it; its bytes are
reported with that kernel but are not part of the step's model above.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNELS = ["fwd", "fwd_merge", "bwd_rows", "bwd_rows_merge", "bwd_cols", "bwd_cols_merge",
           "bwd_dbias"]
CSRC = os.path.join(ROOT, "graph_transformer_sparse_amd", "csrc")


def byte_model(cfg, R, M, E, M_nz, reads_y):
    """Algorithmic bytes of each kernel (module docstring); reads_y: the row
    pass reads Y (with a bias it takes D = <dY, Y> up front)."""
    s = 4 if cfg.dtype == "f32" else 2
    H, D = cfg.heads, cfg.heads * cfg.head_dim
    b = 1 if cfg.bias else 0
    y = 1 if reads_y else 0
    return {
        "fwd": R * (4 + 2 * D * s + 4 * H) + E * (4 + 2 * D * s + 4 * H * b),
        "bwd_rows": R * (4 + (3 + y) * D * s + 12 * H) + E * (4 + 2 * D * s + 8 * H * b),
        "bwd_cols": M * (4 + 2 * D * s) + M_nz * 2 * D * s
        + E * (4 + 2 * D * s + 8 * H + (4 + 4 * H) * b),
    }


def aux_model(cfg, R, E):
    """Bytes of the pass that finishes dbias from its staged values (with a
    bias): every staged value read and written back once, plus two floats
    per row and head.  Not part of the step's algorithmic bytes above (the
    method itself needs no staging), but a kernel of the step."""
    if not cfg.bias:
        return {}
    return {"bwd_dbias": E * 8 * cfg.heads + R * 8 * cfg.heads}


# the sources that decide what the kernels read and write: the kernels, their
# device helpers and layouts, and the schedule they run over
KERNEL_SOURCES = ["attn.hip", "device.hpp", "layout.hpp", "prep.hip"]
# the dense projection kernels of the layer and what they include
PROJ_SOURCES = ["proj.hip", "device.hpp"]


def kernel_source_hash(kernel: str = "") -> str:
    h = hashlib.sha256()
    for f in (PROJ_SOURCES if kernel.startswith("proj") else KERNEL_SOURCES):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel and workload, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        m = re.match(r"^([a-z_]+):\s*(\S+)", line.strip())
        if m:
            rec[m.group(1)] = m.group(2)
    if rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


RTOL = {"f32": 1e-5, "bf16": 2e-2}
U32 = 2.0 ** -24


def _compare(got, ref, rtol, mag=None, head_axis=1):
    """Relative L2 error per head (the largest) and the largest elementwise
    error over its bound rtol |r| + rtol rms(r) + 8 u mag (mag: the oracle's
    sum of the absolute values of the terms of each element)."""
    axes = tuple(a for a in range(ref.ndim) if a != head_axis)
    rms = np.sqrt(np.mean(ref ** 2, axis=axes, keepdims=True))
    r2 = np.sqrt(np.sum(ref ** 2, axis=axes))
    d2 = np.sqrt(np.sum((got - ref) ** 2, axis=axes))
    rel = float(np.max(np.where(r2 > 0, d2 / np.maximum(r2, 1e-300), 0.0)))
    bound = rtol * np.abs(ref) + rtol * rms
    if mag is not None:
        bound = bound + 8 * U32 * mag
    err = np.abs(got - ref)
    ratio = float(np.max(np.where(err > 0, err / np.maximum(bound, 1e-300), 0.0)))
    return {"rel_l2": rel, "max_err_over_bound": ratio, "ok": bool(rel <= rtol and ratio <= 1.0)}


def _compare_lse(got, ref, rtol):
    ninf = np.isneginf(ref)
    same = bool(np.array_equal(np.isneginf(got), ninf))
    f = ~ninf
    ratio = float(np.max(np.abs(got[f] - ref[f]) / (rtol * np.maximum(1.0, np.abs(ref[f])))))\
        if f.any() else 0.0
    return {"max_err_over_bound": ratio, "ok": bool(same and ratio <= 1.0)}


def cpu_baseline(P, budget_s: float):
    """The oracle (fp64, OpenMP) timed on a row block of the same workload
    whose size is picked so the run takes about budget_s seconds."""
    from oracle import oracle as O
    cfg = P.cfg
    # the oracle works in float64: widen the inputs once, outside the timing
    Q, K, V, dY = (np.ascontiguousarray(x, dtype=np.float64) for x in (P.Q, P.K, P.V, P.dY))
    B = None if P.bias is None else np.ascontiguousarray(P.bias, dtype=np.float64)

    def run(k):
        ip = P.indptr[: k + 1]
        e = int(ip[-1])
        ix, bias = P.indices[:e], (B[:e] if B is not None else None)
        q, dy = np.ascontiguousarray(Q[:k]), np.ascontiguousarray(dY[:k])
        t = time.perf_counter()
        O.fwd(ip, ix, cfg.n_cols, q, K, V, bias, P.scale)
        O.bwd(ip, ix, cfg.n_cols, q, K, V, dy, bias, P.scale)
        return time.perf_counter() - t, e

    # calibrate on a small row block, then size the measured block
    def sized(budget):
        R = cfg.n_rows
        k = min(R, 4096)
        t, e = run(k)
        while t < 0.5 * budget / 15 and k < R:
            k = min(R, k * 4)
            t, e = run(k)
        if k < R and t < budget:
            k = min(R, int(k * budget / max(t, 1e-3)))
            t, e = run(k)
        runs, total = 1, t
        while total < budget:    # the whole workload is cheaper than the budget: repeat it
            t, e = run(k)
            runs += 1
            total += t
        return k, e, runs, total

    k, e, runs, total = sized(budget_s)
    cores = O.threads()
    out = {"value": e * runs / total / 1e9, "unit": "GEdges/s", "cores": cores,
           "kind": "oracle",
           "sample": (f"rows 0..{k - 1} of the {cfg.name} workload ({e} of {P.nnz} edges, "
                      f"all {cfg.n_cols} key/value rows), fwd+bwd in float64, {runs} run(s) "
                      f"in {total:.1f} s"),
           "cpu": cpu_model()}
    # the same oracle on one thread, on a quarter of the budget
    O.set_threads(1)
    try:
        k1, e1, runs1, total1 = sized(budget_s / 4)
    finally:
        O.set_threads(cores)
    out["single_thread"] = {"value": e1 * runs1 / total1 / 1e9, "unit": "GEdges/s",
                            "sample": f"rows 0..{k1 - 1}, {runs1} run(s) in {total1:.1f} s"}
    # the oracle's own CSR transpose of the whole graph (serial counting
    # sort), the step the GPU's prepare does once per graph
    t = time.perf_counter()
    O.transpose(P.indptr, P.indices, cfg.n_cols)
    out["transpose_s"] = time.perf_counter() - t
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


SUITE = ["tiny", "mid", "large", "shard", "hub"]   # the last one is the headline


def arith_dtype(storage: str) -> str:
    """The type the attention kernels compute in: float32 for either storage
    type (bf16 inputs are widened exactly, sums run in float32)."""
    return {"f32": "f32", "bf16": "f32"}[storage]


def unique_bytes(cfg, R, M, E, reads_y):
    """Compulsory bytes of one step: every array the two calls read or write,
    counted once per call (a lower bound on HBM traffic; gathers that come
    back from HBM more than once are what separates the kernels from it).
      forward : CSR (indptr, indices), Q, K, V, bias in; Y, lse out
      backward: CSR, its transpose (indptr_t, indices_t, perm), Q, K, V, dY,
                lse, bias (and Y when the row pass reads it) in; dQ, dK, dV,
                dbias out; the row statistics written once and read once."""
    s = 4 if cfg.dtype == "f32" else 2
    H, D = cfg.heads, cfg.heads * cfg.head_dim
    b = 1 if cfg.bias else 0
    csr = 4 * (R + 1) + 4 * E
    csr_t = 4 * (M + 1) + 8 * E
    fwd = csr + R * D * s + 2 * M * D * s + 4 * E * H * b + R * D * s + 4 * R * H
    bwd = (csr + csr_t + (2 + (1 if reads_y else 0)) * R * D * s + 2 * M * D * s + 4 * R * H
           + 4 * E * H * b + R * D * s + 2 * M * D * s + 4 * E * H * b + 2 * 8 * R * H)
    return fwd + bwd


def counter_record(workload: str, bias: bool):
    """Counter-measured bytes (FETCH_SIZE + WRITE_SIZE, calibrated) of one
    step's main kernels (the three passes, and with a bias the pass that
    finishes dbias) from the committed rocprofv3 records of this workload --
    a stored record, used only if every one was taken on the current kernel
    sources (the merges, under 0.3 % of a step, have no record)."""
    per = {}
    for k in ("fwd", "bwd_rows", "bwd_cols") + (("bwd_dbias",) if bias else ()):
        v = traffic_record(k, workload)
        if v is None:
            return None
        per[k] = v
    return {"bytes_per_step": sum(per.values()), "per_kernel": per,
            "source": f"profiles/traffic_{{{','.join(per)}}}_{workload}.txt",
            "source_hash": kernel_source_hash(), "stored": True}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None, choices=SUITE,
                    help="measure one workload only (default: all five, the hub workload "
                         "as the headline and the others in detail.configs)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0: skip it and the "
                         "parity check of the timed run)")
    ap.add_argument("--layer", action="store_true",
                    help="time a whole layer (dense projections + attention, fwd+bwd) "
                         "instead of the attention alone")
    ap.add_argument("--head-split", type=int, default=0, metavar="P",
                    help="time the head repack of graph parallelism with all-to-all for P "
                         "workers (split of Q, K, V and merge of Y) and the attention run on "
                         "the P head slices, instead of the plain attention step")
    ap.add_argument("--hidden", type=int, default=0, metavar="D",
                    help="run the workload's graph and head count at hidden size D (head_dim = "
                         "D / heads) instead of its own; the pages vary the hidden size over 64, "
                         "128 and 256 at 8 heads (Section 5.4, Figure 7)")
    ap.add_argument("--nodes", type=int, default=0, metavar="N",
                    help="mid only: the same R-MAT recipe on N nodes (a power of two); the "
                         "pages compare sparse graph attention at 64K, 128K and 512K nodes "
                         "(Section 5.4, Figure 6)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, 5 times "
                         "(calibrates the HBM byte counters against a known size)")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    from graph_transformer_sparse_amd import gtattn as T
    from graph_transformer_sparse_amd import inputs as I

    T.lib()
    single = args.config is not None or args.layer or args.head_split or args.hidden or args.nodes
    if single:
        cfg = I.CONFIGS[args.config or "mid"]
        if args.nodes:
            if cfg.name != "mid" or args.nodes < 2 or args.nodes & (args.nodes - 1):
                sys.exit("--nodes takes a power of two, with the mid workload")
            cfg = dataclasses.replace(cfg, n_rows=args.nodes, n_cols=args.nodes,
                                      desc=f"{cfg.desc}; {args.nodes} nodes")
        if args.hidden:
            if args.hidden % cfg.heads:
                sys.exit(f"--hidden {args.hidden} is not a multiple of the {cfg.heads} heads")
            cfg = dataclasses.replace(cfg, head_dim=args.hidden // cfg.heads,
                                      desc=f"{cfg.desc}; hidden {args.hidden}")
        if args.layer:
            return layer_bench(args, cfg)
        if args.head_split:
            return head_split_bench(args, cfg)
        plan = [cfg]
    else:
        plan = [I.CONFIGS[n] for n in SUITE]
    t_all = time.perf_counter()
    details = {}
    for k, cfg in enumerate(plan):
        head = k == len(plan) - 1
        print(f"bench: {cfg.name} ({'headline' if head else 'detail'})", file=sys.stderr,
              flush=True)
        r = run_workload(args, cfg, headline=head)
        if not head:
            details[cfg.name] = summary(r)
    line = r["line"]
    if details:
        line["detail"]["configs"] = details
    line["detail"]["bench_wall_s"] = time.perf_counter() - t_all
    bad = [n for n, d in [(cfg.name, summary(r))] + list(details.items())
           if d.get("parity") and d["parity"] != "pass"]
    if bad:
        print(f"bench: the GPU outputs of the timed run do NOT match the oracle on {bad}",
              file=sys.stderr)
    print(json.dumps(line), flush=True)


def summary(r):
    """The per-workload entry of detail.configs."""
    line = r["line"]
    d = line["detail"]
    par = r.get("parity")
    return {"workload": line["config"]["workload"], "nnz": line["config"]["nnz"],
            "storage": line["config"]["storage"], "bias": line["config"]["bias"],
            "ms_per_step": line["ms_per_step"], "GEdges_per_s": line["value"],
            "step_model_GB": d["step_model_GB"], "step_frac": d["step_frac"],
            "unique_GB": d["unique_GB"], "unique_frac": line["roofline"]["unique_frac"],
            "counter_frac": line["roofline"]["counter_frac"],
            "dominant": {"kernel": line["roofline"]["kernel"],
                         "ms_per_launch": d["kernels"][line["roofline"]["kernel"]]["ms_per_launch"],
                         "model_GBps": line["roofline"]["achieved"],
                         "frac": line["roofline"]["frac"]},
            "kernels_ms": {k: v["ms_per_launch"] for k, v in d["kernels"].items()},
            "parity": par["verdict"] if par else None,
            # the oracle's own rate in the parity check: fwd + bwd of the
            # whole graph in float64, all host cores, with the magnitudes of
            # its sums (the headline's cpu_baseline times it without them)
            "oracle_GEdges_per_s": (line["config"]["nnz"] / par["oracle_s"] / 1e9
                                    if par and par.get("oracle_s") else None),
            "parity_detail": par}


def run_workload(args, cfg, headline: bool):
    """One workload: generate it, prepare the graph, warm up, time the steps,
    check the timed run's outputs against the oracle (every output of the
    whole graph) and, for the headline, time the oracle on a bounded sample.
    Returns dict(line=<the JSON line of this workload>, parity=...)."""
    import torch

    from graph_transformer_sparse_amd import gtattn as T
    from graph_transformer_sparse_amd import inputs as I

    t0 = time.perf_counter()
    P = I.make_problem(cfg)
    gen_s = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    put = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(dev).contiguous()
    indptr, indices = put(P.indptr, torch.int32), put(P.indices, torch.int32)
    Q, K, V, dY = (put(x, tdt) for x in (P.Q, P.K, P.V, P.dY))
    bias = put(P.bias, torch.float32) if P.bias is not None else None
    R, M, E, H, dh = cfg.n_rows, cfg.n_cols, P.nnz, cfg.heads, cfg.head_dim

    # prepare once cold (the first call also loads the kernels' code), then
    # time a second, warm prepare of the same graph: the per-graph cost
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g = T.gt_graph_prepare(indptr, indices, M)
    torch.cuda.synchronize()
    prep_cold_ms = (time.perf_counter() - t0) * 1e3
    del g
    t0 = time.perf_counter()
    g = T.gt_graph_prepare(indptr, indices, M, validate=False)
    torch.cuda.synchronize()
    prep_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    assert T.gt_csr_validate(indptr, indices, M) == 0
    validate_ms = (time.perf_counter() - t0) * 1e3

    Y = torch.empty_like(Q)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dbias = torch.empty_like(bias) if bias is not None else None
    work = torch.empty(T.gt_attn_work_bytes(g, H, dh), dtype=torch.uint8, device=dev)

    def step():
        T.gt_attn_fwd(g, Q, K, V, bias, P.scale, work, Y, lse)
        T.gt_attn_bwd(g, Q, K, V, Y, lse, dY, bias, P.scale, work, dQ, dK, dV, dbias)

    def kernel_times():
        out = {}
        for k in KERNELS:
            tot, n = T.prof_query(k)
            if n:
                out[k] = {"ms_per_launch": tot / n, "launches": n}
        return out

    M_nz = int(np.count_nonzero(np.diff(T_np(g.indptr_t))))
    reads_y = T.bwd_reads_y(bias is not None)
    model = byte_model(cfg, R, M, E, M_nz, reads_y)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # device memory a step allocates beyond the resident inputs, outputs and
    # buffers (the library allocates nothing: expected 0)
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    step()
    torch.cuda.synchronize()
    memory = {"step_allocates_bytes": torch.cuda.max_memory_allocated() - base,
              "meta_bytes": g.meta.numel(), "work_bytes": work.numel(),
              # what the forward leaves for the backward besides its inputs and Y
              "saved_fwd_to_bwd_bytes": lse.numel() * lse.element_size(),
              # the same kept as one float32 attention weight per edge and head
              "per_edge_weights_bytes": E * H * 4}
    # three more untimed steps with every kernel timed: per-kernel times and
    # the dominant kernel
    T.prof_reset()
    T.prof_enable(True)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    kern = kernel_times()
    dominant = max((k for k in model if k in kern), key=lambda k: kern[k]["ms_per_launch"])
    # timed region: only the dominant kernel carries events
    T.prof_reset()
    T.prof_enable([dominant])
    cur = torch.cuda.current_stream()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(cur)
    for i in range(args.steps):
        step()
        marks[i + 1].record(cur)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    T.prof_enable(False)
    ms_step = elapsed * 1e3 / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    kern[dominant] = kernel_times()[dominant]
    for k, byt in list(model.items()) + list(aux_model(cfg, R, E).items()):
        if k in kern:
            kern[k]["model_GB"] = byt / 1e9
            kern[k]["GBps"] = byt / (kern[k]["ms_per_launch"] * 1e-3) / 1e9
            kern[k]["frac"] = kern[k]["GBps"] / HBM_PEAK_GBS
    ach = kern[dominant]["GBps"]
    # the committed counter records are for each workload's own shape and size
    shaped = not (args.hidden or args.nodes)
    traffic = traffic_record(dominant, cfg.name) if shaped else None
    counters = counter_record(cfg.name, cfg.bias) if shaped else None
    total_model = sum(model.values())
    uniq = unique_bytes(cfg, R, M, E, reads_y)
    step_s = ms_step * 1e-3
    graph_ms = graph_replay_ms(step, args.steps)
    copy_gbps = copy_rate_gbps()

    line = {
        "metric": "GEdges/s fused sparse-attn fwd+bwd, 1 MI355X; achieved HBM GB/s vs peak",
        "value": E / step_s / 1e9,
        "unit": "GEdges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arith_dtype(cfg.dtype),
        "data": "synthetic (seeded generators standing in for the pages' graphs)",
        "config": {"workload": f"{cfg.name}: {cfg.desc}", "nodes": R, "kv_nodes": M, "nnz": E,
                   "heads": H, "head_dim": dh, "storage": cfg.dtype, "bias": cfg.bias,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": ach, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                     "traffic": traffic,
                     # the step's compulsory bytes (every array once) over the step time
                     "unique_frac": uniq / step_s / 1e9 / HBM_PEAK_GBS,
                     # the step's counter-measured bytes (stored record) over the step time
                     "counter_frac": (counters["bytes_per_step"] / step_s / 1e9 / HBM_PEAK_GBS
                                      if counters else None)},
        "cpu_baseline": None,
        "detail": {"step_model_GB": total_model / 1e9,
                   "step_GBps": total_model / step_s / 1e9,
                   "step_frac": total_model / step_s / 1e9 / HBM_PEAK_GBS,
                   "unique_GB": uniq / 1e9,
                   "counters": counters,
                   "step_ms_events": {"mean": sum(per_step) / len(per_step),
                                      "min": per_step[0],
                                      "median": per_step[len(per_step) // 2]},
                   "kernels": kern, "memory": memory, "prep_ms": prep_ms,
                   "validate_ms": validate_ms,
                   # the first prepare of the process: CSR check included, and
                   # the kernels' code loaded
                   "prep_first_call_ms": prep_cold_ms,
                   "input_gen_s": gen_s,
                   "kernel_source_hash": kernel_source_hash(),
                   "graph_replay_ms_per_step": graph_ms,
                   "copy_GBps": copy_gbps,
                   "frac_of_copy": ach / copy_gbps if copy_gbps else None},
    }
    parity = None
    if args.cpu_budget > 0:
        # the outputs of the last timed step (the graph replays after it
        # recompute them bitwise), then free the device
        f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
        got = {"Y": f64(Y), "lse": f64(lse), "dQ": f64(dQ), "dK": f64(dK), "dV": f64(dV),
               "dbias": f64(dbias) if dbias is not None else None}
        del Q, K, V, dY, bias, Y, lse, dQ, dK, dV, dbias, work, g, indptr, indices
        torch.cuda.empty_cache()
        t0 = time.perf_counter()
        parity = parity_full(P, got)
        parity["oracle_s"] = time.perf_counter() - t0
        del got
        line["detail"]["parity"] = parity
        if headline:
            line["cpu_baseline"] = cpu_baseline(P, args.cpu_budget)
            line["cpu_baseline"]["parity"] = {k: parity[k] for k in ("verdict", "rtol", "compared")}
    return {"line": line, "parity": parity}


def parity_full(P, got):
    """The oracle's outputs on the whole graph (with the magnitudes of its
    sums) against the GPU's outputs of the timed run, at the tests'
    tolerance: every row of Y, lse, dQ (and dbias), every column of dK, dV."""
    from oracle import oracle as O
    cfg, rtol = P.cfg, RTOL[P.cfg.dtype]
    M = cfg.n_cols
    mag = {}
    Q, K, V, dY = (np.ascontiguousarray(x, dtype=np.float64) for x in (P.Q, P.K, P.V, P.dY))
    B = None if P.bias is None else np.ascontiguousarray(P.bias, dtype=np.float64)
    rY, rl = O.fwd(P.indptr, P.indices, M, Q, K, V, B, P.scale, mag=mag)
    rep = {"Y": _compare(got["Y"], rY, rtol, mag.pop("Y")),
           "lse": _compare_lse(got["lse"], rl, 1e-5 if cfg.dtype == "f32" else 1e-4)}
    del rY, rl
    rQ, rK, rV, rB = O.bwd(P.indptr, P.indices, M, Q, K, V, dY, B, P.scale, mag=mag)
    rep["dQ"] = _compare(got["dQ"], rQ, rtol, mag.pop("dQ"))
    rep["dK"] = _compare(got["dK"], rK, rtol, mag.pop("dK"))
    rep["dV"] = _compare(got["dV"], rV, rtol, mag.pop("dV"))
    if rB is not None:
        rep["dbias"] = _compare(got["dbias"], rB, rtol)
    what = "Y, lse, dQ" + (", dbias" if rB is not None else "") + " of every row, dK, dV of every column"
    return {"verdict": "pass" if all(r["ok"] for r in rep.values()) else "FAIL",
            "rtol": rtol, "compared": f"{what}, from the timed run", "tensors": rep}


def copy_rate_gbps(mib: int = 1024, reps: int = 10):
    """Bytes moved (read + write) per second by a plain device-to-device copy
    of `mib` MiB, timed with events after the timed region: the rate that is
    practically achievable for streaming reads and writes on this GPU."""
    import torch
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    rate = 2 * src.numel() * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    return rate


def graph_replay_ms(step, reps):
    """The same step captured once into a HIP graph and replayed `reps`
    times (after the timed region; it does not change `value`): what a
    caller that captures the step saves in launch overhead.  None if the
    capture fails."""
    import torch
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / reps
    except Exception as e:      # report, never fail the benchmark for it
        print(f"graph replay skipped: {e}", file=sys.stderr)
        return None


def T_np(t):
    return t.cpu().numpy()


MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}


def proj_model(n, d, s):
    """Algorithmic bytes and flops of each projection kernel (every node
    array read or written once, weights once, the weight gradient's per-slot
    fp32 partials written and read once; the slot count is the library's:
    a multiple of 8, at most 64 (d = 256 or float32) or 128, at most the
    32-row steps)."""
    steps = -(-max(n, 1) // 32)
    chunks = min(64 if (d >= 256 or s == 4) else 128, -(-steps // 8) * 8)
    nd = n * d * s
    return {
        "proj_qkv": (4 * nd + 3 * d * d * s, 3 * 2 * n * d * d),
        "proj_out": (3 * nd + d * d * s, 2 * n * d * d),
        "proj_bwd_data": (5 * nd + 4 * d * d * s, 4 * 2 * n * d * d),
        "proj_bwd_weight": (5 * nd + 4 * d * d * 4 * (2 * chunks + 1), 4 * 2 * n * d * d),
    }


def layer_bench(args, cfg):
    """A whole layer, fwd + bwd: Q/K/V = X W, attention, Z = X W_o + Y, and
    every gradient.  Same JSON line; `detail` adds the projection kernels'
    rates against their byte model and against the matrix-core peak."""
    import torch

    from graph_transformer_sparse_amd import gtattn as T
    from graph_transformer_sparse_amd import inputs as I

    if cfg.n_rows != cfg.n_cols:
        print("--layer needs a square graph (every node a query and a key)", file=sys.stderr)
        sys.exit(2)
    t0 = time.perf_counter()
    P = I.make_problem(cfg)
    n, H, dh, E = cfg.n_rows, cfg.heads, cfg.head_dim, P.nnz
    d = H * dh
    X, W, dZ = I.layer_inputs(cfg.idx, n, d, cfg.dtype)
    gen_s = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    put = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(dev).contiguous()
    g = T.gt_graph_prepare(put(P.indptr, torch.int32), put(P.indices, torch.int32), n)
    Xd, dZd = put(X, tdt), put(dZ, tdt)
    Wd = {k: put(v, tdt) for k, v in W.items()}
    bias = put(P.bias, torch.float32) if P.bias is not None else None
    shp = (n, H, dh)
    Y = torch.empty(shp, dtype=tdt, device=dev)
    lse = torch.empty((n, H), dtype=torch.float32, device=dev)
    dQ, dK, dV = (torch.empty(shp, dtype=tdt, device=dev) for _ in range(3))
    dbias = torch.empty_like(bias) if bias is not None else None
    work = torch.empty(T.gt_attn_work_bytes(g, H, dh), dtype=torch.uint8, device=dev)
    pwork = torch.empty(T._proj_lib().gt_proj_work_bytes(n, d), dtype=torch.uint8, device=dev)
    ev = {}

    def timed(name, fn):
        if name in ev:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            out = fn()
            b.record()
            ev[name].append((a, b))
            return out
        return fn()

    def step():
        Q, K, V = timed("proj_qkv", lambda: T.gt_proj_qkv(Xd, Wd["q"], Wd["k"], Wd["v"]))
        T.gt_attn_fwd(g, Q.view(shp), K.view(shp), V.view(shp), bias, P.scale, work, Y, lse)
        timed("proj_out", lambda: T.gt_proj_out(Xd, Wd["o"], Y.view(n, d)))
        T.gt_attn_bwd(g, Q.view(shp), K.view(shp), V.view(shp), Y, lse, dZd.view(shp), bias,
                      P.scale, work, dQ, dK, dV, dbias)
        args4 = (dZd, dQ.view(n, d), dK.view(n, d), dV.view(n, d))
        timed("proj_bwd_data", lambda: T.gt_proj_bwd_data(*args4, Wd["o"], Wd["q"], Wd["k"], Wd["v"]))
        timed("proj_bwd_weight", lambda: T.gt_proj_bwd_weight(Xd, *args4, work=pwork))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # three profiled steps: every kernel's time
    for k in ("proj_qkv", "proj_out", "proj_bwd_data", "proj_bwd_weight"):
        ev[k] = []
    T.prof_reset()
    T.prof_enable(True)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    T.prof_enable(False)
    kern = {}
    for k in KERNELS:
        tot, c = T.prof_query(k)
        if c:
            kern[k] = {"ms_per_launch": tot / c, "launches": c}
    for k, lst in ev.items():
        kern[k] = {"ms_per_launch": sum(a.elapsed_time(b) for a, b in lst) / len(lst),
                   "launches": len(lst)}
    ev.clear()
    s = 4 if cfg.dtype == "f32" else 2
    M_nz = int(np.count_nonzero(np.diff(T_np(g.indptr_t))))
    model = byte_model(cfg, n, n, E, M_nz, T.bwd_reads_y(bias is not None))
    pm = proj_model(n, d, s)
    for k, (byt, flops) in pm.items():
        t = kern[k]["ms_per_launch"] * 1e-3
        kern[k].update(model_GB=byt / 1e9, GBps=byt / t / 1e9, TFLOPs=flops / t / 1e12,
                       mfma_frac=flops / t / 1e12 / MFMA_PEAK_TFLOPS[cfg.dtype])
    for k in model:
        if k in kern:
            kern[k]["model_GB"] = model[k] / 1e9
            kern[k]["GBps"] = model[k] / (kern[k]["ms_per_launch"] * 1e-3) / 1e9
    dominant = max(kern, key=lambda k: kern[k]["ms_per_launch"])
    T.prof_reset()
    if dominant in KERNELS:
        T.prof_enable([dominant])
    else:
        ev[dominant] = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    T.prof_enable(False)
    if dominant in KERNELS:
        tot, c = T.prof_query(dominant)
        kern[dominant]["ms_per_launch"] = tot / c
    else:
        lst = ev[dominant]
        kern[dominant]["ms_per_launch"] = sum(a.elapsed_time(b) for a, b in lst) / len(lst)
    dom_bytes = model[dominant] if dominant in model else pm[dominant][0]
    ach = dom_bytes / (kern[dominant]["ms_per_launch"] * 1e-3) / 1e9
    ms_step = elapsed * 1e3 / args.steps
    line = {
        "metric": "GEdges/s sparse graph attention layer (dense projections + attention) fwd+bwd, 1 MI355X",
        "value": E / (ms_step * 1e-3) / 1e9,
        "unit": "GEdges/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        # the projections multiply in the storage type (fp32 accumulation)
        "dtype": cfg.dtype,
        "data": "synthetic (seeded generators standing in for the pages' graphs)",
        "config": {"workload": f"{cfg.name} layer: {cfg.desc}", "nodes": n, "nnz": E,
                   "heads": H, "head_dim": dh, "d": d, "storage": cfg.dtype,
                   "bias": cfg.bias, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": ach, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                     "traffic": (None if (args.hidden or args.nodes)
                                 else traffic_record(dominant, cfg.name))},
        "cpu_baseline": None,
        "detail": {"kernels": kern, "input_gen_s": gen_s,
                   "kernel_source_hash": kernel_source_hash()},
    }
    if args.cpu_budget > 0:
        line["cpu_baseline"] = layer_cpu_baseline(P, X, W, dZ)
    print(json.dumps(line), flush=True)


def layer_cpu_baseline(P, X, W, dZ):
    """The layer oracle (float64; numpy's matmul for the projections, the C
    oracle with OpenMP for the attention) on the whole workload, once."""
    from oracle import layer as L
    from oracle import oracle as O
    cfg = P.cfg
    store = "bf16" if cfg.dtype == "bf16" else None
    t = time.perf_counter()
    L.layer_fwd(P.indptr, P.indices, X, W, cfg.heads, P.bias, P.scale, store)
    L.layer_bwd(P.indptr, P.indices, X, W, cfg.heads, dZ, P.bias, P.scale, store)
    dt = time.perf_counter() - t
    return {"value": P.nnz / dt / 1e9, "unit": "GEdges/s", "cores": O.threads(),
            "kind": "oracle",
            "sample": (f"the whole {cfg.name} layer once: forward and backward in float64 "
                       f"(projections by numpy matmul, attention by the C oracle) in {dt:.1f} s"),
            "cpu": cpu_model()}


def head_split_bench(args, cfg):
    """Graph parallelism with all-to-all, its on-GPU part with the P workers
    on one GPU: split Q, K, V (and the bias) into P head slices, attention
    fwd+bwd on each slice over the whole graph, merge Y, lse and the
    gradients.  The repack kernels are pure copies: `roofline` is theirs
    (2 R D s bytes per split or merge of a [R, H, dh] tensor)."""
    import torch

    from graph_transformer_sparse_amd import gtattn as T
    from graph_transformer_sparse_amd import inputs as I

    parts = args.head_split
    if cfg.heads % parts:
        print(f"{cfg.heads} heads do not divide among {parts} workers", file=sys.stderr)
        sys.exit(2)
    P = I.make_problem(cfg)
    dev = torch.device("cuda:0")
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    put = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(dev).contiguous()
    g = T.gt_graph_prepare(put(P.indptr, torch.int32), put(P.indices, torch.int32), cfg.n_cols)
    Q, K, V, dY = (put(x, tdt) for x in (P.Q, P.K, P.V, P.dY))
    bias = put(P.bias, torch.float32) if P.bias is not None else None
    R, H, dh = Q.shape
    s = Q.element_size()

    def step():
        return T.attn_head_sliced(g, Q, K, V, dY, bias, P.scale, parts)

    # the repack alone: split of Q into a preallocated buffer, merge back
    qs = T.gt_head_split(Q, parts)
    qm = torch.empty_like(Q)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        T.gt_head_split(Q, parts, out=qs)
        T.gt_head_merge(qs, out=qm)
        step()
    torch.cuda.synchronize()
    reps = max(args.steps, 10)
    a, b, c = ev(), ev(), ev()
    a.record()
    for _ in range(reps):
        T.gt_head_split(Q, parts, out=qs)
    b.record()
    for _ in range(reps):
        T.gt_head_merge(qs, out=qm)
    c.record()
    torch.cuda.synchronize()
    assert torch.equal(qm, Q)
    nbytes = 2 * R * H * dh * s
    split_ms, merge_ms = a.elapsed_time(b) / reps, b.elapsed_time(c) / reps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ach = nbytes / (split_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": f"GEdges/s sparse graph attention fwd+bwd on {parts} head slices "
                  "(repack + per-slice attention), 1 MI355X",
        "value": P.nnz / (ms_step * 1e-3) / 1e9, "unit": "GEdges/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": arith_dtype(cfg.dtype),
        "data": "synthetic (seeded generators standing in for the pages' graphs)",
        "config": {"workload": f"{cfg.name}: {cfg.desc}", "parts": parts, "nodes": R,
                   "heads": H, "head_dim": dh, "storage": cfg.dtype, "bias": cfg.bias,
                   "parallelism": "single GPU (the P workers' head slices in turn)"},
        "roofline": {"bound": "hbm", "kernel": "head_split", "achieved": ach,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                     "traffic": None},
        # the attention on head slices is the same mathematics as on all
        # heads at once: the oracle's fwd + bwd of the workload stands beside it
        "cpu_baseline": cpu_baseline(P, args.cpu_budget) if args.cpu_budget > 0 else None,
        "detail": {"head_split_ms": split_ms, "head_merge_ms": merge_ms,
                   "head_merge_GBps": nbytes / (merge_ms * 1e-3) / 1e9,
                   "bytes_per_repack": nbytes},
    }), flush=True)


if __name__ == "__main__":
    main()
