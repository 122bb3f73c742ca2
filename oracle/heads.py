"""CPU oracle of the head repack of graph parallelism with all-to-all.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use this module; the GPU path never does.

"Scalable and Adaptive Parallel Training of Graph Transformer on Large
Graphs", Section 3.2 (GP-A2A) and Algorithm 2: worker k of p holds the
node-partitioned block [N/p, h, d'] of Q, K, V; after the all-to-all it holds
the head-partitioned [N, h/p, d'], i.e. all N nodes with heads
k*h/p .. (k+1)*h/p - 1; the attention runs on those heads over the whole
graph, and the reverse all-to-all returns Y to [N/p, h, d'].

head_split / head_merge are the layout transforms written out (the on-GPU
halves of the exchange; with all nodes on one GPU, head_split part r is
exactly worker r's head-partitioned tensor).  all_to_all_node_to_head and
all_to_all_head_to_node state what each worker holds after each exchange as
an explicit index map from the workers' blocks (nodes numbered block after
block, worker order), so that the transforms can be pinned to it.
"""
from __future__ import annotations

import numpy as np


def head_split(x, parts: int):
    """[rows, heads, ...] -> [parts, rows, heads/parts, ...]."""
    x = np.asarray(x)
    rows, heads = x.shape[0], x.shape[1]
    assert heads % parts == 0, "heads must divide among the workers"
    hp = heads // parts
    out = np.empty((parts, rows, hp) + x.shape[2:], dtype=x.dtype)
    for r in range(parts):
        out[r] = x[:, r * hp:(r + 1) * hp]
    return out


def head_merge(p):
    """[parts, rows, hp, ...] -> [rows, parts*hp, ...] (concatenate the
    slices along the head dimension, slice r first)."""
    p = np.asarray(p)
    return np.concatenate([p[r] for r in range(p.shape[0])], axis=1)


def _owners(counts):
    """For nodes numbered block after block: the worker that holds each node
    and the node's row in that worker's block."""
    counts = np.asarray(counts, np.int64)
    starts = np.concatenate([[0], np.cumsum(counts)])
    owner = np.repeat(np.arange(counts.size), counts)
    return owner, np.arange(starts[-1]) - starts[owner], starts


def all_to_all_node_to_head(blocks):
    """Worker k holds blocks[k] = [n_k, h, d'].  Returns what each worker r
    holds after the exchange, [N, h/p, d'] with N = sum n_k:
        out_r[n, j] = blocks[k][n - start_k, r * h/p + j]
    for the worker k whose block holds node n."""
    p = len(blocks)
    hp = blocks[0].shape[1] // p
    owner, local, _ = _owners([b.shape[0] for b in blocks])
    out = []
    for r in range(p):
        o = np.empty((owner.size, hp) + blocks[0].shape[2:], dtype=blocks[0].dtype)
        for n in range(owner.size):
            for j in range(hp):
                o[n, j] = blocks[owner[n]][local[n], r * hp + j]
        out.append(o)
    return out


def all_to_all_head_to_node(slices, counts):
    """The reverse exchange: worker r holds slices[r] = [N, h/p, d'] for its
    heads, and worker k owns counts[k] consecutive nodes.  Returns what each
    worker k holds afterwards, [counts[k], h, d']:
        back_k[m, r * h/p + j] = slices[r][start_k + m, j]."""
    p = len(slices)
    hp = slices[0].shape[1]
    _, _, starts = _owners(counts)
    out = []
    for k in range(p):
        o = np.empty((int(counts[k]), p * hp) + slices[0].shape[2:], dtype=slices[0].dtype)
        for m in range(int(counts[k])):
            for r in range(p):
                for j in range(hp):
                    o[m, r * hp + j] = slices[r][starts[k] + m, j]
        out.append(o)
    return out
