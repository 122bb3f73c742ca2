"""CPU oracle of the head repack of graph parallelism with all-to-all.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use this module; the GPU path never does.

"Scalable and Adaptive Parallel Training of Graph Transformer on Large
Graphs", Section 3.2 (GP-A2A) and Algorithm 2: worker k of p holds the
node-partitioned block [N/p, h, d'] of Q, K, V; an all-to-all turns it into
the head-partitioned [N, h/p, d'] (all nodes, heads k*h/p .. (k+1)*h/p - 1),
the attention runs on those heads over the whole graph, and a second
all-to-all returns Y to [N/p, h, d'].  The blog page's GP-A2A notes
(section 6.3) give the data movement: cut the head dimension into p equal
chunks, send chunk r to worker r, concatenate what arrives along the node
dimension.

head_split / head_merge are the layout transforms written out (the on-GPU
halves of the exchange; with all nodes on one GPU, head_split part r is
exactly worker r's head-partitioned tensor).  all_to_all_node_to_head and
all_to_all_head_to_node simulate the exchange itself among p workers as
lists of arrays, following the pages' steps, so that the transforms can be
pinned to it.
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


def all_to_all_node_to_head(blocks):
    """Worker k holds blocks[k] = [n_k, h, d']; returns what each worker r
    holds after the exchange: [sum n_k, h/p, d'], its head chunk of every
    node, blocks in worker order."""
    p = len(blocks)
    heads = blocks[0].shape[1]
    hp = heads // p
    # worker k cuts its heads into p chunks and sends chunk r to worker r
    sent = [[blocks[k][:, r * hp:(r + 1) * hp] for r in range(p)] for k in range(p)]
    # worker r concatenates the chunks it received along the node dimension
    return [np.concatenate([sent[k][r] for k in range(p)], axis=0) for r in range(p)]


def all_to_all_head_to_node(slices, counts):
    """The return exchange: worker r holds slices[r] = [N, h/p, d'] for its
    heads; worker k owns counts[k] consecutive nodes.  Returns each worker's
    [counts[k], h, d']."""
    p = len(slices)
    starts = np.concatenate([[0], np.cumsum(counts)])
    # worker r cuts its nodes into the p owners' blocks and sends block k to k
    sent = [[slices[r][starts[k]:starts[k + 1]] for k in range(p)] for r in range(p)]
    # worker k concatenates the head chunks it received along the head dimension
    return [np.concatenate([sent[r][k] for r in range(p)], axis=1) for k in range(p)]
