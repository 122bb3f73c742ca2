/*
 * gt_heads.h -- C ABI of the head repack of graph parallelism with
 * all-to-all (libgtattn.so).
 *
 * "Scalable and Adaptive Parallel Training of Graph Transformer on Large
 * Graphs", Section 3.2 (GP-A2A) and Algorithm 2: a worker that holds all
 * heads of its node block, [N/p, h, d'], exchanges it by all-to-all so that
 * it holds its share of the heads for all nodes, [N, h/p, d'], computes the
 * attention on those heads, and a second all-to-all brings Y back to
 * [N/p, h, d'] (the backward pass mirrors both).  The blog page's GP-A2A
 * implementation notes (section 6.3) spell out the data movement: the head
 * dimension is cut into p equal chunks that are sent to the p workers, and
 * what arrives is concatenated along the node dimension.
 *
 * These two calls are the on-GPU halves of that exchange:
 *   gt_head_split: src [rows, heads, head_bytes] -> dst [parts][rows, heads/parts, head_bytes]
 *                  (dst part r holds heads r*heads/parts .. (r+1)*heads/parts - 1; it is
 *                  the send buffer for worker r, and with all nodes on one GPU it is
 *                  exactly worker r's head-partitioned tensor)
 *   gt_head_merge: the inverse, [parts][rows, heads/parts, head_bytes] -> [rows, heads, head_bytes]
 *                  (what a worker does with the p chunks of Y it receives)
 * A head is head_bytes opaque bytes (head_dim * element size: features in
 * any dtype, or one float32 per head for a per-edge bias [E, heads]), so the
 * result is an exact byte permutation.
 *
 * Conventions: device pointers owned by the caller, src and dst not
 * overlapping; calls enqueue on `stream` (a hipStream_t, NULL = default) and
 * return.  Requires parts >= 1, heads % parts == 0 (Section 3.2: heads are
 * what is divided among workers), head_bytes > 0 a multiple of 4, rows >= 0,
 * src and dst 4-byte aligned (16-byte alignment and chunks that are a
 * multiple of 16 bytes take the 16-byte path).  Errors: GT_E_NULL, GT_E_ALIGN,
 * GT_E_SHAPE (heads % parts, head_bytes), GT_E_ARG (rows, parts), GT_E_HIP.
 */
#ifndef GT_HEADS_H
#define GT_HEADS_H

#include <stddef.h>
#include <stdint.h>

#include "gt_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* [rows, heads, head_bytes] -> [parts][rows, heads/parts, head_bytes]. */
gt_status gt_head_split(int64_t rows, int32_t heads, int32_t head_bytes, int32_t parts,
                        const void *src, void *dst, void *stream);

/* [parts][rows, heads/parts, head_bytes] -> [rows, heads, head_bytes]. */
gt_status gt_head_merge(int64_t rows, int32_t heads, int32_t head_bytes, int32_t parts,
                        const void *src, void *dst, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GT_HEADS_H */
