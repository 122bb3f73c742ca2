/*
 * gt_proj.h -- C ABI of the dense parts of one sparse graph attention layer
 * (libgtattn.so), around the attention of gt_attn.h.
 *
 * The layer ("Scalable and Adaptive Parallel Training of Graph Transformer
 * on Large Graphs", Section 2.1, Eq. 3 and 5):
 *   Q = X W_Q,  K = X W_K,  V = X W_V          (gt_proj_qkv)
 *   Y = sparse graph attention (A, Q, K, V)    (gt_attn_fwd)
 *   Z = X W_o + Y                              (gt_proj_out; Z is the layer output X')
 * and, given dZ, its gradients:
 *   (dQ, dK, dV) from gt_attn_bwd with dY = dZ,
 *   dX = dZ W_o^T + dQ W_Q^T + dK W_K^T + dV W_V^T   (gt_proj_bwd_data)
 *   dW_o = X^T dZ, dW_Q = X^T dQ, dW_K = X^T dK, dW_V = X^T dV  (gt_proj_bwd_weight)
 *
 * Conventions (as gt_attn.h): device pointers owned by the caller, 16-byte
 * aligned; calls enqueue on `stream` (a hipStream_t, NULL = default) and
 * return; status codes only, checked on the host before anything is
 * enqueued.  Node arrays X, Q, K, V, Y, Z and their gradients are [n, d]
 * row-major in dtype dt (d = heads * head_dim, so [n, d] is the [n, heads,
 * head_dim] layout of gt_attn.h); weights W_* are [d, d] row-major in dt and
 * act as X W; weight gradients dW_* are [d, d] float32.  d in {64, 128, 256}.
 * No output may overlap an input or another output (gt_proj_out, for one, has
 * two workgroups share a node strip of X at d = 256, each writing half of Z).
 * The products run on the matrix cores with float32 accumulation; bf16
 * outputs are rounded to nearest even.  Results are bitwise deterministic:
 * the weight gradients sum per-slot partial products (slots of contiguous
 * node rows, a function of n, d and dt only) in slot order.
 * Errors: GT_E_NULL, GT_E_ALIGN, GT_E_DTYPE, GT_E_SHAPE (d), GT_E_ARG (n),
 * GT_E_WORKSPACE, GT_E_HIP.
 */
#ifndef GT_PROJ_H
#define GT_PROJ_H

#include <stddef.h>
#include <stdint.h>

#include "gt_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Q = X W_Q, K = X W_K, V = X W_V (Eq. 3), one launch over X. */
gt_status gt_proj_qkv(int64_t n, int32_t d, gt_dtype dt, const void *X, const void *Wq,
                      const void *Wk, const void *Wv, void *Q, void *K, void *V, void *stream);

/* Z = X W_o + Y (Eq. 5). */
gt_status gt_proj_out(int64_t n, int32_t d, gt_dtype dt, const void *X, const void *Wo,
                      const void *Y, void *Z, void *stream);

/* dX = dZ W_o^T + dQ W_Q^T + dK W_K^T + dV W_V^T, one launch. */
gt_status gt_proj_bwd_data(int64_t n, int32_t d, gt_dtype dt, const void *dZ, const void *dQ,
                           const void *dK, const void *dV, const void *Wo, const void *Wq,
                           const void *Wk, const void *Wv, void *dX, void *stream);

/* Bytes of `work` gt_proj_bwd_weight needs (per-slot partial products),
 * enough for either dtype. */
size_t gt_proj_work_bytes(int64_t n, int32_t d);

/* dW_o = X^T dZ, dW_Q = X^T dQ, dW_K = X^T dK, dW_V = X^T dV (float32). */
gt_status gt_proj_bwd_weight(int64_t n, int32_t d, gt_dtype dt, const void *X, const void *dZ,
                             const void *dQ, const void *dK, const void *dV, float *dWo,
                             float *dWq, float *dWk, float *dWv, void *work, size_t work_bytes,
                             void *stream);

#ifdef __cplusplus
}
#endif
#endif /* GT_PROJ_H */
