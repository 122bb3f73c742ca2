/*
 * gt_attn.h -- C ABI of the MI355X (gfx950) sparse graph attention library
 * (libgtattn.so).
 *
 * The operation is multi-head sparse graph attention over a CSR adjacency,
 * as defined in "Scalable and Adaptive Parallel Training of Graph
 * Transformer on Large Graphs" (Section 2.1, Eq. 1-5; backward operator
 * structure in Section 2.2):
 *
 *   for every stored edge e = (i, j) of A and every head h
 *     s_e,h   = scale * <Q[i,h,:], K[j,h,:]> + bias[e,h]       (SDDMM)
 *     U_e,h   = exp(s_e,h) / sum_{e' in row i} exp(s_e',h)     (softmax over
 *               the stored neighbours j in N(i) of row i only, Eq. 1-2)
 *     Y[i,h,:] = sum_{e in row i} U_e,h V[j,h,:]                (SpMM, Eq. 5)
 *     lse[i,h] = log sum_{e in row i} exp(s_e,h)
 *   backward (the gradients of the same expression):
 *     dU_e,h = <dY[i,h,:], V[j,h,:]>                            (sampled SDDMM)
 *     dS_e,h = U_e,h (dU_e,h - sum_{e' in row i} U_e',h dU_e',h)
 *     dQ[i,h,:] = scale * sum_{e in row i}    dS_e,h K[j,h,:]   (SpMM)
 *     dK[j,h,:] = scale * sum_{e in column j} dS_e,h Q[i,h,:]   (SpMM, A^T)
 *     dV[j,h,:] =         sum_{e in column j} U_e,h dY[i,h,:]   (SpMM, A^T)
 *     dbias[e,h] = dS_e,h
 *
 * Readings of the method: row i is the query (destination) node and column j
 * the key/value (source) node; head h owns channels [h*dh, (h+1)*dh) of a
 * node's contiguous H*dh feature row (the [n, h, d'] layout of the paper's
 * Algorithm 1); the scale is passed in (1/sqrt(dh) in the paper's use); the
 * optional per-edge bias is added, unscaled, to the score before the softmax
 * (the MegaGraph page, Section III-A1, mechanism 3).  An empty row gives
 * Y = 0, lse = -inf and dQ = 0; an empty column gives dK = dV = 0.
 *
 * Conventions shared by every entry point
 *   - Every array argument is DEVICE memory, owned by the caller.  The
 *     library never allocates, frees or keeps device memory between calls;
 *     scratch comes in through the `meta` / `work` arguments, sized by the
 *     *_bytes query functions.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     work on it and return, except gt_graph_prepare and gt_csr_validate,
 *     which synchronise that stream before returning (both run once per
 *     graph).  gt_attn_fwd and gt_attn_bwd enqueue kernels only (no
 *     memsets, copies or host synchronisation), so a caller may capture
 *     them into a HIP graph and replay it.
 *   - Dense features are row-major [n, heads, head_dim] (node-major, heads
 *     contiguous), in the dtype `dt`; rows start 16-byte aligned.
 *     Supported: head_dim in {8, 16, 32, 64, 128}, heads in {1, 2, 4, 8},
 *     and heads * head_dim * sizeof(dt) <= 1024 bytes (a row fits one
 *     wavefront at 16 bytes a lane).  head_dim 8 is the paper's hidden
 *     size 64 over 8 heads (Section 5.4, Figure 7).  Softmax statistics (lse),
 *     bias and dbias are float32.  All arithmetic is float32; bf16 inputs
 *     are widened exactly and bf16 outputs are rounded to nearest even.
 *   - CSR: indptr[n_rows + 1], indices[nnz], int32, columns strictly
 *     ascending within a row, 0 <= column < n_cols.  The content is trusted
 *     (gt_csr_validate checks it); n_rows, n_cols, nnz < 2^31 - 1.
 *   - Results are bitwise deterministic: no floating-point atomics, fixed
 *     summation orders, and the CSR transpose is stable.
 *   - Errors are reported only through the gt_status return value (with a
 *     per-thread detail string from gt_last_error); a call that fails its
 *     argument checks launches nothing and touches no device memory.
 */
#ifndef GT_ATTN_H
#define GT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gt_status;
enum {
  GT_OK = 0,
  GT_E_NULL = 1,        /* a required pointer is NULL */
  GT_E_ARG = 2,         /* a size / count / threshold is out of range */
  GT_E_DTYPE = 3,       /* unknown dtype */
  GT_E_SHAPE = 4,       /* heads / head_dim combination not supported */
  GT_E_ALIGN = 5,       /* a feature array is not 16-byte aligned */
  GT_E_UNSUPPORTED = 6, /* bias and dbias not given together */
  GT_E_WORKSPACE = 7,   /* meta / work buffer smaller than required */
  GT_E_CSR = 8,         /* gt_csr_validate found a malformed CSR */
  GT_E_HIP = 9          /* the HIP runtime reported an error */
};

typedef enum { GT_F32 = 0, GT_BF16 = 1 } gt_dtype;

/* Degree-ordered work schedule of the segments (rows of the CSR, or rows
 * of its transpose = columns of A).  Definition:
 *   order    = segment ids sorted by degree descending, ties by ascending id,
 *              except that in the schedule over the rows of A (`rows`) a
 *              small segment (degree <= t_small) counts its degree rounded
 *              down to a multiple of 4, so each such class runs in id order;
 *   n_big    = #segments with degree >  t_mid   (they lead `order`);
 *   n_mid    = #segments with t_small < degree <= t_mid (next in `order`);
 *   n_small  = #segments with degree <= t_small (the tail of `order`);
 *   pieces   = every big segment s, in `order`, with degree d is cut into
 *              nch = ceil(d / chunk) pieces; piece c is (s, ptr[s] +
 *              floor(c d / nch), ptr[s] + floor((c+1) d / nch), slot), where
 *              slot is the piece's index in this segment-major enumeration
 *              if nch > 1, else -1;
 *   items    = [n_items][4] int32: the pieces, dealt by position: piece c of
 *              nch gets q = floor(64 (2c + 1) / (2 nch)) and queue
 *              x = floor(q / 8), a queue being ordered by (q, segment-major
 *              index); block k of the list (items 4k .. 4k + 3) takes its
 *              items from queue k mod 8 and, once that queue is empty, from
 *              queues k + 1, k + 2, ... (mod 8) in turn.  (Workgroups of
 *              four wavefronts go to the eight XCDs in turn, so each XCD
 *              works on one eighth of every big segment's range at a time.)
 *   merges   = [n_merges][3] int32: (s, first slot, nch) for every big
 *              segment with nch > 1 (its pieces' slots are first ..
 *              first + nch - 1);
 *   spans    = [n_seg][2] int32: (ptr[order[k]], ptr[order[k] + 1]), the
 *              extent of the k-th segment of `order` (so a kernel finds a
 *              segment's nonzeros without a second, dependent load).
 * Big pieces and mid segments are each processed by one 64-lane wavefront;
 * small segments by a group of lanes inside a wavefront.  Split segments
 * are reduced afterwards in piece order, so results are deterministic. */
typedef struct gt_sched {
  int32_t *order;   /* [n_seg] */
  int32_t *items;   /* [cap][4] */
  int32_t *merges;  /* [cap][3] */
  int32_t *spans;   /* [n_seg][2] */
  int64_t n_seg, n_big, n_mid, n_small, n_items, n_merges, max_degree;
} gt_sched;

/* A prepared graph.  Filled by gt_graph_prepare; the device arrays it points
 * to live in the caller's `meta` buffer (and the caller's indptr/indices),
 * so the struct is valid as long as those buffers are. */
typedef struct gt_graph {
  int64_t n_rows, n_cols, nnz;
  const int32_t *indptr, *indices;   /* the caller's CSR, [n_rows+1], [nnz] */
  int32_t *indptr_t;                 /* [n_cols+1] CSR^T row pointer */
  int32_t *indices_t;                /* [nnz] source row of transposed entry t */
  int32_t *perm;                     /* [nnz] CSR edge id of transposed entry t */
  gt_sched rows, cols;               /* schedules over rows of A and of A^T */
  int32_t t_small, t_mid, chunk;     /* thresholds the schedules were built with */
  int32_t reserved;
} gt_graph;

/* ---- graph preparation (once per graph) ------------------------------- */

/* Bytes of device memory gt_graph_prepare needs in `meta` for this graph
 * size and chunk (persistent arrays plus sort scratch).  0 on bad sizes. */
size_t gt_graph_meta_bytes(int64_t n_rows, int64_t n_cols, int64_t nnz, int32_t chunk);

/* Build the CSR transpose and both work schedules on the GPU.
 *   CSR^T: indptr_t[c+1] - indptr_t[c] = in-degree of column c; the entries
 *   of a column are ordered by ascending source row (a stable transpose);
 *   indices_t[t] = source row, perm[t] = CSR edge id (the adjacency's
 *   transpose is what the backward's A^T products of Section 2.2 run on).
 *   Thresholds: 0 <= t_small <= t_mid, chunk >= 1 (gt_graph_thresholds).
 * Synchronises `stream` (the schedule sizes are read back to fill *out).
 * Errors: GT_E_NULL, GT_E_ARG, GT_E_WORKSPACE (meta_bytes too small),
 * GT_E_HIP. */
gt_status gt_graph_prepare(const int32_t *indptr, const int32_t *indices, int64_t n_rows,
                           int64_t n_cols, int64_t nnz, int32_t t_small, int32_t t_mid,
                           int32_t chunk, void *meta, size_t meta_bytes, gt_graph *out,
                           void *stream);

/* The thresholds the kernels are tuned for: t_small = 32, t_mid = chunk = 256. */
void gt_default_thresholds(int32_t *t_small, int32_t *t_mid, int32_t *chunk);

/* The tuned thresholds for a graph of nnz nonzeros (the same for every size
 * since the pieces are dealt to the XCDs by position; kept so that callers
 * need not assume that). */
void gt_graph_thresholds(int64_t nnz, int32_t *t_small, int32_t *t_mid, int32_t *chunk);

/* Debug check of CSR content (the oracle's codes): 0 valid; 1 indptr[0] != 0
 * or indptr[n_rows] != nnz; 2 indptr decreasing; 3 a column outside
 * [0, n_cols); 4 columns of a row not strictly ascending.  When several
 * apply, the first in that order wins, and among 3/4 the lowest edge id.
 * `work` is GT_VALIDATE_WORK_BYTES of device scratch.  Writes the code to
 * *code; returns GT_E_CSR if it is not 0.  Synchronises `stream`.
 * Errors: GT_E_NULL, GT_E_ARG, GT_E_WORKSPACE, GT_E_CSR, GT_E_HIP. */
#define GT_VALIDATE_WORK_BYTES 64
gt_status gt_csr_validate(const int32_t *indptr, const int32_t *indices, int64_t n_rows,
                          int64_t n_cols, int64_t nnz, void *work, size_t work_bytes,
                          int32_t *code, void *stream);

/* ---- attention -------------------------------------------------------- */

/* Bytes of `work` gt_attn_fwd / gt_attn_bwd need (the larger of the two):
 * partial softmax states of split rows, the backward's per-row statistics
 * (lse, D) and partial gradient sums of split rows and columns. */
size_t gt_attn_work_bytes(const gt_graph *g, int32_t heads, int32_t head_dim);

/* Forward (Eq. 4-5): Y [n_rows, heads, head_dim] in dt, lse [n_rows, heads]
 * float32.  Q is [n_rows, heads, head_dim], K and V [n_cols, heads,
 * head_dim], all dt.  bias (nullable) is [nnz, heads] float32 in CSR edge
 * order; a -inf bias masks its edge (weight 0; a row with every edge masked
 * gives Y = 0 and lse = -inf, as an empty row), other bias values must be
 * finite.  Z and U are never materialised: the kernel makes one pass over
 * each row's edges with an online (running max) softmax.
 * Errors: GT_E_NULL, GT_E_DTYPE, GT_E_SHAPE, GT_E_ALIGN, GT_E_WORKSPACE,
 * GT_E_HIP. */
gt_status gt_attn_fwd(const gt_graph *g, int32_t heads, int32_t head_dim, gt_dtype dt,
                      float scale, const void *Q, const void *K, const void *V,
                      const float *bias, void *Y, float *lse, void *work, size_t work_bytes,
                      void *stream);

/* The forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): gt_attn_fwd without the `work` argument.  Its scratch (the
 * softmax states of split rows) is a static device array of
 * GT_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process ends; the
 * call allocates nothing.  Same arguments, results (bitwise) and errors as
 * gt_attn_fwd, plus GT_E_WORKSPACE when the graph needs more scratch than
 * that (gt_attn_work_bytes bounds it; a graph's split rows need about
 * 4 (heads * head_dim + 2 heads) bytes per `chunk` nonzeros of its rows
 * longer than t_mid) and GT_E_HIP if the array's address cannot be found.
 * The first call on a device looks that address up.  Nothing in the array
 * needs clearing: every state is written before it is read.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (several
 * streams, or several host threads) race and must be serialised by the
 * caller. */
#define GT_NOALLOC_SCRATCH_BYTES (16u << 20)
gt_status gt_attn_fwd_noalloc(const gt_graph *g, int32_t heads, int32_t head_dim, gt_dtype dt,
                              float scale, const void *Q, const void *K, const void *V,
                              const float *bias, void *Y, float *lse, void *stream);

/* Backward (Section 2.2): given Y and lse of gt_attn_fwd and the output
 * gradient dY [n_rows, heads, head_dim], writes dQ [n_rows, heads,
 * head_dim], dK, dV [n_cols, heads, head_dim] (all dt, every element
 * written) and, iff bias is given, dbias [nnz, heads] float32 (bias and
 * dbias must both be NULL or both non-NULL; else GT_E_UNSUPPORTED).  The
 * softmax weights are recomputed from lse.  A pass over the rows of A
 * computes dQ and the row term D_i = sum_e U_e dU_e; with a bias it also
 * stages each edge's score gradient in dbias, in CSR edge order, around the
 * shift <dY_i, Y_i> (which is why it reads Y), and a streaming pass finishes
 * dbias in place once D_i is known.  A pass over the rows of A^T computes dK
 * and dV.  No output element is written by more than one wavefront and
 * nothing uses atomics.  With bf16 storage dbias carries the rounding of its
 * bf16 staging (about 2^-9 relative), within the tolerance of bf16 inputs.
 * Y is read only when bias is given (it may be NULL otherwise).  A -inf bias
 * masks its edge (weight 0, dbias 0; a row with every edge masked behaves as
 * an empty row); bias values must otherwise be finite.
 * Errors: as gt_attn_fwd, plus GT_E_UNSUPPORTED. */
gt_status gt_attn_bwd(const gt_graph *g, int32_t heads, int32_t head_dim, gt_dtype dt,
                      float scale, const void *Q, const void *K, const void *V,
                      const float *bias, const void *Y, const float *lse, const void *dY,
                      void *dQ, void *dK, void *dV, float *dbias, void *work,
                      size_t work_bytes, void *stream);

/* ---- instrumentation and misc ----------------------------------------- */

/* Kernel timing.  Bit k of kernel_mask selects kernel k of "fwd",
 * "fwd_merge", "bwd_rows", "bwd_rows_merge", "bwd_cols", "bwd_cols_merge",
 * "bwd_dbias" (0: timing off, GT_PROF_ALL: all); every launch of a selected kernel is
 * bracketed by HIP events on its own stream, and gt_prof_query returns the
 * summed device time and the launch count per kernel name since the last
 * gt_prof_reset.  gt_prof_query synchronises the events. */
#define GT_PROF_ALL 0x7f
gt_status gt_prof_enable(int32_t kernel_mask);
gt_status gt_prof_reset(void);
gt_status gt_prof_query(const char *kernel, double *total_ms, int64_t *launches);

const char *gt_status_str(gt_status s);
/* Detail of the last failed call on this thread ("" if none). */
const char *gt_last_error(void);
/* Version of the ABI: 104 (pieces dealt to the XCDs; gt_attn_fwd_noalloc; gt_attn_bwd
 * takes the forward's Y). */
int32_t gt_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GT_ATTN_H */
