/*
 * gt_oracle.c -- plain, slow, obviously correct fp64 CPU oracle for
 * multi-head sparse graph attention over a CSR adjacency, forward and
 * backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code
 * with the GPU path and the GPU path never calls it.
 *
 * What it computes (Scalable and Adaptive Parallel Training of Graph
 * Transformer on Large Graphs, Section 2.1, Eq. 1-5, and Section 2.2):
 *   per head h, with s_e = scale * <Q_i,h , K_j,h> + bias_e,h for every
 *   stored edge e = (i, j) of A,
 *     U_e   = exp(s_e) / sum_{e' in row i} exp(s_e')     (softmax over the
 *             row's stored neighbours only, Eq. 1-2: j in N(i))
 *     Y_i,h = sum_{e in row i} U_e V_j,h                 (Eq. 5, SpMM)
 *     lse_i,h = log sum_{e in row i} exp(s_e)
 *   backward (textbook softmax-attention gradients; Section 2.2 gives only
 *   the operator count: 3 SpMM + 1 SDDMM):
 *     dU_e  = <dY_i,h , V_j,h>                           (sampled dY V^T)
 *     D_i,h = sum_{e in row i} U_e dU_e
 *     dS_e  = U_e (dU_e - D_i,h)                         (= d bias_e,h)
 *     dQ_i,h = scale * sum_{e in row i} dS_e K_j,h       (SpMM)
 *     dK_j,h = scale * sum_{e in column j} dS_e Q_i,h    (SpMM with A^T)
 *     dV_j,h = sum_{e in column j} U_e dY_i,h            (SpMM with A^T)
 * Readings where the pages are silent or garbled: the scale is passed in
 * (1/sqrt(head_dim) in practice; the square root is lost in the extracted
 * Eq. 2 and Eq. 4, and the engineering blog page restating the method
 * divides by sqrt(d)); head h is channels [h*dh, (h+1)*dh) of a node row;
 * the optional bias is added unscaled to the score before the softmax (the
 * MegaGraph page, Section III-A1, mechanism 3); an empty row gives Y = 0,
 * lse = -inf, dQ = 0; an empty column gives dK = dV = 0.  A bias of -inf
 * masks its edge: the edge gets weight 0 (exactly as if it were not stored)
 * and dbias 0, and a row whose every edge is masked is an empty row.
 *
 * Inputs Q, K, V, dY and bias are double arrays (float32 and bf16 data arrive
 * widened exactly); every product and sum is done in double.
 *
 * The graph side (CSR check, CSR transpose, the degree-ordered work
 * schedule) is integer work and is written here from its definitions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef int64_t i64;
typedef int32_t i32;

/* ------------------------------------------------------------------------ */
/* graph side                                                                */
/* ------------------------------------------------------------------------ */

/* 0: valid CSR.  1: indptr[0] != 0 or indptr[R] != E.  2: indptr decreasing.
 * 3: a column outside [0, M).  4: columns of a row not strictly ascending. */
int or_csr_check(i64 R, i64 M, i64 E, const i32 *indptr, const i32 *indices) {
  if (indptr[0] != 0 || (i64)indptr[R] != E) return 1;
  for (i64 r = 0; r < R; ++r)
    if (indptr[r + 1] < indptr[r]) return 2;
  for (i64 r = 0; r < R; ++r) {
    for (i64 e = indptr[r]; e < indptr[r + 1]; ++e) {
      if (indices[e] < 0 || (i64)indices[e] >= M) return 3;
      if (e > indptr[r] && indices[e] <= indices[e - 1]) return 4;
    }
  }
  return 0;
}

/* CSR transpose by a serial stable counting sort: count the entries of each
 * column, prefix-sum the counts, then walk the edges in CSR order and drop
 * each into the next free slot of its column.  Within a column the entries
 * therefore come in ascending source row.  indices_t[t] is the source row of
 * the t-th transposed entry and perm[t] its CSR edge id. */
void or_transpose(i64 R, i64 M, i64 E, const i32 *indptr, const i32 *indices,
                  i32 *indptr_t, i32 *indices_t, i32 *perm) {
  i64 *next = (i64 *)calloc((size_t)M + 1, sizeof(i64));
  for (i64 e = 0; e < E; ++e) next[indices[e] + 1] += 1;
  for (i64 c = 0; c < M; ++c) next[c + 1] += next[c];
  for (i64 c = 0; c <= M; ++c) indptr_t[c] = (i32)next[c];
  for (i64 r = 0; r < R; ++r) {
    for (i64 e = indptr[r]; e < indptr[r + 1]; ++e) {
      i64 t = next[indices[e]]++;
      indices_t[t] = (i32)r;
      perm[t] = (i32)e;
    }
  }
  free(next);
}

/* The degree-ordered work schedule, from its definition:
 *   order  = segment ids sorted by (order degree descending, id ascending),
 *            the order degree being the degree, or for a small segment
 *            (degree <= t_small) the degree rounded down to a multiple of
 *            small_class (so small segments stay at the tail);
 *   n_big  = #segments with degree >  t_mid;
 *   n_mid  = #segments with t_small < degree <= t_mid;
 *   n_small= #segments with degree <= t_small;
 *   every big segment s (in order) with degree d is cut into
 *   nch = ceil(d / chunk) pieces, piece c covering
 *   [ptr[s] + floor(c*d/nch), ptr[s] + floor((c+1)*d/nch)); each piece is
 *   (s, begin, end, slot), slot = its index in this segment-major
 *   enumeration when nch > 1 and -1 otherwise; every big segment with
 *   nch > 1 gives one merge record (s, first slot, nch);
 *   the item list is the pieces dealt by position: piece c of a segment cut
 *   into nch gets bucket q = floor(64 (2c+1) / (2 nch)), and queue
 *   floor(q / 8); within a queue the pieces go by bucket, then by their
 *   segment-major index; the list is filled four items at a time, the k-th
 *   four from queue k mod 8, or, while that queue is empty, from the next
 *   queue (k+1, k+2, ... mod 8) that is not.
 * Returns the number of items, or -1 if cap_items / cap_merges is exceeded. */
static void deal_by_position(i64 ni, i32 *items) {
  i32 *pieces = (i32 *)malloc(sizeof(i32) * 4 * (size_t)(ni + 1));
  i64 *q = (i64 *)malloc(sizeof(i64) * (size_t)(ni + 1));
  memcpy(pieces, items, sizeof(i32) * 4 * (size_t)ni);
  /* bucket of each piece */
  for (i64 i = 0; i < ni;) {
    i64 e = i;
    while (e < ni && pieces[4 * e] == pieces[4 * i]) e++;
    i64 nch = e - i;
    for (i64 c = 0; c < nch; ++c) q[i + c] = (64 * (2 * c + 1)) / (2 * nch);
    i = e;
  }
  /* the eight queues as index lists: each one scans the buckets of its
   * eighth in order, and each bucket the pieces in segment-major order */
  i64 *queue[8], qlen[8], used[8];
  for (int x = 0; x < 8; ++x) {
    queue[x] = (i64 *)malloc(sizeof(i64) * (size_t)(ni + 1));
    qlen[x] = 0;
    used[x] = 0;
    for (i64 b = 8 * x; b < 8 * x + 8; ++b)
      for (i64 i = 0; i < ni; ++i)
        if (q[i] == b) queue[x][qlen[x]++] = i;
  }
  i64 filled = 0;
  for (i64 k = 0; filled < ni; ++k) {
    for (int t = 0; t < 4 && filled < ni; ++t) {
      int x = (int)(k % 8);
      while (used[x] == qlen[x]) x = (x + 1) % 8;
      i64 src = queue[x][used[x]++];
      memcpy(items + 4 * filled, pieces + 4 * src, sizeof(i32) * 4);
      filled++;
    }
  }
  for (int x = 0; x < 8; ++x) free(queue[x]);
  free(q);
  free(pieces);
}

/* The degree a segment is ordered by: its degree, except that a small one
 * (degree <= t_small) counts its degree rounded down to a multiple of
 * small_class. */
static const i32 *g_sort_ptr;
static i32 g_sort_small, g_sort_class;
static i32 order_degree(i32 s) {
  i32 d = g_sort_ptr[s + 1] - g_sort_ptr[s];
  return d <= g_sort_small ? d - d % g_sort_class : d;
}
static int cmp_deg_desc(const void *a, const void *b) {
  i32 x = *(const i32 *)a, y = *(const i32 *)b;
  i32 dx = order_degree(x), dy = order_degree(y);
  if (dx != dy) return dx > dy ? -1 : 1;
  return (x > y) - (x < y);
}

i64 or_schedule(i64 n, const i32 *ptr, i32 t_small, i32 t_mid, i32 chunk, i32 small_class,
                i32 *order,
                i32 *counts /* [3] big, mid, small */, i32 *items /* [cap][4] */,
                i64 cap_items, i32 *merges /* [cap][3] */, i64 cap_merges,
                i64 *n_merges_out) {
  for (i64 s = 0; s < n; ++s) order[s] = (i32)s;
  g_sort_ptr = ptr;
  g_sort_small = t_small;
  g_sort_class = small_class > 0 ? small_class : 1;
  qsort(order, (size_t)n, sizeof(i32), cmp_deg_desc);
  i32 nb = 0, nm = 0, ns = 0;
  for (i64 s = 0; s < n; ++s) {
    i32 d = ptr[s + 1] - ptr[s];
    if (d > t_mid) nb++;
    else if (d > t_small) nm++;
    else ns++;
  }
  counts[0] = nb;
  counts[1] = nm;
  counts[2] = ns;
  i64 ni = 0, nmg = 0;
  for (i64 k = 0; k < nb; ++k) {
    i32 s = order[k];
    i64 d = ptr[s + 1] - ptr[s];
    i64 nch = (d + chunk - 1) / chunk;
    if (nch > 1) {
      if (nmg >= cap_merges) return -1;
      merges[3 * nmg + 0] = s;
      merges[3 * nmg + 1] = (i32)ni;
      merges[3 * nmg + 2] = (i32)nch;
      nmg++;
    }
    for (i64 c = 0; c < nch; ++c) {
      if (ni >= cap_items) return -1;
      items[4 * ni + 0] = s;
      items[4 * ni + 1] = (i32)(ptr[s] + (c * d) / nch);
      items[4 * ni + 2] = (i32)(ptr[s] + ((c + 1) * d) / nch);
      items[4 * ni + 3] = nch > 1 ? (i32)ni : -1;
      ni++;
    }
  }
  *n_merges_out = nmg;
  deal_by_position(ni, items);
  return ni;
}

/* ------------------------------------------------------------------------ */
/* attention                                                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
  i64 R, M;
  int H, dh;
  double scale;
  const i32 *indptr, *indices;
  const double *Q, *K, *V, *bias, *dY;
} prob_t;

static double dot_head(const double *a, const double *b, int dh) {
  double z = 0.0;
  for (int c = 0; c < dh; ++c) z += a[c] * b[c];
  return z;
}

/* score s_e of edge e (row i, column j) for head h */
static double score(const prob_t *p, i64 i, i64 e, int h) {
  i64 j = p->indices[e];
  i64 D = (i64)p->H * p->dh;
  double z = dot_head(p->Q + i * D + (i64)h * p->dh, p->K + j * D + (i64)h * p->dh, p->dh);
  double s = p->scale * z;
  if (p->bias) s += p->bias[e * p->H + h];
  return s;
}

/* Outputs of one row pass; every pointer may be NULL.
 * Y[D], lse[H], dQ[D], Dsum[H] (sum_e U_e dU_e), dB (deg*H, CSR edge order of
 * the row), and the magnitudes of the sums that define Y and dQ:
 *   Ymag[h,c]  = sum_e U_e |V[j,h,c]|
 *   dQmag[h,c] = scale sum_e U_e (|dU_e| + |D|) |K[j,h,c]|
 * (the sum of the absolute values of the terms, with the term dS_e =
 * U_e (dU_e - D) bounded by U_e (|dU_e| + |D|)); Tm (deg*H) gets
 * U_e (|dU_e| + |D|) for the column side. */
typedef struct {
  double *Y, *lse, *dQ, *Dsum, *dB, *Ymag, *dQmag, *Tm;
} row_out_t;

/* Everything the definition gives for one row i, all heads.
 * U, dU, dS: scratch of deg*H doubles ([edge-in-row][head]); U and dS hold
 * the row's softmax weights and score gradients on return.
 * The backward part runs only when a backward output is requested. */
static void row_pass(const prob_t *p, i64 i, double *U, double *dU, double *dS,
                     const row_out_t *o) {
  const i64 e0 = p->indptr[i], deg = p->indptr[i + 1] - e0;
  const int H = p->H, dh = p->dh;
  const int want_bwd = (o->dQ || o->dB || o->Dsum || o->dQmag || o->Tm);
  for (int h = 0; h < H; ++h) {
    /* scores and softmax over the stored neighbours of row i */
    double m = -INFINITY;
    for (i64 k = 0; k < deg; ++k) {
      double s = score(p, i, e0 + k, h);
      U[k * H + h] = s;
      if (s > m) m = s;
    }
    /* A score of -inf (an edge masked by a -inf bias) gets weight 0, the
     * same as an edge that is not stored; a row whose every score is -inf
     * has no support and is treated as an empty row (U = 0, lse = -inf). */
    double l = 0.0;
    if (m > -INFINITY) {
      for (i64 k = 0; k < deg; ++k) l += exp(U[k * H + h] - m);
      for (i64 k = 0; k < deg; ++k) U[k * H + h] = exp(U[k * H + h] - m) / l;
    } else {
      for (i64 k = 0; k < deg; ++k) U[k * H + h] = 0.0;
    }
    if (o->lse) o->lse[h] = l > 0.0 ? m + log(l) : -INFINITY;
    for (int c = 0; c < dh; ++c) {
      double y = 0.0, ya = 0.0;
      for (i64 k = 0; k < deg; ++k) {
        i64 j = p->indices[e0 + k];
        double v = p->V[j * (i64)H * dh + (i64)h * dh + c];
        y += U[k * H + h] * v;
        ya += U[k * H + h] * fabs(v);
      }
      if (o->Y) o->Y[(i64)h * dh + c] = y;
      if (o->Ymag) o->Ymag[(i64)h * dh + c] = ya;
    }
    if (!want_bwd) continue;
    /* softmax backward */
    const i64 D = (i64)H * dh;
    double Ds = 0.0;
    for (i64 k = 0; k < deg; ++k) {
      i64 j = p->indices[e0 + k];
      dU[k * H + h] = dot_head(p->dY + i * D + (i64)h * dh, p->V + j * D + (i64)h * dh, dh);
      Ds += U[k * H + h] * dU[k * H + h];
    }
    if (o->Dsum) o->Dsum[h] = Ds;
    for (i64 k = 0; k < deg; ++k) dS[k * H + h] = U[k * H + h] * (dU[k * H + h] - Ds);
    if (o->dB)
      for (i64 k = 0; k < deg; ++k) o->dB[k * H + h] = dS[k * H + h];
    if (o->Tm)
      for (i64 k = 0; k < deg; ++k)
        o->Tm[k * H + h] = U[k * H + h] * (fabs(dU[k * H + h]) + fabs(Ds));
    for (int c = 0; c < dh; ++c) {
      double g = 0.0, ga = 0.0;
      for (i64 k = 0; k < deg; ++k) {
        i64 j = p->indices[e0 + k];
        double kv = p->K[j * D + (i64)h * dh + c];
        g += dS[k * H + h] * kv;
        ga += U[k * H + h] * (fabs(dU[k * H + h]) + fabs(Ds)) * fabs(kv);
      }
      if (o->dQ) o->dQ[(i64)h * dh + c] = p->scale * g;
      if (o->dQmag) o->dQmag[(i64)h * dh + c] = p->scale * ga;
    }
  }
}

static i64 max_degree(const i32 *ptr, i64 n) {
  i64 m = 0;
  for (i64 s = 0; s < n; ++s)
    if (ptr[s + 1] - ptr[s] > m) m = ptr[s + 1] - ptr[s];
  return m;
}

static int g_threads = 0; /* 0: OpenMP default */

void or_set_threads(int n) { g_threads = n; }

int or_get_threads(void) {
#ifdef _OPENMP
  if (g_threads > 0) return g_threads;
  return omp_get_max_threads();
#else
  return 1;
#endif
}

#ifdef _OPENMP
#define OMP_THREADS num_threads(or_get_threads())
#else
#define OMP_THREADS
#endif

#define OFF(ptr, n) ((ptr) ? (ptr) + (n) : NULL)

/* Forward on every row: Y [R*D], lse [R*H]; U (nullable) [E*H]; Ymag
 * (nullable) [R*D]. */
void or_fwd(i64 R, i64 M, int H, int dh, double scale, const i32 *indptr, const i32 *indices,
            const double *Q, const double *K, const double *V, const double *bias, double *Y,
            double *lse, double *U_out, double *Ymag) {
  prob_t p = {R, M, H, dh, scale, indptr, indices, Q, K, V, bias, NULL};
  const i64 D = (i64)H * dh;
  const i64 md = max_degree(indptr, R);
#pragma omp parallel OMP_THREADS
  {
    double *U = (double *)malloc(sizeof(double) * (size_t)(md * H + 1));
#pragma omp for schedule(dynamic, 64)
    for (i64 i = 0; i < R; ++i) {
      row_out_t o = {Y + i * D, lse + i * H, NULL, NULL, NULL, OFF(Ymag, i * D), NULL, NULL};
      row_pass(&p, i, U, NULL, NULL, &o);
      if (U_out) memcpy(U_out + (i64)indptr[i] * H, U, sizeof(double) * (size_t)((indptr[i + 1] - indptr[i]) * H));
    }
    free(U);
  }
}

/* Backward on the whole graph: dQ [R*D], dK, dV [M*D], dB (nullable iff bias
 * is NULL) [E*H]; the magnitudes dQmag [R*D], dKmag, dVmag [M*D] (each
 * nullable):
 *   dKmag[j,h,c] = scale sum_{e in column j} U_e (|dU_e| + |D_i|) |Q[i,h,c]|
 *   dVmag[j,h,c] =       sum_{e in column j} U_e |dY[i,h,c]|.
 * Recomputes the forward row by row. */
void or_bwd(i64 R, i64 M, int H, int dh, double scale, const i32 *indptr, const i32 *indices,
            const double *Q, const double *K, const double *V, const double *bias, const double *dY,
            double *dQ, double *dK, double *dV, double *dB, double *dQmag, double *dKmag,
            double *dVmag) {
  prob_t p = {R, M, H, dh, scale, indptr, indices, Q, K, V, bias, dY};
  const i64 D = (i64)H * dh;
  const i64 E = indptr[R];
  const i64 md = max_degree(indptr, R);
  const int want_mag = dKmag || dVmag;
  double *Uall = (double *)malloc(sizeof(double) * (size_t)(E * H + 1));
  double *dSall = (double *)malloc(sizeof(double) * (size_t)(E * H + 1));
  double *Tall = want_mag ? (double *)malloc(sizeof(double) * (size_t)(E * H + 1)) : NULL;
  /* row side: U, dS, dQ, dB */
#pragma omp parallel OMP_THREADS
  {
    double *dU = (double *)malloc(sizeof(double) * (size_t)(md * H + 1));
#pragma omp for schedule(dynamic, 64)
    for (i64 i = 0; i < R; ++i) {
      i64 e0 = indptr[i];
      row_out_t o = {NULL, NULL, dQ + i * D, NULL, OFF(dB, e0 * H), NULL, OFF(dQmag, i * D),
                     OFF(Tall, e0 * H)};
      row_pass(&p, i, Uall + e0 * H, dU, dSall + e0 * H, &o);
    }
    free(dU);
  }
  /* column side over the transpose: dV = U^T dY, dK = scale dS^T Q */
  i32 *ptr_t = (i32 *)malloc(sizeof(i32) * (size_t)(M + 1));
  i32 *src = (i32 *)malloc(sizeof(i32) * (size_t)(E + 1));
  i32 *perm = (i32 *)malloc(sizeof(i32) * (size_t)(E + 1));
  or_transpose(R, M, E, indptr, indices, ptr_t, src, perm);
#pragma omp parallel for schedule(dynamic, 64) OMP_THREADS
  for (i64 j = 0; j < M; ++j) {
    for (int h = 0; h < H; ++h) {
      for (int c = 0; c < dh; ++c) {
        double gv = 0.0, gk = 0.0, av = 0.0, ak = 0.0;
        for (i64 t = ptr_t[j]; t < ptr_t[j + 1]; ++t) {
          i64 i = src[t], e = perm[t];
          double y = dY[i * D + (i64)h * dh + c], q = Q[i * D + (i64)h * dh + c];
          gv += Uall[e * H + h] * y;
          gk += dSall[e * H + h] * q;
          if (want_mag) {
            av += Uall[e * H + h] * fabs(y);
            ak += Tall[e * H + h] * fabs(q);
          }
        }
        dV[j * D + (i64)h * dh + c] = gv;
        dK[j * D + (i64)h * dh + c] = scale * gk;
        if (dVmag) dVmag[j * D + (i64)h * dh + c] = av;
        if (dKmag) dKmag[j * D + (i64)h * dh + c] = scale * ak;
      }
    }
  }
  free(ptr_t);
  free(src);
  free(perm);
  free(Uall);
  free(dSall);
  free(Tall);
}

/* Selected rows only: Y, lse, dQ of rows[k] into Y[k*D], lse[k*H], dQ[k*D];
 * dB (nullable) of their edges, packed row after row ([sum deg][H]);
 * Ymag, dQmag (nullable) like Y, dQ. */
void or_rows(i64 R, i64 M, int H, int dh, double scale, const i32 *indptr, const i32 *indices,
             const double *Q, const double *K, const double *V, const double *bias, const double *dY,
             i64 n_sel, const i32 *rows, double *Y, double *lse, double *dQ, double *dB,
             double *Ymag, double *dQmag) {
  prob_t p = {R, M, H, dh, scale, indptr, indices, Q, K, V, bias, dY};
  const i64 D = (i64)H * dh;
  i64 *off = (i64 *)malloc(sizeof(i64) * (size_t)(n_sel + 1));
  off[0] = 0;
  i64 md = 0;
  for (i64 k = 0; k < n_sel; ++k) {
    i64 d = indptr[rows[k] + 1] - indptr[rows[k]];
    off[k + 1] = off[k] + d;
    if (d > md) md = d;
  }
#pragma omp parallel OMP_THREADS
  {
    double *U = (double *)malloc(sizeof(double) * (size_t)(md * H + 1));
    double *dU = (double *)malloc(sizeof(double) * (size_t)(md * H + 1));
    double *dS = (double *)malloc(sizeof(double) * (size_t)(md * H + 1));
#pragma omp for schedule(dynamic, 1)
    for (i64 k = 0; k < n_sel; ++k) {
      row_out_t o = {Y + k * D, lse + k * H, dQ + k * D, NULL, OFF(dB, off[k] * H),
                     OFF(Ymag, k * D), OFF(dQmag, k * D), NULL};
      row_pass(&p, rows[k], U, dU, dS, &o);
    }
    free(U);
    free(dU);
    free(dS);
  }
  free(off);
}

/* Selected columns only: dK, dV of cols[k] into dK[k*D], dV[k*D], and their
 * magnitudes dKmag, dVmag (nullable).  U_e and dS_e of an in-edge come from
 * its source row's own softmax statistics (lse and D = sum U dU), computed by
 * the same row pass. */
void or_cols(i64 R, i64 M, int H, int dh, double scale, const i32 *indptr, const i32 *indices,
             const double *Q, const double *K, const double *V, const double *bias, const double *dY,
             i64 n_sel, const i32 *cols, double *dK, double *dV, double *dKmag, double *dVmag) {
  prob_t p = {R, M, H, dh, scale, indptr, indices, Q, K, V, bias, dY};
  const i64 D = (i64)H * dh;
  const i64 E = indptr[R];
  i64 *slot = (i64 *)malloc(sizeof(i64) * (size_t)M);
  for (i64 j = 0; j < M; ++j) slot[j] = -1;
  for (i64 k = 0; k < n_sel; ++k) slot[cols[k]] = k;
  /* in-edges of every selected column, in ascending source row */
  i64 *cnt = (i64 *)calloc((size_t)n_sel + 1, sizeof(i64));
  for (i64 e = 0; e < E; ++e)
    if (slot[indices[e]] >= 0) cnt[slot[indices[e]] + 1]++;
  for (i64 k = 0; k < n_sel; ++k) cnt[k + 1] += cnt[k];
  i64 n_in = cnt[n_sel];
  i64 *fill = (i64 *)malloc(sizeof(i64) * (size_t)(n_sel + 1));
  memcpy(fill, cnt, sizeof(i64) * (size_t)(n_sel + 1));
  i64 *in_row = (i64 *)malloc(sizeof(i64) * (size_t)(n_in + 1));
  i64 *in_edge = (i64 *)malloc(sizeof(i64) * (size_t)(n_in + 1));
  char *need = (char *)calloc((size_t)R, 1);
  for (i64 i = 0; i < R; ++i)
    for (i64 e = indptr[i]; e < indptr[i + 1]; ++e) {
      i64 k = slot[indices[e]];
      if (k >= 0) {
        in_row[fill[k]] = i;
        in_edge[fill[k]] = e;
        fill[k]++;
        need[i] = 1;
      }
    }
  double *lse = (double *)malloc(sizeof(double) * (size_t)(R * H));
  double *Dr = (double *)malloc(sizeof(double) * (size_t)(R * H));
  const i64 md = max_degree(indptr, R);
#pragma omp parallel OMP_THREADS
  {
    double *U = (double *)malloc(sizeof(double) * (size_t)(md * H + 1));
    double *dU = (double *)malloc(sizeof(double) * (size_t)(md * H + 1));
    double *dS = (double *)malloc(sizeof(double) * (size_t)(md * H + 1));
#pragma omp for schedule(dynamic, 64)
    for (i64 i = 0; i < R; ++i)
      if (need[i]) {
        row_out_t o = {NULL, lse + i * H, NULL, Dr + i * H, NULL, NULL, NULL, NULL};
        row_pass(&p, i, U, dU, dS, &o);
      }
    free(U);
    free(dU);
    free(dS);
  }
#pragma omp parallel for schedule(dynamic, 1) OMP_THREADS
  for (i64 k = 0; k < n_sel; ++k) {
    i64 j = cols[k];
    for (int h = 0; h < H; ++h) {
      double *gk = dK + k * D + (i64)h * dh, *gv = dV + k * D + (i64)h * dh;
      double *mk = OFF(dKmag, k * D + (i64)h * dh), *mv = OFF(dVmag, k * D + (i64)h * dh);
      for (int c = 0; c < dh; ++c) {
        gk[c] = gv[c] = 0.0;
        if (mk) mk[c] = 0.0;
        if (mv) mv[c] = 0.0;
      }
      for (i64 t = cnt[k]; t < cnt[k + 1]; ++t) {
        i64 i = in_row[t], e = in_edge[t];
        /* weight 0 for every edge of a row without support (lse = -inf) */
        double u = lse[i * H + h] > -INFINITY ? exp(score(&p, i, e, h) - lse[i * H + h]) : 0.0;
        double du = dot_head(dY + i * D + (i64)h * dh, V + j * D + (i64)h * dh, dh);
        double ds = u * (du - Dr[i * H + h]);
        double tm = u * (fabs(du) + fabs(Dr[i * H + h]));
        for (int c = 0; c < dh; ++c) {
          double y = dY[i * D + (i64)h * dh + c], q = Q[i * D + (i64)h * dh + c];
          gv[c] += u * y;
          gk[c] += ds * q;
          if (mv) mv[c] += u * fabs(y);
          if (mk) mk[c] += tm * fabs(q);
        }
      }
      for (int c = 0; c < dh; ++c) {
        gk[c] *= scale;
        if (mk) mk[c] *= scale;
      }
    }
  }
  free(slot);
  free(cnt);
  free(fill);
  free(in_row);
  free(in_edge);
  free(need);
  free(lse);
  free(Dr);
}
