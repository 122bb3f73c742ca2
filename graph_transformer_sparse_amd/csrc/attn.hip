// Sparse graph attention kernels for gfx950 ("Scalable and Adaptive Parallel
// Training of Graph Transformer on Large Graphs", Section 2.1 Eq. 1-5 for the
// forward, Section 2.2 for the backward's operators).
//
// Mapping.  A node's feature row of D = H*dh elements is spread over a lane
// group of G = D*sizeof(T)/16 lanes, one 16-byte slice per lane, so every
// gathered K/V/Q/dY row is one coalesced 16-byte-per-lane load.  The dh
// channels of a head sit on HL = G/H adjacent lanes; per-edge dot products
// are lane-local FMAs followed by a DPP sum over those HL lanes.
//
// Work.  The degree-ordered schedule of the prepared graph drives a single
// launch per pass: wavefront w takes, in order, a piece of a big segment
// (split into pieces of at most `chunk` nonzeros), a whole mid segment, or
// (64/G) small segments, one per lane group.  Inside a wavefront that owns
// one segment, lane group g takes the segment's nonzeros g, g + 64/G, ...
// and the groups' partial results are combined by a fixed butterfly.  Split
// segments leave per-piece partials that a merge kernel combines in piece
// order.  Every output element is written by exactly one lane, with no
// atomics, so results are bitwise reproducible.
//
// Softmax.  Scores are kept in base 2: q is pre-multiplied by
// scale*log2(e) and the bias by log2(e), so exp(s - m) = 2^(s2 - m2) runs on
// v_exp_f32.  The forward keeps a running maximum and sum per head (online
// softmax); the bias enters the score before that update (the MegaGraph
// page, Section III-A1, mechanism 3).  The backward recomputes each weight
// from the forward's log-sum-exp instead of storing U.
#include <math.h>

#include "device.hpp"
#include "host.hpp"
#include "layout.hpp"

namespace gt {

constexpr int BLOCK = 256;
constexpr int WPB = BLOCK / WAVE;

struct Sched {
  const int32_t *ptr;    // [n_seg + 1] segment pointer (indptr or indptr_t)
  const int32_t *order;  // degree order
  const int32_t *items;  // [n_items][4]
  const int32_t *merges; // [n_merges][3]
  int64_t n_big, n_mid, n_small, n_items, n_merges;
};

// The segment a lane group works on.  wave_item: the whole wavefront shares
// one (piece of a) segment.
struct Work {
  int32_t seg, eb, ee, slot;
  bool wave_item, active;
};

template <int RPW>
__device__ inline Work decode(const Sched &s, int grp) {
  const int64_t w = (int64_t)blockIdx.x * WPB + threadIdx.x / WAVE;
  Work k;
  k.active = true;
  if (w < s.n_items) {
    const int4 it = *reinterpret_cast<const int4 *>(s.items + 4 * w);
    k.seg = it.x;
    k.eb = it.y;
    k.ee = it.z;
    k.slot = it.w;
    k.wave_item = true;
  } else if (w < s.n_items + s.n_mid) {
    k.seg = s.order[s.n_big + (w - s.n_items)];
    k.eb = s.ptr[k.seg];
    k.ee = s.ptr[k.seg + 1];
    k.slot = -1;
    k.wave_item = true;
  } else {
    const int64_t q = (w - s.n_items - s.n_mid) * RPW + grp;
    k.wave_item = false;
    k.slot = -1;
    if (q >= s.n_small) {
      k.active = false;
      k.seg = 0;
      k.eb = k.ee = 0;
    } else {
      k.seg = s.order[s.n_big + s.n_mid + q];
      k.eb = s.ptr[k.seg];
      k.ee = s.ptr[k.seg + 1];
    }
  }
  return k;
}

template <typename T> struct Raw;
template <> struct Raw<float> { using type = float4; };
template <> struct Raw<bf16_t> { using type = uint4; };

template <typename T>
__device__ inline typename Raw<T>::type load_raw(const T *p) {
  return *reinterpret_cast<const typename Raw<T>::type *>(p);
}
__device__ inline void unpack(const float4 &v, float (&x)[4]) {
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ inline void unpack(const uint4 &v, float (&x)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}

// Online-softmax state merge: (m, l, a) (+) (m', l', a') with M = max(m, m')
// gives (M, l 2^(m-M) + l' 2^(m'-M), a 2^(m-M) + a' 2^(m'-M)); an empty state
// (m = -inf) contributes nothing.
__device__ inline void merge_weights(float m, float mo, float &mn, float &fa, float &fb) {
  mn = fmaxf(m, mo);
  fa = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
  fb = (mo == -INFINITY) ? 0.f : fast_exp2(mo - mn);
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
struct FwdArgs {
  Sched s;
  const int32_t *idx;
  const void *Q, *K, *V;
  const float *bias;
  void *Y;
  float *lse;
  float *part_ml;   // [slots][H][2]  (m2, l) of split-row pieces
  float *part_acc;  // [slots][D]
  float qscale;     // scale * log2(e)
};

template <typename T, int HL, int H, int U, bool BIAS>
__global__ __launch_bounds__(BLOCK) void k_fwd(FwdArgs a) {
  constexpr int N = Vec<T>::N, G = HL * H, D = G * N, RPW = WAVE / G;
  const int lane = threadIdx.x & (WAVE - 1), grp = lane / G, gl = lane % G, h = gl / HL;
  const Work wk = decode<RPW>(a.s, grp);
  if (!wk.active) return;
  const T *Qp = (const T *)a.Q, *Kp = (const T *)a.K, *Vp = (const T *)a.V;
  const int64_t row = wk.seg;
  float q[N];
  Vec<T>::load(Qp + row * D + gl * N, q);
#pragma unroll
  for (int c = 0; c < N; ++c) q[c] *= a.qscale;
  float m = -INFINITY, l = 0.f, acc[N];
#pragma unroll
  for (int c = 0; c < N; ++c) acc[c] = 0.f;
  const int gstart = wk.wave_item ? grp : 0, gstep = wk.wave_item ? RPW : 1;
  for (int64_t e = (int64_t)wk.eb + gstart; e < wk.ee; e += (int64_t)gstep * U) {
    int32_t j[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t eu = e + (int64_t)u * gstep;
      ok[u] = eu < wk.ee;
      j[u] = a.idx[ok[u] ? eu : e];
    }
    typename Raw<T>::type kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kr[u] = load_raw(Kp + (int64_t)j[u] * D + gl * N);
#pragma unroll
    for (int u = 0; u < U; ++u) vr[u] = load_raw(Vp + (int64_t)j[u] * D + gl * N);
    float b[U];
    if constexpr (BIAS) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t eu = e + (int64_t)u * gstep;
        b[u] = a.bias[(ok[u] ? eu : e) * H + h] * LOG2E;
      }
    }
    float sc[U];
    float mn = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kx[N];
      unpack(kr[u], kx);
      float d = 0.f;
#pragma unroll
      for (int c = 0; c < N; ++c) d = fmaf(q[c], kx[c], d);
      d = group_sum<HL>(d);
      if constexpr (BIAS) d += b[u];
      sc[u] = ok[u] ? d : -INFINITY;
      mn = fmaxf(mn, sc[u]);
    }
    const float alpha = fast_exp2(m - mn);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < N; ++c) acc[c] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = fast_exp2(sc[u] - mn);
      float vx[N];
      unpack(vr[u], vx);
      l += p;
#pragma unroll
      for (int c = 0; c < N; ++c) acc[c] = fmaf(p, vx[c], acc[c]);
    }
    m = mn;
  }
  if (wk.wave_item) {
#pragma unroll
    for (int off = G; off < WAVE; off <<= 1) {
      const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
      float mn, fa, fb;
      merge_weights(m, mo, mn, fa, fb);
      l = l * fa + lo * fb;
#pragma unroll
      for (int c = 0; c < N; ++c) acc[c] = acc[c] * fa + __shfl_xor(acc[c], off) * fb;
      m = mn;
    }
    if (grp != 0) return;
    if (wk.slot >= 0) {
      float *pa = a.part_acc + (int64_t)wk.slot * D + gl * N;
#pragma unroll
      for (int c = 0; c < N; c += 4)
        *reinterpret_cast<float4 *>(pa + c) = make_float4(acc[c], acc[c + 1], acc[c + 2], acc[c + 3]);
      if (gl % HL == 0)
        *reinterpret_cast<float2 *>(a.part_ml + ((int64_t)wk.slot * H + h) * 2) = make_float2(m, l);
      return;
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float y[N];
#pragma unroll
  for (int c = 0; c < N; ++c) y[c] = acc[c] * inv;
  Vec<T>::store((T *)a.Y + row * D + gl * N, y);
  if (gl % HL == 0) a.lse[row * H + h] = l > 0.f ? (m + fast_log2(l)) * LN2 : -INFINITY;
}

// One wavefront per split row: merge its pieces' states in piece order.
template <typename T, int HL, int H>
__global__ __launch_bounds__(BLOCK) void k_fwd_merge(FwdArgs a) {
  constexpr int N = Vec<T>::N, G = HL * H, D = G * N;
  const int64_t w = (int64_t)blockIdx.x * WPB + threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  if (w >= a.s.n_merges || lane >= G) return;
  const int gl = lane, h = gl / HL;
  const int32_t *rec = a.s.merges + 3 * w;
  const int64_t row = rec[0], first = rec[1], nch = rec[2];
  float m = -INFINITY, l = 0.f, acc[N];
#pragma unroll
  for (int c = 0; c < N; ++c) acc[c] = 0.f;
  for (int64_t k = 0; k < nch; ++k) {
    const int64_t slot = first + k;
    const float2 ml = *reinterpret_cast<const float2 *>(a.part_ml + (slot * H + h) * 2);
    const float *pa = a.part_acc + slot * D + gl * N;
    float mn, fa, fb;
    merge_weights(m, ml.x, mn, fa, fb);
    l = l * fa + ml.y * fb;
#pragma unroll
    for (int c = 0; c < N; ++c) acc[c] = acc[c] * fa + pa[c] * fb;
    m = mn;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float y[N];
#pragma unroll
  for (int c = 0; c < N; ++c) y[c] = acc[c] * inv;
  Vec<T>::store((T *)a.Y + row * D + gl * N, y);
  if (gl % HL == 0) a.lse[row * H + h] = l > 0.f ? (m + fast_log2(l)) * LN2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// backward, row pass over A: dQ and the per-row (lse2, D) statistics
//
// With U_e = p_e / L, p_e = 2^(s2_e - lse2_i) recomputed from the forward's
// log-sum-exp and L = sum_e p_e (1 up to the rounding of lse), and
// dU_e = <dY_i, V_j>, the row term is D_i = sum_e U_e dU_e and
// dQ_i = scale sum_e U_e (dU_e - D_i) K_j.  One pass over the row's edges
// accumulates, around a shift c (the dU of the first edge a lane group sees),
//   L = sum p,  S = sum p (dU - c),  A1 = sum p (dU - c) K,  A2 = sum p K,
// and then D = c + S / L and dQ = scale (A1 - (S / L) A2) / L.  Dividing by L
// makes the weights sum to 1 whatever the rounding of lse (the column pass
// gets lse2 + log2(L) so that its weights are the same U_e); the shift keeps
// the subtraction small, and a row with one edge gets dQ = 0 and D = dU
// exactly.  Two partial states combine at the shift of the first non-empty
// one: S = S_a + S_b + (c_b - c_a) L_b, A1 = A1_a + A1_b + (c_b - c_a) A2_b.
// ---------------------------------------------------------------------------
struct BwdArgs {
  Sched rows, cols;
  const int32_t *idx;     // CSR columns
  const int32_t *idx_t;   // CSR^T source rows
  const int32_t *perm;    // CSR^T -> CSR edge id
  const void *Q, *K, *V, *dY;
  const float *lse, *bias;
  void *dQ, *dK, *dV;
  float *dbias;
  float2 *rowstat;        // [R][H] (lse * log2(e) + log2(L), D)
  float *part_rows;       // [slots][2D + 3H]: A1, A2, S, L, c of split-row pieces
  float *part_cols;       // [slots][2D]: dK partial, then dV partial
  float qscale, scale;
};

// Row-pass state of one lane: its N channels of A1 and A2, and the per-head
// L, S and shift c (equal on the HL lanes of a head).
template <int N> struct RowState {
  float a1[N], a2[N], s, l, c;
};

// st (+)= o, at the shift of st unless st is empty.
template <int N> __device__ inline void row_merge(RowState<N> &st, const RowState<N> &o) {
  if (st.l == 0.f) {
    st = o;
    return;
  }
  const float dc = o.c - st.c;
  st.s += o.s + dc * o.l;
  st.l += o.l;
#pragma unroll
  for (int c = 0; c < N; ++c) {
    st.a1[c] += o.a1[c] + dc * o.a2[c];
    st.a2[c] += o.a2[c];
  }
}

// dQ and the row statistics of one row from its state (all lanes of the
// row's group; lane gl holds channels [gl*N, gl*N + N)).
template <typename T, int HL, int H>
__device__ inline void finish_row(const BwdArgs &a, int64_t row, int gl, int h, float lse2,
                                  const RowState<Vec<T>::N> &st) {
  constexpr int N = Vec<T>::N, D = HL * H * N;
  const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
  const float ds = st.s * inv;
  float g[N];
#pragma unroll
  for (int c = 0; c < N; ++c) g[c] = a.scale * ((st.a1[c] - ds * st.a2[c]) * inv);
  Vec<T>::store((T *)a.dQ + row * D + gl * N, g);
  if (gl % HL == 0)
    a.rowstat[row * H + h] =
        st.l > 0.f ? make_float2(lse2 + fast_log2(st.l), st.c + ds) : make_float2(-INFINITY, 0.f);
}

template <typename T, int HL, int H, int U, bool BIAS>
__global__ __launch_bounds__(BLOCK) void k_bwd_rows(BwdArgs a) {
  constexpr int N = Vec<T>::N, G = HL * H, D = G * N, RPW = WAVE / G;
  const int lane = threadIdx.x & (WAVE - 1), grp = lane / G, gl = lane % G, h = gl / HL;
  const Work wk = decode<RPW>(a.rows, grp);
  if (!wk.active) return;
  const T *Kp = (const T *)a.K, *Vp = (const T *)a.V;
  const int64_t row = wk.seg;
  float q[N], dy[N];
  Vec<T>::load((const T *)a.Q + row * D + gl * N, q);
  Vec<T>::load((const T *)a.dY + row * D + gl * N, dy);
#pragma unroll
  for (int c = 0; c < N; ++c) q[c] *= a.qscale;
  const float lse2 = a.lse[row * H + h] * LOG2E;
  RowState<N> st;
  st.s = st.l = st.c = 0.f;
#pragma unroll
  for (int c = 0; c < N; ++c) st.a1[c] = st.a2[c] = 0.f;
  const int gstart = wk.wave_item ? grp : 0, gstep = wk.wave_item ? RPW : 1;
  bool first = true;
  for (int64_t e = (int64_t)wk.eb + gstart; e < wk.ee; e += (int64_t)gstep * U) {
    int32_t j[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t eu = e + (int64_t)u * gstep;
      ok[u] = eu < wk.ee;
      j[u] = a.idx[ok[u] ? eu : e];
    }
    typename Raw<T>::type kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kr[u] = load_raw(Kp + (int64_t)j[u] * D + gl * N);
#pragma unroll
    for (int u = 0; u < U; ++u) vr[u] = load_raw(Vp + (int64_t)j[u] * D + gl * N);
    float b[U];
    if constexpr (BIAS) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t eu = e + (int64_t)u * gstep;
        b[u] = a.bias[(ok[u] ? eu : e) * H + h] * LOG2E;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kx[N], vx[N];
      unpack(kr[u], kx);
      unpack(vr[u], vx);
      float s = 0.f, du = 0.f;
#pragma unroll
      for (int c = 0; c < N; ++c) {
        s = fmaf(q[c], kx[c], s);
        du = fmaf(dy[c], vx[c], du);
      }
      s = group_sum<HL>(s);
      du = group_sum<HL>(du);
      if constexpr (BIAS) s += b[u];
      if (u == 0 && first) st.c = du;   // edge e is valid in every round
      const float p = ok[u] ? fast_exp2(s - lse2) : 0.f;
      const float pt = p * (du - st.c);
      st.l += p;
      st.s += pt;
#pragma unroll
      for (int c = 0; c < N; ++c) {
        st.a1[c] = fmaf(pt, kx[c], st.a1[c]);
        st.a2[c] = fmaf(p, kx[c], st.a2[c]);
      }
    }
    first = false;
  }
  if (wk.wave_item) {
#pragma unroll
    for (int off = G; off < WAVE; off <<= 1) {
      RowState<N> o;
      o.s = __shfl_xor(st.s, off);
      o.l = __shfl_xor(st.l, off);
      o.c = __shfl_xor(st.c, off);
#pragma unroll
      for (int c = 0; c < N; ++c) {
        o.a1[c] = __shfl_xor(st.a1[c], off);
        o.a2[c] = __shfl_xor(st.a2[c], off);
      }
      row_merge(st, o);
    }
    if (grp != 0) return;
    if (wk.slot >= 0) {
      float *pa = a.part_rows + (int64_t)wk.slot * (2 * D + 3 * H);
#pragma unroll
      for (int c = 0; c < N; ++c) {
        pa[gl * N + c] = st.a1[c];
        pa[D + gl * N + c] = st.a2[c];
      }
      if (gl % HL == 0) {
        pa[2 * D + h] = st.s;
        pa[2 * D + H + h] = st.l;
        pa[2 * D + 2 * H + h] = st.c;
      }
      return;
    }
  }
  finish_row<T, HL, H>(a, row, gl, h, lse2, st);
}

// Split rows: combine the pieces' states in piece order, then dQ and the row
// statistics.
template <typename T, int HL, int H>
__global__ __launch_bounds__(BLOCK) void k_bwd_rows_merge(BwdArgs a) {
  constexpr int N = Vec<T>::N, G = HL * H, D = G * N;
  const int64_t w = (int64_t)blockIdx.x * WPB + threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  if (w >= a.rows.n_merges || lane >= G) return;
  const int gl = lane, h = gl / HL;
  const int32_t *rec = a.rows.merges + 3 * w;
  const int64_t row = rec[0], first = rec[1], nch = rec[2];
  RowState<N> st;
  st.s = st.l = st.c = 0.f;
#pragma unroll
  for (int c = 0; c < N; ++c) st.a1[c] = st.a2[c] = 0.f;
  for (int64_t k = 0; k < nch; ++k) {
    const float *pa = a.part_rows + (first + k) * (2 * D + 3 * H);
    RowState<N> o;
#pragma unroll
    for (int c = 0; c < N; ++c) {
      o.a1[c] = pa[gl * N + c];
      o.a2[c] = pa[D + gl * N + c];
    }
    o.s = pa[2 * D + h];
    o.l = pa[2 * D + H + h];
    o.c = pa[2 * D + 2 * H + h];
    row_merge(st, o);
  }
  finish_row<T, HL, H>(a, row, gl, h, a.lse[row * H + h] * LOG2E, st);
}

// ---------------------------------------------------------------------------
// backward, column pass over A^T: dK, dV
// ---------------------------------------------------------------------------
template <typename T, int HL, int H, int U, bool BIAS>
__global__ __launch_bounds__(BLOCK) void k_bwd_cols(BwdArgs a) {
  constexpr int N = Vec<T>::N, G = HL * H, D = G * N, RPW = WAVE / G;
  const int lane = threadIdx.x & (WAVE - 1), grp = lane / G, gl = lane % G, h = gl / HL;
  const Work wk = decode<RPW>(a.cols, grp);
  if (!wk.active) return;
  const T *Qp = (const T *)a.Q, *dYp = (const T *)a.dY;
  const int64_t col = wk.seg;
  float k[N], v[N];
  Vec<T>::load((const T *)a.K + col * D + gl * N, k);
  Vec<T>::load((const T *)a.V + col * D + gl * N, v);
  float ak[N], av[N];
#pragma unroll
  for (int c = 0; c < N; ++c) ak[c] = av[c] = 0.f;
  const int gstart = wk.wave_item ? grp : 0, gstep = wk.wave_item ? RPW : 1;
  for (int64_t t = (int64_t)wk.eb + gstart; t < wk.ee; t += (int64_t)gstep * U) {
    int32_t i[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tu = t + (int64_t)u * gstep;
      ok[u] = tu < wk.ee;
      i[u] = a.idx_t[ok[u] ? tu : t];
    }
    typename Raw<T>::type qr[U], gr[U];
    float2 rs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) qr[u] = load_raw(Qp + (int64_t)i[u] * D + gl * N);
#pragma unroll
    for (int u = 0; u < U; ++u) gr[u] = load_raw(dYp + (int64_t)i[u] * D + gl * N);
#pragma unroll
    for (int u = 0; u < U; ++u) rs[u] = a.rowstat[(int64_t)i[u] * H + h];
    float b[U];
    int64_t eid[U];
    if constexpr (BIAS) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t tu = t + (int64_t)u * gstep;
        eid[u] = a.perm[ok[u] ? tu : t];
        b[u] = a.bias[eid[u] * H + h] * LOG2E;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float qx[N], gx[N];
      unpack(qr[u], qx);
      unpack(gr[u], gx);
      // same operands and order as the row pass, so s, p and dU match it
      float s = 0.f, du = 0.f;
#pragma unroll
      for (int c = 0; c < N; ++c) {
        s = fmaf(qx[c] * a.qscale, k[c], s);
        du = fmaf(gx[c], v[c], du);
      }
      s = group_sum<HL>(s);
      du = group_sum<HL>(du);
      if constexpr (BIAS) s += b[u];
      const float p = ok[u] ? fast_exp2(s - rs[u].x) : 0.f;
      const float ds = p * (du - rs[u].y);
#pragma unroll
      for (int c = 0; c < N; ++c) {
        av[c] = fmaf(p, gx[c], av[c]);
        ak[c] = fmaf(ds, qx[c], ak[c]);
      }
      if constexpr (BIAS) {
        if (ok[u] && gl % HL == 0) a.dbias[eid[u] * H + h] = ds;
      }
    }
  }
  if (wk.wave_item) {
#pragma unroll
    for (int off = G; off < WAVE; off <<= 1) {
#pragma unroll
      for (int c = 0; c < N; ++c) {
        ak[c] += __shfl_xor(ak[c], off);
        av[c] += __shfl_xor(av[c], off);
      }
    }
    if (grp != 0) return;
    if (wk.slot >= 0) {
      float *pk = a.part_cols + (int64_t)wk.slot * 2 * D + gl * N;
      float *pv = pk + D;
#pragma unroll
      for (int c = 0; c < N; c += 4) {
        *reinterpret_cast<float4 *>(pk + c) = make_float4(ak[c], ak[c + 1], ak[c + 2], ak[c + 3]);
        *reinterpret_cast<float4 *>(pv + c) = make_float4(av[c], av[c + 1], av[c + 2], av[c + 3]);
      }
      return;
    }
  }
#pragma unroll
  for (int c = 0; c < N; ++c) ak[c] *= a.scale;
  Vec<T>::store((T *)a.dK + col * D + gl * N, ak);
  Vec<T>::store((T *)a.dV + col * D + gl * N, av);
}

// Split columns: sum the pieces' dK, dV partials in piece order.
template <typename T, int HL, int H>
__global__ __launch_bounds__(BLOCK) void k_bwd_cols_merge(BwdArgs a) {
  constexpr int N = Vec<T>::N, G = HL * H, D = G * N;
  const int64_t w = (int64_t)blockIdx.x * WPB + threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  if (w >= a.cols.n_merges || lane >= G) return;
  const int gl = lane;
  const int32_t *rec = a.cols.merges + 3 * w;
  const int64_t seg = rec[0], first = rec[1], nch = rec[2];
  float x[N], z[N];
#pragma unroll
  for (int c = 0; c < N; ++c) x[c] = z[c] = 0.f;
  for (int64_t k = 0; k < nch; ++k) {
    const float *pk = a.part_cols + (first + k) * 2 * D + gl * N, *pv = pk + D;
#pragma unroll
    for (int c = 0; c < N; ++c) {
      x[c] += pk[c];
      z[c] += pv[c];
    }
  }
#pragma unroll
  for (int c = 0; c < N; ++c) x[c] *= a.scale;
  Vec<T>::store((T *)a.dK + seg * D + gl * N, x);
  Vec<T>::store((T *)a.dV + seg * D + gl * N, z);
}

// ---------------------------------------------------------------------------
// host side: shape dispatch and launches
// ---------------------------------------------------------------------------
constexpr int UNROLL = 4;

static int64_t waves_for(const Sched &s, int rpw) {
  return s.n_items + s.n_mid + cdiv(s.n_small, rpw);
}

template <typename T, int HL, int H>
static gt_status run_fwd(const FwdArgs &a, bool bias, hipStream_t st) {
  constexpr int G = HL * H, RPW = WAVE / G;
  const int64_t waves = waves_for(a.s, RPW);
  if (waves > 0) {
    const dim3 grid((unsigned)cdiv(waves, WPB));
    const int tok = prof_begin(PK_FWD, st);
    if (bias) k_fwd<T, HL, H, UNROLL, true><<<grid, BLOCK, 0, st>>>(a);
    else k_fwd<T, HL, H, UNROLL, false><<<grid, BLOCK, 0, st>>>(a);
    prof_end(tok, st);
    GT_CHECK_LAUNCH();
  }
  if (a.s.n_merges > 0) {
    const int tok = prof_begin(PK_FWD_MERGE, st);
    k_fwd_merge<T, HL, H><<<dim3((unsigned)cdiv(a.s.n_merges, WPB)), BLOCK, 0, st>>>(a);
    prof_end(tok, st);
    GT_CHECK_LAUNCH();
  }
  return GT_OK;
}

template <typename T, int HL, int H>
static gt_status run_bwd(const BwdArgs &a, bool bias, hipStream_t st) {
  constexpr int G = HL * H, RPW = WAVE / G;
  int64_t waves = waves_for(a.rows, RPW);
  if (waves > 0) {
    const dim3 grid((unsigned)cdiv(waves, WPB));
    const int tok = prof_begin(PK_BWD_ROWS, st);
    if (bias) k_bwd_rows<T, HL, H, UNROLL, true><<<grid, BLOCK, 0, st>>>(a);
    else k_bwd_rows<T, HL, H, UNROLL, false><<<grid, BLOCK, 0, st>>>(a);
    prof_end(tok, st);
    GT_CHECK_LAUNCH();
  }
  if (a.rows.n_merges > 0) {
    const int tok = prof_begin(PK_BWD_ROWS_MERGE, st);
    k_bwd_rows_merge<T, HL, H><<<dim3((unsigned)cdiv(a.rows.n_merges, WPB)), BLOCK, 0, st>>>(a);
    prof_end(tok, st);
    GT_CHECK_LAUNCH();
  }
  waves = waves_for(a.cols, RPW);
  if (waves > 0) {
    const dim3 grid((unsigned)cdiv(waves, WPB));
    const int tok = prof_begin(PK_BWD_COLS, st);
    if (bias) k_bwd_cols<T, HL, H, UNROLL, true><<<grid, BLOCK, 0, st>>>(a);
    else k_bwd_cols<T, HL, H, UNROLL, false><<<grid, BLOCK, 0, st>>>(a);
    prof_end(tok, st);
    GT_CHECK_LAUNCH();
  }
  if (a.cols.n_merges > 0) {
    const int tok = prof_begin(PK_BWD_COLS_MERGE, st);
    k_bwd_cols_merge<T, HL, H><<<dim3((unsigned)cdiv(a.cols.n_merges, WPB)), BLOCK, 0, st>>>(a);
    prof_end(tok, st);
    GT_CHECK_LAUNCH();
  }
  return GT_OK;
}

// Calls F<T, HL, H>() for the supported (dtype, head_dim, heads); returns
// false if the combination is not instantiated.
template <typename T, int HL, typename F>
static bool by_heads(int heads, F &&f) {
  switch (heads) {
    case 1: if constexpr (HL * 1 * Vec<T>::N * sizeof(T) <= 1024) { f.template operator()<T, HL, 1>(); return true; } break;
    case 2: if constexpr (HL * 2 * Vec<T>::N * sizeof(T) <= 1024) { f.template operator()<T, HL, 2>(); return true; } break;
    case 4: if constexpr (HL * 4 * Vec<T>::N * sizeof(T) <= 1024) { f.template operator()<T, HL, 4>(); return true; } break;
    case 8: if constexpr (HL * 8 * Vec<T>::N * sizeof(T) <= 1024) { f.template operator()<T, HL, 8>(); return true; } break;
  }
  return false;
}

template <typename F>
static bool dispatch(gt_dtype dt, int heads, int head_dim, F &&f) {
  if (dt == GT_F32) {
    switch (head_dim) {
      case 16: return by_heads<float, 4>(heads, f);
      case 32: return by_heads<float, 8>(heads, f);
      case 64: return by_heads<float, 16>(heads, f);
    }
  } else if (dt == GT_BF16) {
    switch (head_dim) {
      case 16: return by_heads<bf16_t, 2>(heads, f);
      case 32: return by_heads<bf16_t, 4>(heads, f);
      case 64: return by_heads<bf16_t, 8>(heads, f);
    }
  }
  return false;
}

struct NopF {
  template <typename T, int HL, int H> void operator()() {}
};

struct FwdF {
  const FwdArgs &a;
  bool bias;
  hipStream_t st;
  gt_status &rc;
  template <typename T, int HL, int H> void operator()() { rc = run_fwd<T, HL, H>(a, bias, st); }
};

struct BwdF {
  const BwdArgs &a;
  bool bias;
  hipStream_t st;
  gt_status &rc;
  template <typename T, int HL, int H> void operator()() { rc = run_bwd<T, HL, H>(a, bias, st); }
};

bool shape_supported(gt_dtype dt, int heads, int head_dim) {
  return dispatch(dt, heads, head_dim, NopF{});
}

static Sched sched_of(const gt_sched &s, const int32_t *ptr) {
  Sched r;
  r.ptr = ptr;
  r.order = s.order;
  r.items = s.items;
  r.merges = s.merges;
  r.n_big = s.n_big;
  r.n_mid = s.n_mid;
  r.n_small = s.n_small;
  r.n_items = s.n_items;
  r.n_merges = s.n_merges;
  return r;
}

gt_status launch_fwd(const gt_graph *g, int heads, int head_dim, gt_dtype dt, float scale,
                     const void *Q, const void *K, const void *V, const float *bias, void *Y,
                     float *lse, float *part_ml, float *part_acc, hipStream_t st) {
  FwdArgs a;
  a.s = sched_of(g->rows, g->indptr);
  a.idx = g->indices;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.bias = bias;
  a.Y = Y;
  a.lse = lse;
  a.part_ml = part_ml;
  a.part_acc = part_acc;
  a.qscale = scale * LOG2E;
  gt_status rc = GT_OK;
  FwdF f{a, bias != nullptr, st, rc};
  if (!dispatch(dt, heads, head_dim, f)) return fail(GT_E_SHAPE, "unsupported shape");
  return rc;
}

gt_status launch_bwd(const gt_graph *g, int heads, int head_dim, gt_dtype dt, float scale,
                     const void *Q, const void *K, const void *V, const float *bias,
                     const float *lse, const void *dY, void *dQ, void *dK,
                     void *dV, float *dbias, float *rowstat, float *part_rows, float *part_cols,
                     hipStream_t st) {
  BwdArgs a;
  a.rows = sched_of(g->rows, g->indptr);
  a.cols = sched_of(g->cols, g->indptr_t);
  a.idx = g->indices;
  a.idx_t = g->indices_t;
  a.perm = g->perm;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.dY = dY;
  a.lse = lse;
  a.bias = bias;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.dbias = dbias;
  a.rowstat = reinterpret_cast<float2 *>(rowstat);
  a.part_rows = part_rows;
  a.part_cols = part_cols;
  a.qscale = scale * LOG2E;
  a.scale = scale;
  gt_status rc = GT_OK;
  BwdF f{a, bias != nullptr, st, rc};
  if (!dispatch(dt, heads, head_dim, f)) return fail(GT_E_SHAPE, "unsupported shape");
  return rc;
}

}  // namespace gt
