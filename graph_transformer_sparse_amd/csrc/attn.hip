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

#include <stdlib.h>

#include "device.hpp"
#include "host.hpp"
#include "layout.hpp"

namespace gt {

constexpr int BLOCK = 256;
constexpr int WPB = BLOCK / WAVE;

struct Sched {
  const int32_t *order;  // degree order
  const int32_t *items;  // [n_items][4]
  const int32_t *merges; // [n_merges][3]
  const int32_t *spans;  // [n_seg][2] extent of each segment of `order`
  int64_t n_big, n_mid, n_small, n_items, n_merges;
  int64_t block_base;    // workgroup offset of this launch (grids larger than one launch
                         // allows go out in several launches)
};

// The segment a lane group works on.  wave_item: the whole wavefront shares
// one (piece of a) segment.
struct Work {
  int32_t seg, eb, ee, slot;
  bool wave_item, active;
};

template <int RPW>
__device__ inline Work decode(const Sched &s, int grp) {
  const int64_t w = (s.block_base + blockIdx.x) * WPB + threadIdx.x / WAVE;
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
    const int64_t o = s.n_big + (w - s.n_items);
    k.seg = s.order[o];
    const int2 sp = *reinterpret_cast<const int2 *>(s.spans + 2 * o);
    k.eb = sp.x;
    k.ee = sp.y;
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
      const int64_t o = s.n_big + s.n_mid + q;
      k.seg = s.order[o];
      const int2 sp = *reinterpret_cast<const int2 *>(s.spans + 2 * o);
      k.eb = sp.x;
      k.ee = sp.y;
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
// Per-pass partial states.  A state is one lane's share of a segment's
// partial result: vectors over the lane's N channels and per-head scalars
// (equal on the HL lanes of a head).  merge() folds another state in, in a
// fixed order; xor_lane() fetches a partner lane's state; put()/get() move
// it to / from a piece slot (layouts in layout.hpp).
// ---------------------------------------------------------------------------
template <int N> struct FwdState {
  float m, l, acc[N];
  __device__ void init() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int c = 0; c < N; ++c) acc[c] = 0.f;
  }
  __device__ void merge(const FwdState &o) {
    float mn, fa, fb;
    merge_weights(m, o.m, mn, fa, fb);
    l = l * fa + o.l * fb;
#pragma unroll
    for (int c = 0; c < N; ++c) acc[c] = acc[c] * fa + o.acc[c] * fb;
    m = mn;
  }
  __device__ FwdState xor_lane(int off) const {
    FwdState o;
    o.m = __shfl_xor(m, off);
    o.l = __shfl_xor(l, off);
#pragma unroll
    for (int c = 0; c < N; ++c) o.acc[c] = __shfl_xor(acc[c], off);
    return o;
  }
  template <int D, int H> __device__ void put(float *slot, int gl, int h, bool head_lane) const {
#pragma unroll
    for (int c = 0; c < N; c += 4)
      *reinterpret_cast<float4 *>(slot + gl * N + c) = make_float4(acc[c], acc[c + 1], acc[c + 2], acc[c + 3]);
    if (head_lane) {
      slot[D + h] = m;
      slot[D + H + h] = l;
    }
  }
  template <int D, int H> __device__ void get(const float *slot, int gl, int h) {
#pragma unroll
    for (int c = 0; c < N; c += 4) {
      const float4 v = *reinterpret_cast<const float4 *>(slot + gl * N + c);
      acc[c] = v.x; acc[c + 1] = v.y; acc[c + 2] = v.z; acc[c + 3] = v.w;
    }
    m = slot[D + h];
    l = slot[D + H + h];
  }
};

// Backward row pass (see the comment above k_bwd_rows).
template <int N> struct RowState {
  float a1[N], a2[N], s, l, c;
  __device__ void init() {
    s = l = c = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k) a1[k] = a2[k] = 0.f;
  }
  // this (+)= o at this state's shift, unless this one is empty
  __device__ void merge(const RowState &o) {
    if (l == 0.f) {
      *this = o;
      return;
    }
    const float dc = o.c - c;
    s += o.s + dc * o.l;
    l += o.l;
#pragma unroll
    for (int k = 0; k < N; ++k) {
      a1[k] += o.a1[k] + dc * o.a2[k];
      a2[k] += o.a2[k];
    }
  }
  __device__ RowState xor_lane(int off) const {
    RowState o;
    o.s = __shfl_xor(s, off);
    o.l = __shfl_xor(l, off);
    o.c = __shfl_xor(c, off);
#pragma unroll
    for (int k = 0; k < N; ++k) {
      o.a1[k] = __shfl_xor(a1[k], off);
      o.a2[k] = __shfl_xor(a2[k], off);
    }
    return o;
  }
  template <int D, int H> __device__ void put(float *slot, int gl, int h, bool head_lane) const {
#pragma unroll
    for (int k = 0; k < N; k += 4) {
      *reinterpret_cast<float4 *>(slot + gl * N + k) = make_float4(a1[k], a1[k + 1], a1[k + 2], a1[k + 3]);
      *reinterpret_cast<float4 *>(slot + D + gl * N + k) = make_float4(a2[k], a2[k + 1], a2[k + 2], a2[k + 3]);
    }
    if (head_lane) {
      slot[2 * D + h] = s;
      slot[2 * D + H + h] = l;
      slot[2 * D + 2 * H + h] = c;
    }
  }
  template <int D, int H> __device__ void get(const float *slot, int gl, int h) {
#pragma unroll
    for (int k = 0; k < N; k += 4) {
      const float4 x = *reinterpret_cast<const float4 *>(slot + gl * N + k);
      const float4 y = *reinterpret_cast<const float4 *>(slot + D + gl * N + k);
      a1[k] = x.x; a1[k + 1] = x.y; a1[k + 2] = x.z; a1[k + 3] = x.w;
      a2[k] = y.x; a2[k + 1] = y.y; a2[k + 2] = y.z; a2[k + 3] = y.w;
    }
    s = slot[2 * D + h];
    l = slot[2 * D + H + h];
    c = slot[2 * D + 2 * H + h];
  }
};

// Backward column pass: plain sums of the dK and dV terms.
template <int N> struct ColState {
  float k[N], v[N];
  __device__ void init() {
#pragma unroll
    for (int c = 0; c < N; ++c) k[c] = v[c] = 0.f;
  }
  __device__ void merge(const ColState &o) {
#pragma unroll
    for (int c = 0; c < N; ++c) {
      k[c] += o.k[c];
      v[c] += o.v[c];
    }
  }
  __device__ ColState xor_lane(int off) const {
    ColState o;
#pragma unroll
    for (int c = 0; c < N; ++c) {
      o.k[c] = __shfl_xor(k[c], off);
      o.v[c] = __shfl_xor(v[c], off);
    }
    return o;
  }
  template <int D, int H> __device__ void put(float *slot, int gl, int, bool) const {
#pragma unroll
    for (int c = 0; c < N; c += 4) {
      *reinterpret_cast<float4 *>(slot + gl * N + c) = make_float4(k[c], k[c + 1], k[c + 2], k[c + 3]);
      *reinterpret_cast<float4 *>(slot + D + gl * N + c) = make_float4(v[c], v[c + 1], v[c + 2], v[c + 3]);
    }
  }
  template <int D, int H> __device__ void get(const float *slot, int gl, int) {
#pragma unroll
    for (int c = 0; c < N; c += 4) {
      const float4 x = *reinterpret_cast<const float4 *>(slot + gl * N + c);
      const float4 y = *reinterpret_cast<const float4 *>(slot + D + gl * N + c);
      k[c] = x.x; k[c + 1] = x.y; k[c + 2] = x.z; k[c + 3] = x.w;
      v[c] = y.x; v[c + 1] = y.y; v[c + 2] = y.z; v[c + 3] = y.w;
    }
  }
};

// Fold the lane groups of a wavefront into group 0 by a fixed butterfly
// (group g first meets g ^ 1, then g ^ 2, ...).
template <class S, int G> __device__ inline void wave_combine(S &st) {
#pragma unroll
  for (int off = G; off < WAVE; off <<= 1) {
    const S o = st.xor_lane(off);
    st.merge(o);
  }
}

// The edge ids e, e + step, ... of one round, clamped to the round's first
// (valid) edge past the segment end, and the values idx holds there.
template <int U>
__device__ inline void round_ids(const int32_t *idx, int64_t e, int64_t ee, int step,
                                 int32_t (&v)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t eu = e + (int64_t)u * step;
    v[u] = idx[eu < ee ? eu : e];
  }
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
  float *part;      // [slots][fwd_slot_floats] states of split-row pieces
  float qscale;     // scale * log2(e)
};

template <typename T, int HL, int H>
__device__ inline void finish_fwd(const FwdArgs &a, int64_t row, int gl, int h,
                                  const FwdState<Vec<T>::N> &st) {
  constexpr int N = Vec<T>::N, D = HL * H * N;
  const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
  float y[N];
#pragma unroll
  for (int c = 0; c < N; ++c) y[c] = st.acc[c] * inv;
  Vec<T>::store((T *)a.Y + row * D + gl * N, y);
  if (gl % HL == 0) a.lse[row * H + h] = st.l > 0.f ? (st.m + fast_log2(st.l)) * LN2 : -INFINITY;
}

template <typename T, int HL, int H, int U, bool BIAS>
__global__ __launch_bounds__(BLOCK) void k_fwd(FwdArgs a) {
  constexpr int N = Vec<T>::N, G = HL * H, D = G * N, RPW = WAVE / G;
  const int lane = threadIdx.x & (WAVE - 1), grp = lane / G, gl = lane % G, h = gl / HL;
  const Work wk = decode<RPW>(a.s, grp);
  if (!wk.active) return;
  const T *Kp = (const T *)a.K, *Vp = (const T *)a.V;
  const int64_t row = wk.seg;
  float q[N];
  Vec<T>::load((const T *)a.Q + row * D + gl * N, q);
#pragma unroll
  for (int c = 0; c < N; ++c) q[c] *= a.qscale;
  FwdState<N> st;
  st.init();
  const int gstep = wk.wave_item ? RPW : 1;
  int64_t e = (int64_t)wk.eb + (wk.wave_item ? grp : 0);
  int32_t jn[U];
  if (e < wk.ee) round_ids<U>(a.idx, e, wk.ee, gstep, jn);
  for (; e < wk.ee; e += (int64_t)gstep * U) {
    int32_t j[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      j[u] = jn[u];
      ok[u] = e + (int64_t)u * gstep < wk.ee;
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
    const int64_t en = e + (int64_t)gstep * U;   // prefetch the next round's columns
    if (en < wk.ee) round_ids<U>(a.idx, en, wk.ee, gstep, jn);
    float sc[U];
    float mn = st.m;
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
    // ms: the running maximum, or 0 while every score seen is -inf (edges
    // masked by a -inf bias), so that 2^(-inf - ms) = 0 instead of NaN
    const float ms = mn > -INFINITY ? mn : 0.f;
    const float alpha = fast_exp2(st.m - ms);
    st.l *= alpha;
#pragma unroll
    for (int c = 0; c < N; ++c) st.acc[c] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = fast_exp2(sc[u] - ms);
      float vx[N];
      unpack(vr[u], vx);
      st.l += p;
#pragma unroll
      for (int c = 0; c < N; ++c) st.acc[c] = fmaf(p, vx[c], st.acc[c]);
    }
    st.m = mn;
  }
  if (wk.wave_item) {
    wave_combine<FwdState<N>, G>(st);
    if (grp != 0) return;
    if (wk.slot >= 0) {
      st.template put<D, H>(a.part + (int64_t)wk.slot * fwd_slot_floats(D, H), gl, h, gl % HL == 0);
      return;
    }
  }
  finish_fwd<T, HL, H>(a, row, gl, h, st);
}

// ---------------------------------------------------------------------------
// merge of split segments: one workgroup per segment; lane group g of the
// workgroup folds in pieces g, g + NG, g + 2 NG, ... (NG groups), then the
// groups are folded by the butterfly inside each wavefront and the
// wavefronts in order through LDS.  Returns true on the one group holding
// the result (wavefront 0, group 0).
// ---------------------------------------------------------------------------
template <class S, int D, int H, int G, int64_t SLOT>
__device__ inline bool merge_pieces(S &st, const float *part, int64_t first, int64_t nch, int wv,
                                    int grp, int gl, int h) {
  constexpr int RPW = WAVE / G, NG = WPB * RPW, UNR = 4;
  __shared__ S lds[WPB * G];
  const int gid = wv * RPW + grp;
  st.init();
  for (int64_t k = gid; k < nch; k += (int64_t)NG * UNR) {
    S o[UNR];
#pragma unroll
    for (int q = 0; q < UNR; ++q) {
      const int64_t kk = k + (int64_t)q * NG;
      if (kk < nch) o[q].template get<D, H>(part + (first + kk) * SLOT, gl, h);
      else o[q].init();
    }
#pragma unroll
    for (int q = 0; q < UNR; ++q) st.merge(o[q]);
  }
  wave_combine<S, G>(st);
  if (grp == 0) lds[wv * G + gl] = st;
  __syncthreads();
  if (wv != 0 || grp != 0) return false;
#pragma unroll
  for (int w = 1; w < WPB; ++w) st.merge(lds[w * G + gl]);
  return true;
}

template <typename T, int HL, int H>
__global__ __launch_bounds__(BLOCK) void k_fwd_merge(FwdArgs a) {
  constexpr int N = Vec<T>::N, G = HL * H, D = G * N;
  const int lane = threadIdx.x & (WAVE - 1), grp = lane / G, gl = lane % G, h = gl / HL;
  const int32_t *rec = a.s.merges + 3 * (a.s.block_base + blockIdx.x);
  const int64_t row = rec[0], first = rec[1], nch = rec[2];
  FwdState<N> st;
  if (merge_pieces<FwdState<N>, D, H, G, fwd_slot_floats(D, H)>(st, a.part, first, nch,
                                                                threadIdx.x / WAVE, grp, gl, h))
    finish_fwd<T, HL, H>(a, row, gl, h, st);
}

// ---------------------------------------------------------------------------
// backward, row pass over A: dQ, the per-row (lse2, D) statistics and, with a
// bias, the staged per-edge values dbias is finished from
//
// The weights are recomputed from the forward's log-sum-exp: p_e =
// 2^(s2_e - lse2_i), L = sum_e p_e (1 up to the rounding of lse), and
// U_e = p_e / L.  With dU_e = <dY_i, V_j>, the row term is
// D_i = sum_e U_e dU_e and dQ_i = scale sum_e U_e (dU_e - D_i) K_j.  One pass
// over the row's edges accumulates, around a shift c,
//   L = sum p,  S = sum p (dU - c),  A1 = sum p (dU - c) K,  A2 = sum p K,
// and then D = c + S / L and dQ = scale (A1 - (S / L) A2) / L.  Dividing by
// L makes the weights sum to 1 whatever the rounding of lse (the column pass
// gets lse2 + log2(L) so that its weights are the same U_e); the shift keeps
// the subtraction small.  Two partial states combine at the shift of the
// first non-empty one: S = S_a + S_b + (c_b - c_a) L_b,
// A1 = A1_a + A1_b + (c_b - c_a) A2_b.
//
// The shift.  Without a bias, c is the dU of the first edge a lane group
// sees (a row with one edge then gets dQ = 0 and D = dU exactly).  With a
// bias, c = <dY_i, Y_i> from the forward's output, the same for every lane
// group and piece of the row.  That is D itself up to the rounding of the
// stored Y (2^-9 relative for bf16), so each edge's
//   w_e = p_e (dU_e - c) = L dS_e + p_e (D_i - c)
// is known as soon as the edge is, and is staged in the dbias array in CSR
// edge order (together with p_e: the pair as two bf16 halves for bf16
// storage, w_e alone as float32 for float32 storage, where D - c is at the
// float32 rounding level).  A streaming pass (k_bwd_dbias) then finishes
//   dbias_e = dS_e = (w_e - p_e (D_i - c)) / L
// in place, from the per-row (D - c, 1 / L).  So dbias leaves in whole
// lines, and the column pass over the transpose touches it not at all (its
// scattered 16-byte writes cost more than the staging and the finishing
// pass together).
// ---------------------------------------------------------------------------
struct BwdArgs {
  Sched rows, cols;
  const int32_t *indptr;  // CSR row pointer
  int64_t n_rows, nnz;
  const int32_t *idx;     // CSR columns
  const int32_t *idx_t;   // CSR^T source rows
  const int32_t *perm;    // CSR^T -> CSR edge id
  const void *Q, *K, *V, *Y, *dY;
  const float *lse, *bias;
  void *dQ, *dK, *dV;
  float *dbias;
  float2 *rowstat;        // [R][H] (lse * log2(e) + log2(L), D)
  float2 *fixstat;        // [R][H] (D - c, 1 / L), with a bias
  float *part_rows;       // [slots][rows_slot_floats] states of split-row pieces
  float *part_cols;       // [slots][cols_slot_floats] states of split-column pieces
  float qscale, scale;
};

// <dY_i, Y_i> for the head of this lane (every lane of the row's group gets
// it), in the same operation order as an edge's dU = <dY_i, V_j>.
template <typename T, int HL, int H>
__device__ inline float row_shift(const BwdArgs &a, int64_t row, int gl,
                                  const float (&dy)[Vec<T>::N]) {
  constexpr int N = Vec<T>::N, D = HL * H * N;
  float y[N];
  Vec<T>::load((const T *)a.Y + row * D + gl * N, y);
  float d = 0.f;
#pragma unroll
  for (int c = 0; c < N; ++c) d = fmaf(dy[c], y[c], d);
  return group_sum<HL>(d);
}

// The staged value of one edge and head: (p, w) as two bf16 halves, or w
// as float32 (see above); and its inverse, used by k_bwd_dbias.
template <typename T> __device__ inline float stage(float p, float w);
template <> __device__ inline float stage<float>(float, float w) { return w; }
template <> __device__ inline float stage<bf16_t>(float p, float w) {
  return __uint_as_float((f32_to_bf16_bits(p) << 16) | f32_to_bf16_bits(w));
}
template <typename T> __device__ inline float unstage(float v, float dc, float inv);
template <> __device__ inline float unstage<float>(float v, float, float inv) { return v * inv; }
template <> __device__ inline float unstage<bf16_t>(float v, float dc, float inv) {
  const uint32_t u = __float_as_uint(v);
  const float p = __uint_as_float(u & 0xffff0000u), w = __uint_as_float(u << 16);
  return (w - p * dc) * inv;
}

// Store one round's staged values (edges e + u gstep, u < U): lane r of a
// head's HL lanes stores that head's value of edge r (and r + HL, ...), so a
// round's values leave in one store instruction.
template <int U, int HL, int H>
__device__ inline void stage_store(float *dbias, int64_t e, int gstep, int gl, int h,
                                   const float (&sv)[U], const bool (&ok)[U]) {
#pragma unroll
  for (int u0 = 0; u0 < U; u0 += HL) {
    const int u = u0 + gl % HL;
    if (u < U) {
      float v = sv[0];
      bool w = ok[0];
#pragma unroll
      for (int k = 1; k < U; ++k)
        if (u == k) {
          v = sv[k];
          w = ok[k];
        }
      if (w) dbias[(e + (int64_t)u * gstep) * H + h] = v;
    }
  }
}

// dQ and the row statistics of one row from its state (all lanes of the
// row's group; lane gl holds channels [gl*N, gl*N + N)).
template <typename T, int HL, int H, bool BIAS>
__device__ inline void finish_row(const BwdArgs &a, int64_t row, int gl, int h, float lse2,
                                  const RowState<Vec<T>::N> &st) {
  constexpr int N = Vec<T>::N, D = HL * H * N;
  const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
  const float ds = st.s * inv;
  float g[N];
#pragma unroll
  for (int c = 0; c < N; ++c) g[c] = a.scale * ((st.a1[c] - ds * st.a2[c]) * inv);
  Vec<T>::store((T *)a.dQ + row * D + gl * N, g);
  if (gl % HL == 0) {
    a.rowstat[row * H + h] =
        st.l > 0.f ? make_float2(lse2 + fast_log2(st.l), st.c + ds) : make_float2(-INFINITY, 0.f);
    if constexpr (BIAS) a.fixstat[row * H + h] = make_float2(ds, inv);
  }
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
  // lse = -inf: every edge of the row is masked (weight 0 throughout)
  const bool live = lse2 > -INFINITY;
  RowState<N> st;
  st.init();
  if constexpr (BIAS) st.c = row_shift<T, HL, H>(a, row, gl, dy);
  const int gstep = wk.wave_item ? RPW : 1;
  int64_t e = (int64_t)wk.eb + (wk.wave_item ? grp : 0);
  int32_t jn[U];
  if (e < wk.ee) round_ids<U>(a.idx, e, wk.ee, gstep, jn);
  bool first = true;
  // the previous round's staged values (bias): stored after this round's
  // loads are issued, so that waiting for those loads (the memory counter
  // is in order) does not also wait for the store
  float sv[U];
  bool sok[U];
  int64_t se = -1;
  for (; e < wk.ee; e += (int64_t)gstep * U) {
    int32_t j[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      j[u] = jn[u];
      ok[u] = e + (int64_t)u * gstep < wk.ee;
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
    const int64_t en = e + (int64_t)gstep * U;
    if (en < wk.ee) round_ids<U>(a.idx, en, wk.ee, gstep, jn);
    if constexpr (BIAS) {
      if (se >= 0) stage_store<U, HL, H>(a.dbias, se, gstep, gl, h, sv, sok);
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
      if (!BIAS && u == 0 && first) st.c = du;   // edge e is valid in every round
      const float p = (ok[u] && live) ? fast_exp2(s - lse2) : 0.f;
      const float pt = p * (du - st.c);
      if constexpr (BIAS) {
        sv[u] = stage<T>(p, pt);
        sok[u] = ok[u];
      }
      st.l += p;
      st.s += pt;
#pragma unroll
      for (int c = 0; c < N; ++c) {
        st.a1[c] = fmaf(pt, kx[c], st.a1[c]);
        st.a2[c] = fmaf(p, kx[c], st.a2[c]);
      }
    }
    if constexpr (BIAS) se = e;
    first = false;
  }
  if constexpr (BIAS) {
    if (se >= 0) stage_store<U, HL, H>(a.dbias, se, gstep, gl, h, sv, sok);
  }
  if (wk.wave_item) {
    wave_combine<RowState<N>, G>(st);
    if (grp != 0) return;
    if (wk.slot >= 0) {
      st.template put<D, H>(a.part_rows + (int64_t)wk.slot * rows_slot_floats(D, H), gl, h,
                            gl % HL == 0);
      return;
    }
  }
  finish_row<T, HL, H, BIAS>(a, row, gl, h, lse2, st);
}

template <typename T, int HL, int H, bool BIAS>
__global__ __launch_bounds__(BLOCK) void k_bwd_rows_merge(BwdArgs a) {
  constexpr int N = Vec<T>::N, G = HL * H, D = G * N;
  const int lane = threadIdx.x & (WAVE - 1), grp = lane / G, gl = lane % G, h = gl / HL;
  const int32_t *rec = a.rows.merges + 3 * (a.rows.block_base + blockIdx.x);
  const int64_t row = rec[0], first = rec[1], nch = rec[2];
  RowState<N> st;
  if (merge_pieces<RowState<N>, D, H, G, rows_slot_floats(D, H)>(st, a.part_rows, first, nch,
                                                                 threadIdx.x / WAVE, grp, gl, h))
    finish_row<T, HL, H, BIAS>(a, row, gl, h, a.lse[row * H + h] * LOG2E, st);
}

// dbias from the staged values, streamed in CSR edge order after the row
// pass and its merges (when every row's (D - c, 1 / L) is known).  A
// workgroup takes DB_TILE consecutive edges: two searches give the rows of
// its first and last edge, the row pointers between them go to LDS, and
// each group of four values finds its row there (a tile spanning more rows
// than fit, i.e. many empty rows, searches the global row pointer instead).
constexpr int DB_THREADS = 256, DB_TILE = 2048, DB_ROWS = 2048;

template <typename T, int H>
__global__ __launch_bounds__(DB_THREADS) void k_bwd_dbias(const int32_t *indptr, int64_t n_rows,
                                                           int64_t nnz, const float2 *fixstat,
                                                           float *dbias) {
  __shared__ int32_t ip[DB_ROWS + 1];
  __shared__ int32_t r01[2];
  const int64_t e0 = (int64_t)blockIdx.x * DB_TILE;
  const int64_t e1 = std::min<int64_t>(e0 + DB_TILE, nnz);   // exclusive
  if (threadIdx.x < 2)
    r01[threadIdx.x] = row_of_edge(indptr, n_rows, (int32_t)(threadIdx.x == 0 ? e0 : e1 - 1));
  __syncthreads();
  const int32_t r0 = r01[0];
  const int64_t nr = (int64_t)r01[1] - r0 + 1;               // rows r0 .. r1
  const bool local = nr <= DB_ROWS;
  if (local)
    for (int64_t k = threadIdx.x; k <= nr; k += DB_THREADS) ip[k] = indptr[r0 + k];
  __syncthreads();
  auto row_of = [&](int64_t e) -> int64_t {
    if (!local) return row_of_edge(indptr, n_rows, (int32_t)e);
    int lo = 0, hi = (int)nr;            // last k with ip[k] <= e, in [lo, hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ip[mid] <= e) lo = mid;
      else hi = mid;
    }
    return r0 + lo;
  };
  // values x = e * H + h; e0 * H is a multiple of 4, so a group of four
  // starts 16-byte aligned; with H >= 4 it belongs to one edge
  const int64_t x1 = e1 * H;
  for (int64_t x = e0 * H + 4 * threadIdx.x; x < x1; x += 4 * DB_THREADS) {
    if (x + 4 <= x1) {
      float4 v = *reinterpret_cast<const float4 *>(dbias + x);
      float o[4] = {v.x, v.y, v.z, v.w};
      if constexpr (H >= 4) {
        const int64_t rh = row_of(x / H) * H;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float2 f = fixstat[rh + (x + k) % H];
          o[k] = unstage<T>(o[k], f.x, f.y);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float2 f = fixstat[row_of((x + k) / H) * H + (x + k) % H];
          o[k] = unstage<T>(o[k], f.x, f.y);
        }
      }
      *reinterpret_cast<float4 *>(dbias + x) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
      for (int64_t y = x; y < x1; ++y) {
        const float2 f = fixstat[row_of(y / H) * H + y % H];
        dbias[y] = unstage<T>(dbias[y], f.x, f.y);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// backward, column pass over A^T: dK and dV
// ---------------------------------------------------------------------------
template <typename T, int HL, int H>
__device__ inline void finish_col(const BwdArgs &a, int64_t col, int gl,
                                  const ColState<Vec<T>::N> &st) {
  constexpr int N = Vec<T>::N, D = HL * H * N;
  float k[N];
#pragma unroll
  for (int c = 0; c < N; ++c) k[c] = st.k[c] * a.scale;
  Vec<T>::store((T *)a.dK + col * D + gl * N, k);
  Vec<T>::store((T *)a.dV + col * D + gl * N, st.v);
}

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
  ColState<N> st;
  st.init();
  const int gstep = wk.wave_item ? RPW : 1;
  int64_t t = (int64_t)wk.eb + (wk.wave_item ? grp : 0);
  int32_t in_[U], pn[U];
  if (t < wk.ee) {
    round_ids<U>(a.idx_t, t, wk.ee, gstep, in_);
    if constexpr (BIAS) round_ids<U>(a.perm, t, wk.ee, gstep, pn);
  }
  for (; t < wk.ee; t += (int64_t)gstep * U) {
    int32_t i[U], eid[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      i[u] = in_[u];
      if constexpr (BIAS) eid[u] = pn[u];
      ok[u] = t + (int64_t)u * gstep < wk.ee;
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
    if constexpr (BIAS) {
#pragma unroll
      for (int u = 0; u < U; ++u) b[u] = a.bias[(int64_t)eid[u] * H + h] * LOG2E;
    }
    const int64_t tn = t + (int64_t)gstep * U;
    if (tn < wk.ee) {
      round_ids<U>(a.idx_t, tn, wk.ee, gstep, in_);
      if constexpr (BIAS) round_ids<U>(a.perm, tn, wk.ee, gstep, pn);
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
      // rowstat.x = -inf: a row whose every edge is masked (weight 0)
      const float p = (ok[u] && rs[u].x > -INFINITY) ? fast_exp2(s - rs[u].x) : 0.f;
      const float ds = p * (du - rs[u].y);
#pragma unroll
      for (int c = 0; c < N; ++c) {
        st.v[c] = fmaf(p, gx[c], st.v[c]);
        st.k[c] = fmaf(ds, qx[c], st.k[c]);
      }
    }
  }
  if (wk.wave_item) {
    wave_combine<ColState<N>, G>(st);
    if (grp != 0) return;
    if (wk.slot >= 0) {
      st.template put<D, H>(a.part_cols + (int64_t)wk.slot * cols_slot_floats(D, H), gl, h, false);
      return;
    }
  }
  finish_col<T, HL, H>(a, col, gl, st);
}

template <typename T, int HL, int H>
__global__ __launch_bounds__(BLOCK) void k_bwd_cols_merge(BwdArgs a) {
  constexpr int N = Vec<T>::N, G = HL * H, D = G * N;
  const int lane = threadIdx.x & (WAVE - 1), grp = lane / G, gl = lane % G, h = gl / HL;
  const int32_t *rec = a.cols.merges + 3 * (a.cols.block_base + blockIdx.x);
  const int64_t col = rec[0], first = rec[1], nch = rec[2];
  ColState<N> st;
  if (merge_pieces<ColState<N>, D, H, G, cols_slot_floats(D, H)>(st, a.part_cols, first, nch,
                                                                 threadIdx.x / WAVE, grp, gl, h))
    finish_col<T, HL, H>(a, col, gl, st);
}

// ---------------------------------------------------------------------------
// host side: shape dispatch and launches
// ---------------------------------------------------------------------------
constexpr int UNROLL = 2;   // edges per lane group per round

static int64_t waves_for(const Sched &s, int rpw) {
  return s.n_items + s.n_mid + cdiv(s.n_small, rpw);
}

// At most 2^22 workgroups (2^30 work-items) per launch: a dispatch counts
// its work-items in 32 bits.  Larger grids (only custom thresholds on
// graphs of billions of nonzeros reach this) go out in several launches,
// each told its workgroup offset.  GT_LAUNCH_BLOCKS (a positive integer)
// lowers the limit, so that tests can take the several-launch path on
// small graphs.
static int64_t max_launch_blocks() {
  constexpr int64_t LIMIT = (int64_t)1 << 22;
  const char *e = getenv("GT_LAUNCH_BLOCKS");
  if (e && *e) {
    const long long v = atoll(e);
    if (v > 0 && v < LIMIT) return v;
  }
  return LIMIT;
}

template <class Args, class Kernel>
static void launch_blocks(Kernel kernel, Args a, Sched Args::*sched, int64_t nblocks,
                          hipStream_t st) {
  const int64_t lim = max_launch_blocks();
  for (int64_t b0 = 0; b0 < nblocks; b0 += lim) {
    (a.*sched).block_base = b0;
    kernel<<<dim3((unsigned)std::min(lim, nblocks - b0)), BLOCK, 0, st>>>(a);
  }
}

template <typename T, int HL, int H>
static gt_status run_fwd(const FwdArgs &a, bool bias, hipStream_t st) {
  constexpr int G = HL * H, RPW = WAVE / G;
  const int64_t waves = waves_for(a.s, RPW);
  if (waves > 0) {
    const int64_t nb = cdiv(waves, WPB);
    const int tok = prof_begin(PK_FWD, st);
    if (bias) launch_blocks(k_fwd<T, HL, H, UNROLL, true>, a, &FwdArgs::s, nb, st);
    else launch_blocks(k_fwd<T, HL, H, UNROLL, false>, a, &FwdArgs::s, nb, st);
    prof_end(tok, st);
    GT_CHECK_LAUNCH();
  }
  if (a.s.n_merges > 0) {
    const int tok = prof_begin(PK_FWD_MERGE, st);
    launch_blocks(k_fwd_merge<T, HL, H>, a, &FwdArgs::s, a.s.n_merges, st);
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
    const int64_t nb = cdiv(waves, WPB);
    const int tok = prof_begin(PK_BWD_ROWS, st);
    if (bias) launch_blocks(k_bwd_rows<T, HL, H, UNROLL, true>, a, &BwdArgs::rows, nb, st);
    else launch_blocks(k_bwd_rows<T, HL, H, UNROLL, false>, a, &BwdArgs::rows, nb, st);
    prof_end(tok, st);
    GT_CHECK_LAUNCH();
  }
  if (a.rows.n_merges > 0) {
    const int tok = prof_begin(PK_BWD_ROWS_MERGE, st);
    if (bias) launch_blocks(k_bwd_rows_merge<T, HL, H, true>, a, &BwdArgs::rows, a.rows.n_merges, st);
    else launch_blocks(k_bwd_rows_merge<T, HL, H, false>, a, &BwdArgs::rows, a.rows.n_merges, st);
    prof_end(tok, st);
    GT_CHECK_LAUNCH();
  }
  if (bias && a.nnz > 0) {
    // at most 2^31 / DB_TILE workgroups: one launch
    const int tok = prof_begin(PK_BWD_DBIAS, st);
    k_bwd_dbias<T, H><<<dim3((unsigned)cdiv(a.nnz, DB_TILE)), DB_THREADS, 0, st>>>(
        a.indptr, a.n_rows, a.nnz, a.fixstat, a.dbias);
    prof_end(tok, st);
    GT_CHECK_LAUNCH();
  }
  waves = waves_for(a.cols, RPW);
  if (waves > 0) {
    const int64_t nb = cdiv(waves, WPB);
    const int tok = prof_begin(PK_BWD_COLS, st);
    if (bias) launch_blocks(k_bwd_cols<T, HL, H, UNROLL, true>, a, &BwdArgs::cols, nb, st);
    else launch_blocks(k_bwd_cols<T, HL, H, UNROLL, false>, a, &BwdArgs::cols, nb, st);
    prof_end(tok, st);
    GT_CHECK_LAUNCH();
  }
  if (a.cols.n_merges > 0) {
    const int tok = prof_begin(PK_BWD_COLS_MERGE, st);
    launch_blocks(k_bwd_cols_merge<T, HL, H>, a, &BwdArgs::cols, a.cols.n_merges, st);
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
  // HL = head_dim * sizeof(T) / 16 lanes per head
  if (dt == GT_F32) {
    switch (head_dim) {
      case 8: return by_heads<float, 2>(heads, f);
      case 16: return by_heads<float, 4>(heads, f);
      case 32: return by_heads<float, 8>(heads, f);
      case 64: return by_heads<float, 16>(heads, f);
      case 128: return by_heads<float, 32>(heads, f);
    }
  } else if (dt == GT_BF16) {
    switch (head_dim) {
      case 8: return by_heads<bf16_t, 1>(heads, f);
      case 16: return by_heads<bf16_t, 2>(heads, f);
      case 32: return by_heads<bf16_t, 4>(heads, f);
      case 64: return by_heads<bf16_t, 8>(heads, f);
      case 128: return by_heads<bf16_t, 16>(heads, f);
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

static Sched sched_of(const gt_sched &s) {
  Sched r;
  r.order = s.order;
  r.items = s.items;
  r.merges = s.merges;
  r.spans = s.spans;
  r.n_big = s.n_big;
  r.n_mid = s.n_mid;
  r.n_small = s.n_small;
  r.n_items = s.n_items;
  r.n_merges = s.n_merges;
  r.block_base = 0;
  return r;
}

gt_status launch_fwd(const gt_graph *g, int heads, int head_dim, gt_dtype dt, float scale,
                     const void *Q, const void *K, const void *V, const float *bias, void *Y,
                     float *lse, float *part, hipStream_t st) {
  FwdArgs a;
  a.s = sched_of(g->rows);
  a.idx = g->indices;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.bias = bias;
  a.Y = Y;
  a.lse = lse;
  a.part = part;
  a.qscale = scale * LOG2E;
  gt_status rc = GT_OK;
  FwdF f{a, bias != nullptr, st, rc};
  if (!dispatch(dt, heads, head_dim, f)) return fail(GT_E_SHAPE, "unsupported shape");
  return rc;
}

gt_status launch_bwd(const gt_graph *g, int heads, int head_dim, gt_dtype dt, float scale,
                     const void *Q, const void *K, const void *V, const float *bias,
                     const void *Y, const float *lse, const void *dY, void *dQ, void *dK,
                     void *dV, float *dbias, float *rowstat, float *fixstat, float *part_rows,
                     float *part_cols, hipStream_t st) {
  BwdArgs a;
  a.rows = sched_of(g->rows);
  a.cols = sched_of(g->cols);
  a.indptr = g->indptr;
  a.n_rows = g->n_rows;
  a.nnz = g->nnz;
  a.idx = g->indices;
  a.idx_t = g->indices_t;
  a.perm = g->perm;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.Y = Y;
  a.dY = dY;
  a.lse = lse;
  a.bias = bias;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.dbias = dbias;
  a.rowstat = reinterpret_cast<float2 *>(rowstat);
  a.fixstat = reinterpret_cast<float2 *>(fixstat);
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
