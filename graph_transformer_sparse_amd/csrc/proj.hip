// Dense projections of a sparse graph attention layer ("Scalable and Adaptive
// Parallel Training of Graph Transformer on Large Graphs", Section 2.1,
// Eq. 3 and 5): Q/K/V = X W_{Q,K,V}, Z = X W_o + Y, and their gradients
// dX = dZ W_o^T + dQ W_Q^T + dK W_K^T + dV W_V^T, dW_* = X^T d*.
//
// These are real dense contractions, so they run on the matrix cores:
// v_mfma_f32_32x32x8_bf16 (bf16 inputs) and v_mfma_f32_32x32x2_f32 (fp32),
// fp32 accumulation.  With n nodes >> d (d = heads * head_dim <= 256) every
// product moves O(n d) bytes for O(n d^2) flops, so the kernels are built to
// stream the node-feature arrays once: 128-row tiles of the [n, d] operands,
// the [d, d] weights (L2-resident) staged through LDS in 32-wide k chunks.
//
// MFMA 32x32 operand layout (per lane l of the wavefront): A[m][k] with
// m = l % 32 and k = KW*(l / 32) + i, B[k][n] with n = l % 32 and the same k,
// i < KW (KW = 4 for bf16, 1 for fp32); accumulator element v of lane l is
// D[m][n] with n = l % 32 and m = 8*(v / 4) + 4*(l / 32) + v % 4.
#include <algorithm>

#include "device.hpp"
#include "host.hpp"

namespace gt {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  static constexpr int KSTEP = 8, KW = 4;    // k per instruction, k per lane
  static constexpr int PAD = 8;              // LDS row padding (elements)
  __device__ static inline v16f mma(const bf16_t *a, const bf16_t *b, v16f c) {
    const v4s av = *reinterpret_cast<const v4s *>(a);
    const v4s bv = *reinterpret_cast<const v4s *>(b);
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(av, bv, c, 0, 0, 0);
  }
  __device__ static inline bf16_t cvt(float x) { return bf16_t{(uint16_t)f32_to_bf16_bits(x)}; }
  __device__ static inline float val(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }
};
template <> struct Mma<float> {
  static constexpr int KSTEP = 2, KW = 1;
  static constexpr int PAD = 4;
  __device__ static inline v16f mma(const float *a, const float *b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(*a, *b, c, 0, 0, 0);
  }
  __device__ static inline float cvt(float x) { return x; }
  __device__ static inline float val(float x) { return x; }
};

constexpr int PKC = 32;  // k chunk staged in LDS

// one 16-byte vector of a row-major operand, zero past the end
template <typename T>
__device__ inline uint4 load16(const T *p, bool ok) {
  return ok ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// row GEMM: C_z[rows, cols] = sum_s A_s[rows, :] op(B_zs) (+ R), with
// op(W) = W or W^T, every operand [n, d] or [d, d] row-major.
// grid (ceil(n/128), d/BN, outputs); 4 wavefronts, wavefront w owns rows
// [32w, 32w+32) of the tile and all BN columns.
// ---------------------------------------------------------------------------
struct RowsGemm {
  const void *A[4];
  const void *B[3][4];
  void *C[3];
  const void *R;     // residual added to C[0] (nullable)
  int64_t n;
  int d, na;
};

template <typename T, int BN, bool TRANSB>
__global__ __launch_bounds__(256) void k_gemm_rows(RowsGemm g) {
  using M = Mma<T>;
  constexpr int BM = 128, LD = PKC + M::PAD, AV = 16 / sizeof(T);
  __shared__ __align__(16) T As[BM * LD];
  __shared__ __align__(16) T Bs[BN * LD];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN, z = blockIdx.z, d = g.d;
  const int koff = M::KW * (lane / 32);
  v16f acc[BN / 32];
#pragma unroll
  for (int j = 0; j < BN / 32; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  for (int s = 0; s < g.na; ++s) {
    const T *A = (const T *)g.A[s];
    const T *B = (const T *)g.B[z][s];
    for (int k0 = 0; k0 < d; k0 += PKC) {
      __syncthreads();
      for (int i = tid; i < BM * PKC / AV; i += 256) {
        const int r = i / (PKC / AV), c = (i % (PKC / AV)) * AV;
        const int64_t row = m0 + r;
        *reinterpret_cast<uint4 *>(&As[r * LD + c]) = load16(A + row * d + k0 + c, row < g.n);
      }
      if constexpr (TRANSB) {   // B[k][n] = W[n][k]: rows of W are k-contiguous
        for (int i = tid; i < BN * PKC / AV; i += 256) {
          const int nn = i / (PKC / AV), c = (i % (PKC / AV)) * AV;
          *reinterpret_cast<uint4 *>(&Bs[nn * LD + c]) = load16(B + (int64_t)(n0 + nn) * d + k0 + c, true);
        }
      } else {                  // B[k][n] = W[k][n]: scatter into Bs[n][k]
        for (int i = tid; i < PKC * BN / AV; i += 256) {
          const int kk = i / (BN / AV), c = (i % (BN / AV)) * AV;
          const uint4 v = load16(B + (int64_t)(k0 + kk) * d + n0 + c, true);
          const T *e = reinterpret_cast<const T *>(&v);
#pragma unroll
          for (int q = 0; q < AV; ++q) Bs[(c + q) * LD + kk] = e[q];
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < PKC; kk += M::KSTEP) {
        const T *a = &As[(32 * w + lane % 32) * LD + kk + koff];
#pragma unroll
        for (int j = 0; j < BN / 32; ++j)
          acc[j] = M::mma(a, &Bs[(32 * j + lane % 32) * LD + kk + koff], acc[j]);
      }
    }
  }
  T *C = (T *)g.C[z];
  const T *R = (z == 0) ? (const T *)g.R : nullptr;
#pragma unroll
  for (int j = 0; j < BN / 32; ++j) {
    const int col = n0 + 32 * j + lane % 32;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = m0 + 32 * w + 8 * (v / 4) + 4 * (lane / 32) + v % 4;
      if (row < g.n) {
        float x = acc[j][v];
        if (R) x += M::val(R[row * d + col]);
        C[row * d + col] = M::cvt(x);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// weight gradient: part[s][chunk] = X[rows of chunk]^T G_s[rows of chunk]
// (an MT x BN tile of the [d, d] result per workgroup), then a fixed-order sum
// over chunks.  grid (chunks, tiles, grads); MT/32 wavefronts.
// ---------------------------------------------------------------------------
struct WgradGemm {
  const void *X;
  const void *G[4];
  float *part;       // [grads][chunks][d][d]
  float *dW[4];
  int64_t n, rows_per_chunk, chunks;
  int d, ngrad;
};

template <typename T, int MT, int BN>
__global__ __launch_bounds__(MT * 2) void k_gemm_wgrad(WgradGemm g) {
  using M = Mma<T>;
  constexpr int NT = MT * 2, LD = PKC + M::PAD, AV = 16 / sizeof(T);
  __shared__ __align__(16) T As[MT * LD];
  __shared__ __align__(16) T Bs[BN * LD];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int d = g.d, tiles_n = d / BN;
  const int m0 = (blockIdx.y / tiles_n) * MT, n0 = (blockIdx.y % tiles_n) * BN, s = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.x * g.rows_per_chunk;
  const int64_t r1 = r0 + g.rows_per_chunk < g.n ? r0 + g.rows_per_chunk : g.n;
  const T *X = (const T *)g.X, *G = (const T *)g.G[s];
  const int koff = M::KW * (lane / 32);
  v16f acc[BN / 32];
#pragma unroll
  for (int j = 0; j < BN / 32; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  for (int64_t k0 = r0; k0 < r1; k0 += PKC) {
    __syncthreads();
    // As[m][k] = X[k0 + k][m0 + m], Bs[n][k] = G[k0 + k][n0 + n]; rows past r1 are 0
    for (int i = tid; i < PKC * MT / AV; i += NT) {
      const int kk = i / (MT / AV), c = (i % (MT / AV)) * AV;
      const int64_t row = k0 + kk;
      const uint4 v = load16(X + row * d + m0 + c, row < r1);
      const T *e = reinterpret_cast<const T *>(&v);
#pragma unroll
      for (int q = 0; q < AV; ++q) As[(c + q) * LD + kk] = e[q];
    }
    for (int i = tid; i < PKC * BN / AV; i += NT) {
      const int kk = i / (BN / AV), c = (i % (BN / AV)) * AV;
      const int64_t row = k0 + kk;
      const uint4 v = load16(G + row * d + n0 + c, row < r1);
      const T *e = reinterpret_cast<const T *>(&v);
#pragma unroll
      for (int q = 0; q < AV; ++q) Bs[(c + q) * LD + kk] = e[q];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < PKC; kk += M::KSTEP) {
      const T *a = &As[(32 * w + lane % 32) * LD + kk + koff];
#pragma unroll
      for (int j = 0; j < BN / 32; ++j)
        acc[j] = M::mma(a, &Bs[(32 * j + lane % 32) * LD + kk + koff], acc[j]);
    }
  }
  float *P = g.part + ((int64_t)s * g.chunks + blockIdx.x) * d * d;
#pragma unroll
  for (int j = 0; j < BN / 32; ++j) {
    const int col = n0 + 32 * j + lane % 32;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m0 + 32 * w + 8 * (v / 4) + 4 * (lane / 32) + v % 4;
      P[(int64_t)row * d + col] = acc[j][v];
    }
  }
}

// dW_s[i] = sum over chunks, in chunk order, of part[s][chunk][i]
__global__ void k_wgrad_reduce(WgradGemm g) {
  const int64_t dd = (int64_t)g.d * g.d;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= dd * g.ngrad) return;
  const int s = (int)(t / dd);
  const int64_t i = t % dd;
  const float *p = g.part + (int64_t)s * g.chunks * dd + i;
  float x = 0.f;
  for (int64_t c = 0; c < g.chunks; ++c) x += p[c * dd];
  g.dW[s][i] = x;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr int64_t WGRAD_ROWS = 8192;   // node rows per weight-gradient chunk

int64_t wgrad_chunks(int64_t n) { return n > 0 ? cdiv(n, WGRAD_ROWS) : 0; }

template <typename T, bool TRANSB>
static gt_status run_rows(const RowsGemm &g, int nout, hipStream_t st) {
  if (g.n == 0) return GT_OK;
  const unsigned gx = (unsigned)cdiv(g.n, 128);
  if (g.d == 64) {
    k_gemm_rows<T, 64, TRANSB><<<dim3(gx, 1, nout), 256, 0, st>>>(g);
  } else {
    k_gemm_rows<T, 128, TRANSB><<<dim3(gx, g.d / 128, nout), 256, 0, st>>>(g);
  }
  GT_CHECK_LAUNCH();
  return GT_OK;
}

gt_status launch_rows_gemm(gt_dtype dt, const RowsGemm &g, int nout, bool transb, hipStream_t st) {
  if (dt == GT_F32)
    return transb ? run_rows<float, true>(g, nout, st) : run_rows<float, false>(g, nout, st);
  return transb ? run_rows<bf16_t, true>(g, nout, st) : run_rows<bf16_t, false>(g, nout, st);
}

template <typename T>
static gt_status run_wgrad(WgradGemm &g, hipStream_t st) {
  if (g.chunks > 0) {
    if (g.d == 64) {
      k_gemm_wgrad<T, 64, 64><<<dim3((unsigned)g.chunks, 1, g.ngrad), 128, 0, st>>>(g);
    } else {
      const int tiles = (g.d / 128) * (g.d / 128);
      k_gemm_wgrad<T, 128, 128><<<dim3((unsigned)g.chunks, tiles, g.ngrad), 256, 0, st>>>(g);
    }
    GT_CHECK_LAUNCH();
  }
  const int64_t total = (int64_t)g.d * g.d * g.ngrad;
  k_wgrad_reduce<<<dim3((unsigned)cdiv(total, 256)), 256, 0, st>>>(g);
  GT_CHECK_LAUNCH();
  return GT_OK;
}

gt_status launch_wgrad(gt_dtype dt, WgradGemm &g, hipStream_t st) {
  return dt == GT_F32 ? run_wgrad<float>(g, st) : run_wgrad<bf16_t>(g, st);
}

}  // namespace gt

// ---------------------------------------------------------------------------
// C ABI (include/gt_proj.h)
// ---------------------------------------------------------------------------
using namespace gt;

namespace {

gt_status check_proj(int64_t n, int32_t d, gt_dtype dt) {
  if (dt != GT_F32 && dt != GT_BF16) return fail(GT_E_DTYPE, "unknown dtype %d", (int)dt);
  if (d != 64 && d != 128 && d != 256) return fail(GT_E_SHAPE, "d = %d: supported 64, 128, 256", d);
  if (n < 0 || n >= INT32_MAX) return fail(GT_E_ARG, "n = %lld out of range", (long long)n);
  return GT_OK;
}

gt_status need(const void *p, const char *name, bool req) {
  if (!req) return GT_OK;
  if (!p) return fail(GT_E_NULL, "%s is NULL", name);
  if (((uintptr_t)p & 15u) != 0) return fail(GT_E_ALIGN, "%s is not 16-byte aligned", name);
  return GT_OK;
}

#define PTRY(x)                 \
  do {                          \
    gt_status s_ = (x);         \
    if (s_ != GT_OK) return s_; \
  } while (0)

}  // namespace

extern "C" gt_status gt_proj_qkv(int64_t n, int32_t d, gt_dtype dt, const void *X,
                                 const void *Wq, const void *Wk, const void *Wv, void *Q, void *K,
                                 void *V, void *stream) {
  clear_error();
  PTRY(check_proj(n, d, dt));
  PTRY(need(Wq, "Wq", true));
  PTRY(need(Wk, "Wk", true));
  PTRY(need(Wv, "Wv", true));
  PTRY(need(X, "X", n > 0));
  PTRY(need(Q, "Q", n > 0));
  PTRY(need(K, "K", n > 0));
  PTRY(need(V, "V", n > 0));
  RowsGemm g = {};
  g.A[0] = X;
  g.B[0][0] = Wq;
  g.B[1][0] = Wk;
  g.B[2][0] = Wv;
  g.C[0] = Q;
  g.C[1] = K;
  g.C[2] = V;
  g.n = n;
  g.d = d;
  g.na = 1;
  return launch_rows_gemm(dt, g, 3, false, (hipStream_t)stream);
}

extern "C" gt_status gt_proj_out(int64_t n, int32_t d, gt_dtype dt, const void *X,
                                 const void *Wo, const void *Y, void *Z, void *stream) {
  clear_error();
  PTRY(check_proj(n, d, dt));
  PTRY(need(Wo, "Wo", true));
  PTRY(need(X, "X", n > 0));
  PTRY(need(Y, "Y", n > 0));
  PTRY(need(Z, "Z", n > 0));
  RowsGemm g = {};
  g.A[0] = X;
  g.B[0][0] = Wo;
  g.C[0] = Z;
  g.R = Y;
  g.n = n;
  g.d = d;
  g.na = 1;
  return launch_rows_gemm(dt, g, 1, false, (hipStream_t)stream);
}

extern "C" gt_status gt_proj_bwd_data(int64_t n, int32_t d, gt_dtype dt, const void *dZ,
                                      const void *dQ, const void *dK, const void *dV,
                                      const void *Wo, const void *Wq, const void *Wk,
                                      const void *Wv, void *dX, void *stream) {
  clear_error();
  PTRY(check_proj(n, d, dt));
  const void *ins[4] = {dZ, dQ, dK, dV}, *ws[4] = {Wo, Wq, Wk, Wv};
  const char *in_names[4] = {"dZ", "dQ", "dK", "dV"}, *w_names[4] = {"Wo", "Wq", "Wk", "Wv"};
  RowsGemm g = {};
  for (int s = 0; s < 4; ++s) {
    PTRY(need(ins[s], in_names[s], n > 0));
    PTRY(need(ws[s], w_names[s], true));
    g.A[s] = ins[s];
    g.B[0][s] = ws[s];
  }
  PTRY(need(dX, "dX", n > 0));
  g.C[0] = dX;
  g.n = n;
  g.d = d;
  g.na = 4;
  return launch_rows_gemm(dt, g, 1, true, (hipStream_t)stream);
}

extern "C" size_t gt_proj_work_bytes(int64_t n, int32_t d) {
  if (n < 0 || d <= 0) return 0;
  return (size_t)std::max<int64_t>(4 * wgrad_chunks(n) * (int64_t)d * d * 4, 256);
}

extern "C" gt_status gt_proj_bwd_weight(int64_t n, int32_t d, gt_dtype dt, const void *X,
                                        const void *dZ, const void *dQ, const void *dK,
                                        const void *dV, float *dWo, float *dWq, float *dWk,
                                        float *dWv, void *work, size_t work_bytes,
                                        void *stream) {
  clear_error();
  PTRY(check_proj(n, d, dt));
  const void *gs[4] = {dZ, dQ, dK, dV};
  float *dws[4] = {dWo, dWq, dWk, dWv};
  const char *g_names[4] = {"dZ", "dQ", "dK", "dV"}, *w_names[4] = {"dWo", "dWq", "dWk", "dWv"};
  WgradGemm g = {};
  PTRY(need(X, "X", n > 0));
  for (int s = 0; s < 4; ++s) {
    PTRY(need(gs[s], g_names[s], n > 0));
    PTRY(need(dws[s], w_names[s], true));
    g.G[s] = gs[s];
    g.dW[s] = dws[s];
  }
  PTRY(need(work, "work", true));
  const size_t nb = gt_proj_work_bytes(n, d);
  if (work_bytes < nb) return fail(GT_E_WORKSPACE, "work has %zu bytes, needs %zu", work_bytes, nb);
  g.X = X;
  g.part = (float *)work;
  g.n = n;
  g.rows_per_chunk = WGRAD_ROWS;
  g.chunks = wgrad_chunks(n);
  g.d = d;
  g.ngrad = 4;
  return launch_wgrad(dt, g, (hipStream_t)stream);
}
