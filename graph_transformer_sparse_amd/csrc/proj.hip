// Dense projections of a sparse graph attention layer ("Scalable and Adaptive
// Parallel Training of Graph Transformer on Large Graphs", Section 2.1,
// Eq. 3 and 5): Q/K/V = X W_{Q,K,V}, Z = X W_o + Y, and their gradients
// dX = dZ W_o^T + dQ W_Q^T + dK W_K^T + dV W_V^T, dW_* = X^T d*.
//
// These are real dense contractions, so they run on the matrix cores:
// v_mfma_f32_32x32x16_bf16 (bf16 inputs) and v_mfma_f32_32x32x2_f32 (fp32),
// fp32 accumulation.  With n nodes >> d (d = heads * head_dim <= 256) every
// product streams O(n d) bytes of node features for O(n d^2) flops.
//
// Operand layout.  A 16-byte "vector" holds AV = 8 bf16 or 4 fp32 values.
// For a k range of 2 AV, lane l of a wavefront holds the vector of row
// m = l % 32 at k offset AV * (l / 32) for the A operand, and of column
// n = l % 32 likewise for B.  For bf16 that vector is exactly the operand of
// one 32x32x16 MFMA; for fp32 it feeds four 32x32x2 MFMAs, step t taking
// element t of both vectors.  Either way every product A[m][k] B[k][n] of the
// range enters the sum once (the fp32 steps visit k in a permuted order,
// the same on both operands).  Accumulator element v of lane l is
// C[m][n] with n = l % 32 and m = 8 (v / 4) + 4 (l / 32) + v % 4.
//
// LDS tiles are rows of 16-byte chunks with an XOR swizzle on the chunk
// index, chosen so that the operand reads (8 rows, one chunk each) and the
// transposing writes of the staging code spread over the banks; the slab
// tiles of the input gradient, whose rows are short, are padded instead.
#include <algorithm>

#include "device.hpp"
#include "host.hpp"

namespace gt {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  __device__ static inline v16f mma(const uint4 &a, const uint4 &b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  __device__ static inline v16f mma(const uint4 &a, const uint4 &b, v16f c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

// one 16-byte vector of a row-major operand, zero past the end
template <typename T>
__device__ inline uint4 load16(const T *p, bool ok) {
  return ok ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
}

__device__ inline uint32_t u4get(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Transposing store of two consecutive rows r0, r1 (AV columns each) into a
// [column][k] tile: column c receives the pair (r0[c], r1[c]) at k, k + 1.
// bf16: one dword per column; fp32: one 8-byte store per column.
template <typename T>
__device__ inline void store_pair_t(T *tile, const uint4 &r0, const uint4 &r1,
                                    int (&off)[16 / sizeof(T)]);
template <>
__device__ inline void store_pair_t<bf16_t>(bf16_t *tile, const uint4 &r0, const uint4 &r1,
                                            int (&off)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t a = u4get(r0, c / 2), b = u4get(r1, c / 2);
    const uint32_t w = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    *reinterpret_cast<uint32_t *>(tile + off[c]) = w;
  }
}
template <>
__device__ inline void store_pair_t<float>(float *tile, const uint4 &r0, const uint4 &r1,
                                           int (&off)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    *reinterpret_cast<uint2 *>(tile + off[c]) = make_uint2(u4get(r0, c), u4get(r1, c));
}

// ---------------------------------------------------------------------------
// row GEMM: C_z[rows, :] = sum_s A_s[rows, :] op(W_zs) (+ R), op(W) = W or W^T,
// every operand [n, D] or [D, D] row-major.  The general, column-tiled form;
// it serves fp32 at D = 256, where neither the weight (256 KB) fits LDS for
// the resident kernel nor a strip with its whole result fits the registers
// for the slab kernel below.
//
// A workgroup of 8 wavefronts takes 256 node rows; wavefront w owns rows
// [32w, 32w + 32) and holds its A strip in registers, loaded straight from
// memory in the operand layout (lane l: row l % 32, vectors at k = 2 AV c +
// AV (l / 32)).  op(W) streams through LDS one 32-column tile at a time,
// stored [n][k], double-buffered: tile t + 1 is fetched into registers while
// tile t is multiplied.  With one source (NA = 1: the Q/K/V and output
// projections) each 32x32 result block is written as soon as it is done;
// with four (NA = 4: the input gradient) the whole row strip accumulates
// before the write.
// ---------------------------------------------------------------------------
struct RowsGemm {
  const void *A[4];
  const void *B[3][4];
  void *C[3];
  const void *R;     // residual added to C[0] (nullable)
  int64_t n;
  int d, na, nout;
};

constexpr int RG_WAVES = 8, RG_THREADS = RG_WAVES * WAVE, RG_ROWS = RG_WAVES * 32;

// chunk swizzle of the [32][D] weight tile: row n, chunk q -> element offset
template <int D, int AV>
__device__ inline int btile_off(int n, int q) {
  return n * D + ((q ^ ((n ^ (n >> 3)) & 7)) * AV);
}

// store the 32 x 32 block (m0.., col0..) of acc to C (+ residual R)
template <typename T>
__device__ inline void store_block(T *C, const T *R, int64_t m0, int col0, int D, int64_t n,
                                   const v16f &acc, int lane);

template <>
__device__ inline void store_block<float>(float *C, const float *R, int64_t m0, int col0, int D,
                                          int64_t n, const v16f &acc, int lane) {
  const int h = lane / 32, col = col0 + lane % 32;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t row = m0 + 8 * (v / 4) + 4 * h + v % 4;
    if (row < n) {
      float x = acc[v];
      if (R) x += R[row * D + col];
      C[row * D + col] = x;
    }
  }
}

// bf16: neighbouring lanes swap one element so that each lane writes two
// adjacent columns of one row as a dword.
template <>
__device__ inline void store_block<bf16_t>(bf16_t *C, const bf16_t *R, int64_t m0, int col0,
                                           int D, int64_t n, const v16f &acc, int lane) {
  const int h = lane / 32, nn = lane % 32, odd = nn & 1;
  const int col = col0 + nn - odd;
#pragma unroll
  for (int v = 0; v < 16; v += 2) {
    const float give = odd ? acc[v] : acc[v + 1];
    const float got = dpp<DPP_QUAD_XOR1>(give);
    const float lo = odd ? got : acc[v], hi = odd ? acc[v + 1] : got;
    const int64_t row = m0 + 8 * (v / 4) + 4 * h + v % 4 + odd;
    if (row < n) {
      float x0 = lo, x1 = hi;
      if (R) {
        const uint32_t r = *reinterpret_cast<const uint32_t *>(R + row * D + col);
        x0 += __uint_as_float(r << 16);
        x1 += __uint_as_float(r & 0xffff0000u);
      }
      *reinterpret_cast<uint32_t *>(C + row * D + col) =
          f32_to_bf16_bits(x0) | (f32_to_bf16_bits(x1) << 16);
    }
  }
}

template <typename T, int D, bool TRANSB, int NA>
__global__ __launch_bounds__(RG_THREADS) void k_gemm_rows(RowsGemm g) {
  using M = Mma<T>;
  constexpr int AV = 16 / sizeof(T);          // elements per vector
  constexpr int CH = D / (2 * AV);            // k ranges of 2 AV
  constexpr int J = D / 32;                   // 32-column blocks (even)
  static_assert(J % 2 == 0, "tile parity");
  constexpr int TILE = 32 * D;                // elements of one weight tile
  // staging: each thread moves SV vectors of a tile (SV = 0.5: half the threads)
  constexpr int TV = TILE / AV;
  constexpr int SV = TV >= RG_THREADS ? TV / RG_THREADS : 1;
  constexpr int SU = TRANSB ? SV : (SV + 1) / 2;   // units: vectors or row pairs
  __shared__ __align__(16) T Bs[2][TILE];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, h = lane / 32;
  const int64_t m0 = (int64_t)blockIdx.x * RG_ROWS + 32 * w;
  const int64_t arow = m0 + lane % 32;
  const bool arow_ok = arow < g.n;
  const int nout = NA == 1 ? g.nout : 1;
  const int ntiles = (NA == 1 ? nout : NA) * J;

  // fetch tile t of the sequence (source s = t / J for NA = 4, output z =
  // t / J for NA = 1; columns 32 (t % J) ..) into registers
  uint4 st[TRANSB ? SV : 2 * SU];
  auto fetch = [&](int t) {
    const int zs = t / J, j = t % J;
    const T *W = (const T *)(NA == 1 ? g.B[zs][0] : g.B[0][zs]);
    if constexpr (TRANSB) {      // tile[n][k] = W[32 j + n][k]
#pragma unroll
      for (int i = 0; i < SV; ++i) {
        const int u = tid + i * RG_THREADS;
        const int q = u % (D / AV), nn = u / (D / AV);
        st[i] = load16(W + (int64_t)(32 * j + nn) * D + q * AV, u < TV);
      }
    } else {                     // tile[n][k] = W[k][32 j + n], rows k, k + 1
#pragma unroll
      for (int i = 0; i < SU; ++i) {
        const int u = tid + i * RG_THREADS;
        const int ng = u % (32 / AV), kp = u / (32 / AV);
        const bool ok = u < TV / 2;
        st[2 * i] = load16(W + (int64_t)(2 * kp) * D + 32 * j + ng * AV, ok);
        st[2 * i + 1] = load16(W + (int64_t)(2 * kp + 1) * D + 32 * j + ng * AV, ok);
      }
    }
  };
  auto put = [&](T *tile) {
    if constexpr (TRANSB) {
#pragma unroll
      for (int i = 0; i < SV; ++i) {
        const int u = tid + i * RG_THREADS;
        if (u < TV)
          *reinterpret_cast<uint4 *>(tile + btile_off<D, AV>(u / (D / AV), u % (D / AV))) = st[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < SU; ++i) {
        const int u = tid + i * RG_THREADS;
        if (u < TV / 2) {
          const int ng = u % (32 / AV), kp = u / (32 / AV), k0 = 2 * kp;
          int off[AV];
#pragma unroll
          for (int c = 0; c < AV; ++c) off[c] = btile_off<D, AV>(ng * AV + c, k0 / AV) + k0 % AV;
          store_pair_t<T>(tile, st[2 * i], st[2 * i + 1], off);
        }
      }
    }
  };

  uint4 a[CH];
  auto load_a = [&](int s) {
    const T *A = (const T *)g.A[s];
#pragma unroll
    for (int c = 0; c < CH; ++c) a[c] = load16(A + arow * D + c * 2 * AV + h * AV, arow_ok);
  };

  v16f acc[NA == 1 ? 1 : J];
#pragma unroll
  for (int j = 0; j < (NA == 1 ? 1 : J); ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;

  fetch(0);
  load_a(0);
  put(Bs[0]);
  __syncthreads();
  // outer loop: output z (NA = 1) or source s (NA = 4); inner: column blocks
  for (int zs = 0; zs < (NA == 1 ? nout : NA); ++zs) {
    if (NA > 1 && zs > 0) load_a(zs);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int t = zs * J + j;          // J is even: tile t sits in Bs[j & 1]
      if (t + 1 < ntiles) fetch(t + 1);
      v16f &c_acc = acc[NA == 1 ? 0 : j];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const uint4 b = *reinterpret_cast<const uint4 *>(Bs[j & 1] + btile_off<D, AV>(lane % 32, 2 * c + h));
        c_acc = M::mma(a[c], b, c_acc);
      }
      if constexpr (NA == 1) {
        store_block<T>((T *)g.C[zs], zs == 0 ? (const T *)g.R : nullptr, m0, 32 * j, D, g.n,
                       c_acc, lane);
#pragma unroll
        for (int v = 0; v < 16; ++v) c_acc[v] = 0.f;
      }
      if (t + 1 < ntiles) put(Bs[(j + 1) & 1]);
      __syncthreads();
    }
  }
  if constexpr (NA > 1) {
#pragma unroll
    for (int j = 0; j < J; ++j)
      store_block<T>((T *)g.C[0], nullptr, m0, 32 * j, D, g.n, acc[j], lane);
  }
}

// ---------------------------------------------------------------------------
// one-source row GEMM with the weight resident in LDS: C_z = A W_z (+ R).
//
// Used where W fits in LDS (D * D elements of at most 128 KB: bf16 up to
// D = 256, fp32 up to D = 128).  A workgroup of 8 wavefronts stages its
// weights once, as [n][k] with the chunk swizzle: all NZ = 3 of Q/K/V where
// they fit together, else the one W_z of its output.  Its wavefronts then
// run without barriers: each takes 32-row strips of A in turn and holds the
// strip in registers (operand layout as above) while the next strip's loads
// are in flight; for each 32-column block it runs CH MFMAs with the strip as
// the B operand and the weight rows as A, so that lane l ends up with row
// l % 32 and columns 8 g + 4 (l / 32) + i of the block (g, i < 4): four
// contiguous values.  fp32 writes them as one 16-byte store; bf16 trades a
// group between lane halves to write 16 bytes too, a pair of blocks at a
// time.  The residual of a block is fetched one or two blocks ahead.  Every global
// access goes through a buffer resource bounded to the strip, so rows past
// n read as zero and their stores are dropped without a branch (which also
// keeps the memory counters exact).  Workgroups that share strips for
// different z sit eight block indices apart (same XCD, same L2).
// ---------------------------------------------------------------------------
constexpr int RR_WAVES = 8, RR_THREADS = RR_WAVES * WAVE;
constexpr uint32_t BUF_WORD3 = 0x00020000u;   // raw buffer, 32-bit elements (gfx9 layout)

__device__ inline __amdgpu_buffer_rsrc_t strip_rsrc(const void *base, int64_t row0, int64_t n,
                                                    int row_bytes) {
  const int64_t rows = row0 < n ? std::min<int64_t>(32, n - row0) : 0;
  const char *p = (const char *)base + (row0 < n ? row0 : 0) * row_bytes;
  return __builtin_amdgcn_make_buffer_rsrc((void *)p, 0, (int)(rows * row_bytes), BUF_WORD3);
}

// float32 -> bfloat16 bits, nearest even, without a branch (NaN stays NaN)
__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return (u & 0x7fffffffu) > 0x7f800000u ? ((u >> 16) | 0x40u) : r;
}

// the four outputs of a lane in one 32x32 block, as stored
template <typename T> struct OutVec;
template <> struct OutVec<float> {
  typedef uint4 type;
  __device__ static inline type load(__amdgpu_buffer_rsrc_t r, int o) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
  }
  __device__ static inline void add(float (&x)[4], const type &v) {
    x[0] += __uint_as_float(v.x); x[1] += __uint_as_float(v.y);
    x[2] += __uint_as_float(v.z); x[3] += __uint_as_float(v.w);
  }
  __device__ static inline void store(__amdgpu_buffer_rsrc_t r, int o, const float (&x)[4]) {
    const uint4 v = make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]),
                               __float_as_uint(x[2]), __float_as_uint(x[3]));
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, o, 0, 0);
  }
};
template <> struct OutVec<bf16_t> {
  typedef uint2 type;
  __device__ static inline type load(__amdgpu_buffer_rsrc_t r, int o) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0));
  }
  __device__ static inline void add(float (&x)[4], const type &v) {
    x[0] += __uint_as_float(v.x << 16); x[1] += __uint_as_float(v.x & 0xffff0000u);
    x[2] += __uint_as_float(v.y << 16); x[3] += __uint_as_float(v.y & 0xffff0000u);
  }
};

// chunk swizzle of the resident weight: the same for rows n and n + 32, so
// that a lane's read offsets do not depend on the column block
__device__ inline int rsw(int n) { return (n ^ ((n >> 3) & 3)) & 7; }

template <typename T, int D, bool RESID, int NZ>
__global__ __launch_bounds__(RR_THREADS) void k_rows_resident(RowsGemm g, int groups) {
  using M = Mma<T>;
  using O = OutVec<T>;
  constexpr int AV = 16 / sizeof(T), CH = D / (2 * AV), J = D / 32, RB = D * (int)sizeof(T);
  constexpr int UNITS = (D / 2) * (D / AV);      // (row pair, column group) units of W
  __shared__ __align__(16) T Ws[NZ * D * D];
  // the wavefront index is uniform: say so, so that strip addresses and the
  // buffer resources built from them live in scalar registers
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), h = lane / 32;
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  // NZ = 1: workgroups split the outputs (z = slot % nout); NZ > 1: every
  // workgroup holds all NZ weights and writes every output of its strips
  const int nsplit = NZ == 1 ? g.nout : 1;
  const int b = blockIdx.x, xcd = b % 8, slot = b / 8;
  const int zs = slot % nsplit, group = slot / nsplit;
  // stage W_z: Ws[z][n][k] = W_z[k][n]
  for (int zz = 0; zz < NZ; ++zz) {
    const T *W = (const T *)g.B[NZ == 1 ? zs : zz][0];
    T *Wz = Ws + zz * D * D;
    for (int u = tid; u < UNITS; u += RR_THREADS) {
      const int ng = u % (D / AV), kp = u / (D / AV), k0 = 2 * kp;
      const uint4 r0 = *reinterpret_cast<const uint4 *>(W + (int64_t)k0 * D + ng * AV);
      const uint4 r1 = *reinterpret_cast<const uint4 *>(W + (int64_t)(k0 + 1) * D + ng * AV);
      int off[AV];
#pragma unroll
      for (int c = 0; c < AV; ++c) {
        const int nn = ng * AV + c;
        off[c] = nn * D + (((k0 / AV) ^ rsw(nn)) * AV) + k0 % AV;
      }
      store_pair_t<T>(Wz, r0, r1, off);
    }
  }
  __syncthreads();
  const int64_t strips = (g.n + 31) / 32;
  const int64_t stride = (int64_t)8 * groups * RR_WAVES;
  const T *A = (const T *)g.A[0];
  const T *R = (const T *)g.R;
  const int aoff = (lane % 32) * RB + h * 16;                  // lane's first A vector
  const int ooff = (lane % 32) * RB + 4 * h * (int)sizeof(T);  // lane's first output
  int woff[4];                                                 // lane's weight chunks
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) woff[c4] = (lane % 32) * D + (((2 * c4 + h) ^ rsw(lane % 32)) * AV);
  // A strips: the next strip's loads go out before this strip's stores, so
  // that waiting for them (the memory counter is in order) never waits for
  // stores.  Two register sets alternate (the loop body is two strips), and
  // everything inside a strip is unrolled so that the counter waits are exact.
  const int64_t q0 = ((int64_t)group * 8 + xcd) * RR_WAVES + w;
  auto load_strip = [&](uint4 (&dst)[CH], int64_t q) {
    const auto ra = strip_rsrc(A, 32 * q, g.n, RB);
#pragma unroll
    for (int c = 0; c < CH; ++c)
      dst[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, aoff + 32 * c, 0, 0));
  };
  auto run_strip = [&](const uint4 (&a)[CH], uint4 (&next)[CH], int64_t q) {
    load_strip(next, q + stride);
    const int64_t row0 = 32 * q;
    const auto rr = strip_rsrc(RESID ? (const void *)R : g.C[0], row0, g.n, RB);
    // residual of block j, fetched RD blocks ahead (one where registers are
    // short: fp32 blocks take twice the registers, and D = 256 holds more)
    constexpr int RD = (sizeof(T) == 4 || D == 256) ? 1 : 2;
    typename O::type rv[RESID ? J : 1][4];
    auto fetch_r = [&](int j) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        rv[j][gq] = O::load(rr, ooff + (32 * j + 8 * gq) * (int)sizeof(T));
    };
    if constexpr (RESID) {
#pragma unroll
      for (int j = 0; j < RD && j < J; ++j) fetch_r(j);
    }
    uint4 held[2];                       // bf16: the even block's stores, see below
#pragma unroll
    for (int t = 0; t < NZ * J; ++t) {
      const int z = t / J, j = t % J;
      const auto rc = strip_rsrc(g.C[NZ == 1 ? zs : z], row0, g.n, RB);
      // keep each block's weight reads in place (hoisting them all would need
      // D * D / 64 registers per lane)
      asm volatile("" ::: "memory");
      if constexpr (RESID) {
        if (j + RD < J) fetch_r(j + RD);
      }
      v16f acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
      const T *wrow = Ws + (z * D + 32 * j) * D;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        // at most 8 (4 at D = 256, where registers are short) weight
        // vectors in flight per wavefront
        if (c % (D == 256 ? 4 : 8) == 0 && c > 0) asm volatile("" ::: "memory");
        // chunk 2c + h of row 32 j + m: its low 3 bits are swizzled, the rest
        // is a constant offset
        const uint4 wv = *reinterpret_cast<const uint4 *>(wrow + woff[c % 4] + (c / 4) * 8 * AV);
        acc = M::mma(wv, a[c], acc);
      }
      if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float x[4] = {acc[4 * gq], acc[4 * gq + 1], acc[4 * gq + 2], acc[4 * gq + 3]};
          if constexpr (RESID) O::add(x, rv[j][gq]);
          O::store(rc, ooff + (32 * j + 8 * gq) * (int)sizeof(T), x);
        }
      } else {
        // bf16: pack each group of four, then lanes l and l ^ 32 trade one
        // group per pair so that each writes eight adjacent columns (16 B):
        // lane half 0 columns 16 p .. 16 p + 7, half 1 the next eight
        uint2 pk[4];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float x[4] = {acc[4 * gq], acc[4 * gq + 1], acc[4 * gq + 2], acc[4 * gq + 3]};
          if constexpr (RESID) O::add(x, rv[j][gq]);
          pk[gq] = make_uint2(bf16_rne(x[0]) | (bf16_rne(x[1]) << 16),
                              bf16_rne(x[2]) | (bf16_rne(x[3]) << 16));
        }
        uint4 v[2];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const uint2 mine = h ? pk[2 * pp + 1] : pk[2 * pp];
          const uint2 give = h ? pk[2 * pp] : pk[2 * pp + 1];
          const uint2 got = make_uint2((uint32_t)__shfl_xor((int)give.x, 32),
                                       (uint32_t)__shfl_xor((int)give.y, 32));
          v[pp] = h ? make_uint4(got.x, got.y, mine.x, mine.y)
                    : make_uint4(mine.x, mine.y, got.x, got.y);
        }
        // a 32-column block is half of a row's 128-byte line: hold an even
        // block until its odd neighbour is done and write the two together,
        // so no line leaves L2 half written
        if (j % 2 == 0) {
          held[0] = v[0];
          held[1] = v[1];
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int jj = j - 1 + k / 2, pp = k % 2;
            const uint4 x = k / 2 ? v[pp] : held[pp];
            const int o = (lane % 32) * RB + (32 * jj + 16 * pp + 8 * h) * 2;
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(rc, 0, 0, 0)), x),
                rc, o, 0, 0);
          }
        }
      }
    }
  };
  uint4 a0[CH], a1[CH];
  load_strip(a0, q0);
  for (int64_t q = q0; q < strips; q += 2 * stride) {
    run_strip(a0, a1, q);
    if (q + stride >= strips) break;
    run_strip(a1, a0, q + stride);
  }
}

// ---------------------------------------------------------------------------
// One-source row GEMM without a residual for bf16 at D = 128 and 256 (the
// Q/K/V projections): the resident kernel above with the node strips and the
// results staged through LDS.
//
// In the operand layout a 16-byte load or store instruction touches 32 rows
// x 32 bytes, i.e. 32 cache lines.  Here a wavefront loads its 32-row strip
// as contiguous 16-byte chunks (an instruction covers 8 rows x 128 bytes, or
// 4 rows x 256 bytes: 8 whole lines), writes them into its own LDS slice and
// reads them back in the operand layout; the results of a pair of 32-column
// blocks go out the same way (packed to bf16 into the slice, then 8 rows x
// 128 bytes per store).  What LDS the resident weights leave (160 KB in all)
// is split among the 8 wavefronts; where a slice holds less than a strip
// (D = 256: 4 KB, a quarter of the strip's k range), the strip is staged in
// k phases and every 32-column block's accumulator stays live across them.
// The global data of a phase is loaded two phases ahead, into two register
// sets used in turn.  Chunks sit in the slice XOR-swizzled by row, so the
// operand reads (32 rows, one chunk each) and the staging writes spread over
// the banks.  LDS operations of one wavefront complete in order; a wait on
// the LDS counter separates a slice's writes from the reads of other lanes.
// ---------------------------------------------------------------------------
template <int D, int NZ> struct Staged {
  static constexpr int RB = 2 * D;                                   // bytes per node row
  static constexpr int WB = NZ * D * D * 2;                          // resident weights
  static constexpr int SLICE = (160 * 1024 - WB) / RR_WAVES;         // LDS bytes per wavefront
  static constexpr int PB = RB < SLICE / 32 ? RB : SLICE / 32;       // bytes of a row per phase
  static constexpr int P = RB / PB;                                  // phases per strip
  static constexpr int KS = PB / 32;                                 // MFMA k steps per phase
  static constexpr int CPR = PB / 16;                                // chunks of a row per phase
  static constexpr int LPP = 32 * CPR / WAVE;                        // loads per lane per phase
  static_assert(CPR >= 8 && P * PB == RB && SLICE >= 32 * PB && 32 * PB >= 4096, "shape");
};

__device__ inline void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int D, int NZ>
__global__ __launch_bounds__(RR_THREADS) void k_rows_staged(RowsGemm g, int groups) {
  using T = bf16_t;
  using M = Mma<T>;
  using S = Staged<D, NZ>;
  constexpr int AV = 8, RB = S::RB, P = S::P, KS = S::KS, CPR = S::CPR, LPP = S::LPP;
  constexpr int J = D / 32, NACC = P == 1 ? 1 : NZ * J;
  constexpr int UNITS = (D / 2) * (D / AV);
  __shared__ __align__(16) T Ws[NZ * D * D];
  __shared__ __align__(16) uint4 Sl[RR_WAVES][32 * CPR];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), h = lane / 32, m32 = lane % 32;
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int nsplit = NZ == 1 ? g.nout : 1;
  const int b = blockIdx.x, xcd = b % 8, slot = b / 8;
  const int zs = slot % nsplit, group = slot / nsplit;
  // stage W_z: Ws[z][n][k] = W_z[k][n] (the resident kernel's layout)
  for (int zz = 0; zz < NZ; ++zz) {
    const T *W = (const T *)g.B[NZ == 1 ? zs : zz][0];
    T *Wz = Ws + zz * D * D;
    for (int u = tid; u < UNITS; u += RR_THREADS) {
      const int ng = u % (D / AV), kp = u / (D / AV), k0 = 2 * kp;
      const uint4 r0 = *reinterpret_cast<const uint4 *>(W + (int64_t)k0 * D + ng * AV);
      const uint4 r1 = *reinterpret_cast<const uint4 *>(W + (int64_t)(k0 + 1) * D + ng * AV);
      int off[AV];
#pragma unroll
      for (int c = 0; c < AV; ++c) {
        const int nn = ng * AV + c;
        off[c] = nn * D + (((k0 / AV) ^ rsw(nn)) * AV) + k0 % AV;
      }
      store_pair_t<T>(Wz, r0, r1, off);
    }
  }
  __syncthreads();
  uint4 *sl = Sl[w];
  const int64_t strips = (g.n + 31) / 32;
  const int64_t stride = (int64_t)8 * groups * RR_WAVES;
  const int64_t q0 = ((int64_t)group * 8 + xcd) * RR_WAVES + w;
  const T *A = (const T *)g.A[0];
  int woff[4];                                     // lane's weight chunks
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) woff[c4] = m32 * D + (((2 * c4 + h) ^ rsw(m32)) * AV);

  // phase t of this wavefront: strip q0 + (t / P) stride, k phase t % P
  auto load_phase = [&](uint4 (&dst)[LPP], int64_t t) {
    const int64_t q = q0 + (t / P) * stride;
    const int p = (int)(t % P);
    const auto ra = strip_rsrc(A, 32 * q, g.n, RB);   // rows past n (or past the strips) read 0
#pragma unroll
    for (int i = 0; i < LPP; ++i) {
      const int u = i * WAVE + lane, r = u / CPR, c = u % CPR;
      dst[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, r * RB + p * S::PB + c * 16, 0, 0));
    }
  };
  auto put_phase = [&](const uint4 (&src)[LPP]) {
#pragma unroll
    for (int i = 0; i < LPP; ++i) {
      const int u = i * WAVE + lane, r = u / CPR, c = u % CPR;
      sl[r * CPR + (c ^ (r & 7))] = src[i];
    }
  };
  // the bf16 results of the block pair (j0, j0 + 1) of output z for strip q
  auto out_pair = [&](int64_t q, int z, int j0, const v16f &a0, const v16f &a1) {
    uint2 *s2 = reinterpret_cast<uint2 *>(sl);
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const v16f &a = bj ? a1 : a0;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int ch = 4 * bj + gq;              // 16-byte chunk of the 128-byte row
        s2[2 * (m32 * 8 + (ch ^ (m32 & 7))) + h] =
            make_uint2(bf16_rne(a[4 * gq]) | (bf16_rne(a[4 * gq + 1]) << 16),
                       bf16_rne(a[4 * gq + 2]) | (bf16_rne(a[4 * gq + 3]) << 16));
      }
    }
    lds_fence();
    const auto rc = strip_rsrc(g.C[z], 32 * q, g.n, RB);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = i * WAVE + lane, r = u / 8, c = u % 8;
      const uint4 v = sl[r * 8 + (c ^ (r & 7))];
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(rc, 0, 0, 0)), v), rc,
          r * RB + j0 * 64 + c * 16, 0, 0);
    }
    lds_fence();
  };
  v16f acc[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[k][v] = 0.f;
  // one phase: stage it, start the loads two phases ahead, multiply
  auto phase = [&](int64_t t, uint4 (&cur)[LPP]) {
    const int64_t q = q0 + (t / P) * stride;
    const int p = (int)(t % P);
    put_phase(cur);
    load_phase(cur, t + 2);
    lds_fence();
    uint4 bv[KS];
#pragma unroll
    for (int c = 0; c < KS; ++c) bv[c] = sl[m32 * CPR + ((2 * c + h) ^ (m32 & 7))];
    lds_fence();
    if constexpr (P == 1) {
#pragma unroll
      for (int zz = 0; zz < NZ; ++zz) {
        v16f held;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          asm volatile("" ::: "memory");
          v16f a;
#pragma unroll
          for (int v = 0; v < 16; ++v) a[v] = 0.f;
          const T *wrow = Ws + (zz * D + 32 * j) * D;
#pragma unroll
          for (int c = 0; c < KS; ++c) {
            if (c % 8 == 0 && c > 0) asm volatile("" ::: "memory");
            const uint4 wv = *reinterpret_cast<const uint4 *>(wrow + woff[c % 4] + (c / 4) * 8 * AV);
            a = M::mma(wv, bv[c], a);
          }
          if (j % 2 == 0) held = a;
          else out_pair(q, NZ == 1 ? zs : zz, j - 1, held, a);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        asm volatile("" ::: "memory");
        const T *wrow = Ws + (32 * j) * D;
#pragma unroll
        for (int c = 0; c < KS; ++c) {
          const int kc = p * KS + c;               // k step within the row
          const uint4 wv = *reinterpret_cast<const uint4 *>(wrow + woff[kc % 4] + (kc / 4) * 8 * AV);
          acc[j] = M::mma(wv, bv[c], acc[j]);
        }
      }
      if (p == P - 1) {
#pragma unroll
        for (int j = 0; j < J; j += 2) {
          out_pair(q, zs, j, acc[j], acc[j + 1]);
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[j][v] = acc[j + 1][v] = 0.f;
        }
      }
    }
  };
  uint4 g0[LPP], g1[LPP];
  load_phase(g0, 0);
  load_phase(g1, 1);
  const int64_t nt = q0 < strips ? ((strips - 1 - q0) / stride + 1) * P : 0;   // phases to run
  for (int64_t t = 0; t < nt; t += 2) {
    phase(t, g0);
    if (t + 1 >= nt) break;
    phase(t + 1, g1);
  }
}

// ---------------------------------------------------------------------------
// The output projection Z = X W_o + Y for bf16 at D = 128 and 256, staged
// like k_rows_staged.  The residual must be added to the float32 products
// before the one rounding to bf16, so the results of a pair of 32-column
// blocks go into the wavefront's slice as float32 (8 KB), come back as
// contiguous runs of a row (an instruction covers 4 rows x 64 columns), have
// the residual added (read the same contiguous way, ahead of time) and leave
// as bf16, 4 whole lines per store.  At D = 256 a workgroup holds one half
// of W_o's columns (NH = 2: 64 KB), so that the slices have room for the
// float32 pair; the two workgroups of a strip sit eight indices apart (same
// XCD), so the strip's second read of X comes from L2.
// ---------------------------------------------------------------------------
template <int D, int NH> struct StagedOut {
  static constexpr int RB = 2 * D;
  static constexpr int DC = D / NH;                                   // output columns held
  static constexpr int WB = DC * D * 2;
  static constexpr int SLICE = (160 * 1024 - WB) / RR_WAVES;
  static constexpr int PB = 32 * RB <= SLICE ? RB : RB / 2;           // bytes of a row per phase
  static constexpr int P = RB / PB;
  static constexpr int KS = PB / 32;
  static constexpr int CPR = PB / 16;
  static constexpr int LPP = 32 * CPR / WAVE;
  static constexpr int J = DC / 32;
  static_assert(SLICE >= 32 * PB && SLICE >= 8192 && J % 2 == 0 && CPR >= 8, "shape");
};

template <int D, int NH>
__global__ __launch_bounds__(RR_THREADS) void k_rows_staged_out(RowsGemm g, int groups) {
  using T = bf16_t;
  using M = Mma<T>;
  using S = StagedOut<D, NH>;
  constexpr int AV = 8, RB = S::RB, P = S::P, KS = S::KS, CPR = S::CPR, LPP = S::LPP;
  constexpr int J = S::J, DC = S::DC, NACC = P == 1 ? 1 : J;
  __shared__ __align__(16) T Ws[DC * D];
  __shared__ __align__(16) uint4 Sl[RR_WAVES][S::SLICE / 16];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), h = lane / 32, m32 = lane % 32;
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int b = blockIdx.x, xcd = b % 8, slot = b / 8;
  const int half = slot % NH, group = slot / NH;
  // stage W_o's columns [half DC, half DC + DC): Ws[n][k] = W_o[k][half DC + n]
  {
    const T *W = (const T *)g.B[0][0];
    constexpr int UNITS = (D / 2) * (DC / AV);
    for (int u = tid; u < UNITS; u += RR_THREADS) {
      const int ng = u % (DC / AV), kp = u / (DC / AV), k0 = 2 * kp;
      const int col = half * DC + ng * AV;
      const uint4 r0 = *reinterpret_cast<const uint4 *>(W + (int64_t)k0 * D + col);
      const uint4 r1 = *reinterpret_cast<const uint4 *>(W + (int64_t)(k0 + 1) * D + col);
      int off[AV];
#pragma unroll
      for (int c = 0; c < AV; ++c) {
        const int nn = ng * AV + c;
        off[c] = nn * D + (((k0 / AV) ^ rsw(nn)) * AV) + k0 % AV;
      }
      store_pair_t<T>(Ws, r0, r1, off);
    }
  }
  __syncthreads();
  uint4 *sl = Sl[w];
  const int64_t strips = (g.n + 31) / 32;
  const int64_t stride = (int64_t)8 * groups * RR_WAVES;
  const int64_t q0 = ((int64_t)group * 8 + xcd) * RR_WAVES + w;
  const T *A = (const T *)g.A[0];
  int woff[4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) woff[c4] = m32 * D + (((2 * c4 + h) ^ rsw(m32)) * AV);

  auto load_phase = [&](uint4 (&dst)[LPP], int64_t t) {
    const int64_t q = q0 + (t / P) * stride;
    const int p = (int)(t % P);
    const auto ra = strip_rsrc(A, 32 * q, g.n, RB);
#pragma unroll
    for (int i = 0; i < LPP; ++i) {
      const int u = i * WAVE + lane, r = u / CPR, c = u % CPR;
      dst[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, r * RB + p * S::PB + c * 16, 0, 0));
    }
  };
  auto put_phase = [&](const uint4 (&src)[LPP]) {
#pragma unroll
    for (int i = 0; i < LPP; ++i) {
      const int u = i * WAVE + lane, r = u / CPR, c = u % CPR;
      sl[r * CPR + (c ^ (r & 7))] = src[i];
    }
  };
  // residual of the pair of blocks (jp, jp + 1) (local indices), in the
  // read-back layout: run i of a lane is row (i 64 + lane) / 16, columns
  // 4 ((i 64 + lane) % 16) .. + 3 of the pair
  uint2 rres[J / 2][8];
  auto load_resid = [&](int64_t q, int pr) {
    const auto rr = strip_rsrc(g.R, 32 * q, g.n, RB);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = i * WAVE + lane, r = u / 16, c = u % 16;
      rres[pr][i] = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(rr, r * RB + (half * DC + 64 * pr + 4 * c) * 2, 0, 0));
    }
  };
  // Z of the block pair pr: the float32 products through the slice (row m32,
  // 16 chunks of four floats), the residual added, bf16 out
  auto out_pair = [&](int64_t q, int pr, const v16f &a0, const v16f &a1) {
    float4 *s4 = reinterpret_cast<float4 *>(sl);
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const v16f &a = bj ? a1 : a0;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int ch = 8 * bj + 2 * gq + h;     // four columns 32 bj + 8 gq + 4 h ..
        s4[m32 * 16 + (ch ^ (m32 & 7))] = make_float4(a[4 * gq], a[4 * gq + 1], a[4 * gq + 2], a[4 * gq + 3]);
      }
    }
    lds_fence();
    const auto rc = strip_rsrc(g.C[0], 32 * q, g.n, RB);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = i * WAVE + lane, r = u / 16, c = u % 16;
      const float4 x = s4[r * 16 + (c ^ (r & 7))];
      const uint2 y = rres[pr][i];
      const float z0 = x.x + __uint_as_float(y.x << 16), z1 = x.y + __uint_as_float(y.x & 0xffff0000u);
      const float z2 = x.z + __uint_as_float(y.y << 16), z3 = x.w + __uint_as_float(y.y & 0xffff0000u);
      const uint2 v = make_uint2(bf16_rne(z0) | (bf16_rne(z1) << 16), bf16_rne(z2) | (bf16_rne(z3) << 16));
      __builtin_amdgcn_raw_buffer_store_b64(
          __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b64(rc, 0, 0, 0)), v), rc,
          r * RB + (half * DC + 64 * pr + 4 * c) * 2, 0, 0);
    }
    lds_fence();
  };
  v16f acc[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[k][v] = 0.f;
  auto phase = [&](int64_t t, uint4 (&cur)[LPP]) {
    const int64_t q = q0 + (t / P) * stride;
    const int p = (int)(t % P);
    put_phase(cur);
    // the strip's residual, in its first phase and ahead of the prefetch, so
    // that waiting for it (the memory counter is in order) leaves the
    // prefetch in flight
    if (p == 0) {
#pragma unroll
      for (int pr = 0; pr < J / 2; ++pr) load_resid(q, pr);
    }
    load_phase(cur, t + 2);
    lds_fence();
    uint4 bv[KS];
#pragma unroll
    for (int c = 0; c < KS; ++c) bv[c] = sl[m32 * CPR + ((2 * c + h) ^ (m32 & 7))];
    lds_fence();
    if constexpr (P == 1) {
      v16f held;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        asm volatile("" ::: "memory");
        v16f a;
#pragma unroll
        for (int v = 0; v < 16; ++v) a[v] = 0.f;
        const T *wrow = Ws + (32 * j) * D;
#pragma unroll
        for (int c = 0; c < KS; ++c) {
          if (c % 8 == 0 && c > 0) asm volatile("" ::: "memory");
          const uint4 wv = *reinterpret_cast<const uint4 *>(wrow + woff[c % 4] + (c / 4) * 8 * AV);
          a = M::mma(wv, bv[c], a);
        }
        if (j % 2 == 0) held = a;
        else out_pair(q, j / 2, held, a);
      }
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        asm volatile("" ::: "memory");
        const T *wrow = Ws + (32 * j) * D;
#pragma unroll
        for (int c = 0; c < KS; ++c) {
          const int kc = p * KS + c;
          const uint4 wv = *reinterpret_cast<const uint4 *>(wrow + woff[kc % 4] + (kc / 4) * 8 * AV);
          acc[j] = M::mma(wv, bv[c], acc[j]);
        }
      }
      if (p == P - 1) {
#pragma unroll
        for (int j = 0; j < J; j += 2) {
          out_pair(q, j / 2, acc[j], acc[j + 1]);
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[j][v] = acc[j + 1][v] = 0.f;
        }
      }
    }
  };
  uint4 g0[LPP], g1[LPP];
  load_phase(g0, 0);
  load_phase(g1, 1);
  const int64_t nt = q0 < strips ? ((strips - 1 - q0) / stride + 1) * P : 0;
  for (int64_t t = 0; t < nt; t += 2) {
    phase(t, g0);
    if (t + 1 >= nt) break;
    phase(t + 1, g1);
  }
}

// ---------------------------------------------------------------------------
// four-source row GEMM (the input gradient): C = sum_s A_s W_s^T (fp32 at
// D = 64 and 128, bf16 at D = 64; bf16 at D = 128 and 256 takes the staged
// variant below, fp32 at D = 256 the column-tiled kernel).
//
// Each wavefront owns a 32-row strip and keeps the whole [32, D] result in
// registers (J accumulator blocks) while the k dimension streams through in
// slabs of NCS 16-byte chunks: for each source s and slab, the workgroup
// stages rows n of W_s restricted to the slab's k (contiguous in W_s, since
// B_s = W_s^T) into LDS, double-buffered with one barrier per slab, and each
// wavefront multiplies its strip's chunks of A_s by them.  A chunk of the
// strip is dead once its slab is done, so its register is refilled at once
// with the same chunk of the next source (or of the next strip's first
// source): the A loads run one source ahead without extra registers, and
// they are issued before the strip's stores, so waiting for them never waits
// for a store (the memory counter is in order).  Workgroups are persistent
// over 256-row strips; all global accesses go through bounded buffer
// resources (no branches at the ragged end).
// ---------------------------------------------------------------------------
constexpr int S4_WAVES = 8, S4_THREADS = S4_WAVES * WAVE;
constexpr int S4_ROWS = S4_WAVES * 32;
constexpr int S4_NCS = 2;                          // 16-byte chunks (k) per slab
constexpr int S4_PITCH = S4_NCS * 32 + 16;         // LDS bytes per weight row of a slab

// the four outputs of block j of a lane (row lane % 32), as stored
template <typename T>
__device__ inline void store_strip_block(__amdgpu_buffer_rsrc_t rc, int RB, int j, int lane,
                                         const v16f &acc) {
  const int h = lane / 32, m = lane % 32;
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const uint4 v = make_uint4(__float_as_uint(acc[4 * gq]), __float_as_uint(acc[4 * gq + 1]),
                                 __float_as_uint(acc[4 * gq + 2]), __float_as_uint(acc[4 * gq + 3]));
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(rc, 0, 0, 0)), v), rc,
          m * RB + (32 * j + 8 * gq + 4 * h) * 4, 0, 0);
    }
  } else {
    uint2 pk[4];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
      pk[gq] = make_uint2(bf16_rne(acc[4 * gq]) | (bf16_rne(acc[4 * gq + 1]) << 16),
                          bf16_rne(acc[4 * gq + 2]) | (bf16_rne(acc[4 * gq + 3]) << 16));
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const uint2 mine = h ? pk[2 * pp + 1] : pk[2 * pp];
      const uint2 give = h ? pk[2 * pp] : pk[2 * pp + 1];
      const uint2 got = make_uint2((uint32_t)__shfl_xor((int)give.x, 32),
                                   (uint32_t)__shfl_xor((int)give.y, 32));
      const uint4 v = h ? make_uint4(got.x, got.y, mine.x, mine.y)
                        : make_uint4(mine.x, mine.y, got.x, got.y);
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(rc, 0, 0, 0)), v), rc,
          m * RB + (32 * j + 16 * pp + 8 * h) * 2, 0, 0);
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(S4_THREADS) void k_rows_sum4(RowsGemm g) {
  using M = Mma<T>;
  constexpr int AV = 16 / sizeof(T), CH = D / (2 * AV), RB = D * (int)sizeof(T);
  constexpr int JW = D / 32;                              // column blocks
  static_assert(D <= 128 || sizeof(T) == 2, "a strip and its result must fit one wavefront's registers");
  constexpr int NSLAB = CH / S4_NCS;                      // slabs per source
  constexpr int SV = D * 2 * S4_NCS;                      // 16-byte vectors per slab
  constexpr int SU = (SV + S4_THREADS - 1) / S4_THREADS;  // per thread
  static_assert(CH % S4_NCS == 0 && NSLAB % 2 == 0, "slab parity");
  __shared__ __align__(16) char Bs[2][D * S4_PITCH];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), h = lane / 32;
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int64_t nblk = (g.n + S4_ROWS - 1) / S4_ROWS;
  const int64_t first = blockIdx.x, stride = gridDim.x;
  const int aoff = (lane % 32) * RB + h * 16;

  // weight slab (source s, slab c0): row n, vectors 0 .. 2 NCS - 1
  uint4 sv[SU];
  // a lane's byte offset in W_s of its staging vectors (the slab adds a
  // uniform offset); buffer loads keep the per-source bases in scalars
  int woff[SU];
#pragma unroll
  for (int i = 0; i < SU; ++i) {
    const int u = (tid + i * S4_THREADS) % SV;       // every thread loads (duplicates unused)
    woff[i] = (u / (2 * S4_NCS)) * RB + (u % (2 * S4_NCS)) * 16;
  }
  auto fetch_w = [&](int s, int slab) {
    const auto rw = __builtin_amdgcn_make_buffer_rsrc((void *)g.B[0][s], 0, D * RB, BUF_WORD3);
#pragma unroll
    for (int i = 0; i < SU; ++i)
      sv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[i], slab * S4_NCS * 32, 0));
  };
  auto put_w = [&](char *buf) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = tid + i * S4_THREADS;
      if (u < SV) {
        const int n = u / (2 * S4_NCS), v = u % (2 * S4_NCS);
        *reinterpret_cast<uint4 *>(buf + n * S4_PITCH + v * 16) = sv[i];
      }
    }
  };
  auto strip_of = [&](int64_t blk) { return (blk * S4_WAVES + w) * 32; };   // first row

  uint4 a[CH];
  {
    const auto ra = strip_rsrc(g.A[0], strip_of(first), g.n, RB);
#pragma unroll
    for (int c = 0; c < CH; ++c)
      a[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, aoff + 32 * c, 0, 0));
  }
  fetch_w(0, 0);
  put_w(Bs[0]);
  for (int64_t blk = first; blk < nblk; blk += stride) {
    const int64_t row0 = strip_of(blk);
    v16f acc[JW];
#pragma unroll
    for (int j = 0; j < JW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // where the chunks freed in this source go: the next source of this
      // strip, or the first source of the next strip
      const auto rn = s < 3 ? strip_rsrc(g.A[s + 1], row0, g.n, RB)
                            : strip_rsrc(g.A[0], strip_of(blk + stride), g.n, RB);
#pragma unroll
      for (int slab = 0; slab < NSLAB; ++slab) {
        __syncthreads();                       // Bs[slab & 1] is complete
        // the next slab's weights (the first slab of source 0 after the last)
        if (slab + 1 < NSLAB) fetch_w(s, slab + 1);
        else fetch_w(s < 3 ? s + 1 : 0, 0);
        const char *buf = Bs[slab & 1];
#pragma unroll
        for (int cc = 0; cc < S4_NCS; ++cc) {
          const int c = slab * S4_NCS + cc;
          asm volatile("" ::: "memory");       // one chunk's weight reads at a time
#pragma unroll
          for (int j = 0; j < JW; ++j) {
            const uint4 wv = *reinterpret_cast<const uint4 *>(
                buf + (32 * j + lane % 32) * S4_PITCH + (2 * cc + h) * 16);
            acc[j] = M::mma(wv, a[c], acc[j]);
          }
          a[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rn, aoff + 32 * c, 0, 0));
        }
        put_w(Bs[(slab + 1) & 1]);
      }
    }
    const auto rc = strip_rsrc(g.C[0], row0, g.n, RB);
#pragma unroll
    for (int j = 0; j < JW; ++j) store_strip_block<T>(rc, RB, j, lane, acc[j]);
  }
}

// ---------------------------------------------------------------------------
// The input gradient for bf16 at D = 128 and 256: k_rows_sum4 with the
// source strips and the results staged through LDS, as in k_rows_staged.
// Each wavefront owns an 8 KB slice beside the weight slabs.  A source strip
// comes in as contiguous 16-byte chunks (an instruction covers 4 rows x 256
// bytes) in phases of 256 bytes of a row (one at D = 128, two at D = 256),
// the next phase's loads in flight while this one is multiplied; the slice
// hands the phase back in the operand layout.  The weight slabs stream
// through LDS exactly as in k_rows_sum4 (double-buffered, one barrier a
// slab), so the products and their order are the same.  Results leave
// through the slice a pair of 32-column blocks at a time, 8 rows x 128
// bytes per store.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(S4_THREADS) void k_rows_sum4_staged(RowsGemm g) {
  using T = bf16_t;
  using M = Mma<T>;
  constexpr int CH = D / 16, RB = 2 * D, JW = D / 32;
  constexpr int PB = RB < 256 ? RB : 256;                 // bytes of a row per phase
  constexpr int P = RB / PB;                              // phases per source
  constexpr int CPP = PB / 32;                            // operand chunks per phase
  constexpr int CPR = PB / 16;                            // 16-byte chunks of a row per phase
  constexpr int LPP = 32 * CPR / WAVE;                    // loads per lane per phase
  constexpr int NSLAB = CH / S4_NCS, SPP = CPP / S4_NCS;  // weight slabs per source, per phase
  constexpr int SV = D * 2 * S4_NCS;
  constexpr int SU = (SV + S4_THREADS - 1) / S4_THREADS;
  static_assert(CPP % S4_NCS == 0 && NSLAB % 2 == 0 && P * CPP == CH && 32 * CPR * 16 >= 4096, "shape");
  __shared__ __align__(16) char Bs[2][D * S4_PITCH];
  __shared__ __align__(16) uint4 Sl[S4_WAVES][32 * CPR];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), h = lane / 32, m32 = lane % 32;
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int64_t nblk = (g.n + S4_ROWS - 1) / S4_ROWS;
  const int64_t first = blockIdx.x, stride = gridDim.x;
  uint4 *sl = Sl[w];

  uint4 sv[SU];
  int woff[SU];
#pragma unroll
  for (int i = 0; i < SU; ++i) {
    const int u = (tid + i * S4_THREADS) % SV;
    woff[i] = (u / (2 * S4_NCS)) * RB + (u % (2 * S4_NCS)) * 16;
  }
  auto fetch_w = [&](int s, int slab) {
    const auto rw = __builtin_amdgcn_make_buffer_rsrc((void *)g.B[0][s], 0, D * RB, BUF_WORD3);
#pragma unroll
    for (int i = 0; i < SU; ++i)
      sv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[i], slab * S4_NCS * 32, 0));
  };
  auto put_w = [&](char *buf) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = tid + i * S4_THREADS;
      if (u < SV) {
        const int n = u / (2 * S4_NCS), v = u % (2 * S4_NCS);
        *reinterpret_cast<uint4 *>(buf + n * S4_PITCH + v * 16) = sv[i];
      }
    }
  };
  auto strip_of = [&](int64_t blk) { return (blk * S4_WAVES + w) * 32; };   // first row
  // phase ph of source s of the strip at row0 (rows past n read 0)
  auto load_phase = [&](uint4 (&dst)[LPP], int s, int64_t row0, int ph) {
    const auto ra = strip_rsrc(g.A[s], row0, g.n, RB);
#pragma unroll
    for (int i = 0; i < LPP; ++i) {
      const int u = i * WAVE + lane, r = u / CPR, c = u % CPR;
      dst[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, r * RB + ph * PB + c * 16, 0, 0));
    }
  };
  // the bf16 results of the block pair (j0, j0 + 1) for the strip at row0
  auto out_pair = [&](int64_t row0, int j0, const v16f &a0, const v16f &a1) {
    uint2 *s2 = reinterpret_cast<uint2 *>(sl);
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const v16f &a = bj ? a1 : a0;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int ch = 4 * bj + gq;
        s2[2 * (m32 * 8 + (ch ^ (m32 & 7))) + h] =
            make_uint2(bf16_rne(a[4 * gq]) | (bf16_rne(a[4 * gq + 1]) << 16),
                       bf16_rne(a[4 * gq + 2]) | (bf16_rne(a[4 * gq + 3]) << 16));
      }
    }
    lds_fence();
    const auto rc = strip_rsrc(g.C[0], row0, g.n, RB);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = i * WAVE + lane, r = u / 8, c = u % 8;
      const uint4 v = sl[r * 8 + (c ^ (r & 7))];
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(rc, 0, 0, 0)), v), rc,
          r * RB + j0 * 64 + c * 16, 0, 0);
    }
    lds_fence();
  };

  uint4 gl[LPP];
  load_phase(gl, 0, strip_of(first), 0);
  fetch_w(0, 0);
  put_w(Bs[0]);
  for (int64_t blk = first; blk < nblk; blk += stride) {
    const int64_t row0 = strip_of(blk);
    v16f acc[JW];
#pragma unroll
    for (int j = 0; j < JW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int ph = 0; ph < P; ++ph) {
        // stage this phase, start the next one's loads, read it back (a
        // second register set, two phases ahead, spills at D = 256 and
        // made no measurable difference at D = 128)
#pragma unroll
        for (int i = 0; i < LPP; ++i) {
          const int u = i * WAVE + lane, r = u / CPR, c = u % CPR;
          sl[r * CPR + (c ^ (r & 7))] = gl[i];
        }
        if (ph + 1 < P) load_phase(gl, s, row0, ph + 1);
        else if (s < 3) load_phase(gl, s + 1, row0, 0);
        else load_phase(gl, 0, strip_of(blk + stride), 0);
        lds_fence();
        uint4 a[CPP];
#pragma unroll
        for (int c = 0; c < CPP; ++c) a[c] = sl[m32 * CPR + ((2 * c + h) ^ (m32 & 7))];
        lds_fence();
#pragma unroll
        for (int sp = 0; sp < SPP; ++sp) {
          const int slab = ph * SPP + sp;      // slab of this source
          __syncthreads();                     // Bs[slab & 1] is complete
          if (slab + 1 < NSLAB) fetch_w(s, slab + 1);
          else fetch_w(s < 3 ? s + 1 : 0, 0);
          const char *buf = Bs[slab & 1];
#pragma unroll
          for (int cc = 0; cc < S4_NCS; ++cc) {
            asm volatile("" ::: "memory");     // one chunk's weight reads at a time
#pragma unroll
            for (int j = 0; j < JW; ++j) {
              const uint4 wv = *reinterpret_cast<const uint4 *>(
                  buf + (32 * j + m32) * S4_PITCH + (2 * cc + h) * 16);
              acc[j] = M::mma(wv, a[sp * S4_NCS + cc], acc[j]);
            }
          }
          put_w(Bs[(slab + 1) & 1]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < JW; j += 2) out_pair(row0, j, acc[j], acc[j + 1]);
  }
}

// ---------------------------------------------------------------------------
// weight gradient: dW_s = X^T G_s, a contraction over the n node rows.
// The rows are cut into `slots` contiguous ranges; workgroup (s, slot)
// computes the whole [D, D] product of its range for gradient s into
// part[s][slot], and a second kernel sums the slots in slot order
// (deterministic, no atomics).  Per step a workgroup stages KT = 32 rows
// of X and G_s into LDS transposed to [column][row] (two rows per thread,
// swapped into column pairs in registers), the rows of the next PD steps
// already in flight, and its wavefronts each multiply a (32 MB) x (32 NB)
// block.
// Workgroups of one slot sit eight block indices apart, so the four that
// share X rows land on the same XCD (and L2).
// ---------------------------------------------------------------------------
struct WgradGemm {
  const void *X;
  const void *G[4];
  float *part;       // [grads][slots][d][d]
  float *dW[4];
  int64_t n, rows_per_slot;
  int slots, d, ngrad;
};

constexpr int WG_KT = 32;

template <int D> struct WgradShape;
template <> struct WgradShape<64> { static constexpr int WM = 2, WN = 2, MB = 1, NB = 1; };
template <> struct WgradShape<128> { static constexpr int WM = 4, WN = 2, MB = 1, NB = 2; };
template <> struct WgradShape<256> { static constexpr int WM = 4, WN = 2, MB = 2, NB = 4; };

// swizzled [column][KT] tile: column m, chunk q -> element offset
template <typename T>
__device__ inline int wtile_off(int m, int q) {
  constexpr int AV = 16 / sizeof(T), NCH = WG_KT / AV;           // chunks per row
  constexpr int RS = sizeof(T) == 2 ? 1 : 0;                    // rows per 128 B = 2^RS
  constexpr int LG = NCH == 4 ? 2 : 3;
  return m * WG_KT + ((q ^ (((m >> RS) ^ (m >> (RS + LG))) & (NCH - 1))) * AV);
}

template <typename T, int D>
__global__ __launch_bounds__(WgradShape<D>::WM * WgradShape<D>::WN * WAVE)
void k_gemm_wgrad(WgradGemm g) {
  using M = Mma<T>;
  using S = WgradShape<D>;
  constexpr int NT = S::WM * S::WN * WAVE;
  constexpr int AV = 16 / sizeof(T);
  constexpr int CH = WG_KT / (2 * AV);          // k ranges per step
  constexpr int UOP = (WG_KT / 2) * (D / AV);   // row-pair units per operand
  constexpr int SU = (2 * UOP + NT - 1) / NT;   // units per thread
  static_assert(UOP % WAVE == 0 && 2 * UOP == SU * NT, "staging units fill the workgroup");
  constexpr int TILE = D * WG_KT;
  __shared__ __align__(16) T Xs[TILE];
  __shared__ __align__(16) T Gs[TILE];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, h = lane / 32;
  const int wm = w % S::WM, wn = w / S::WM;
  const int b = blockIdx.x;
  const int s = (b / 8) % 4, slot = (b % 8) + 8 * (b / 32);
  if (s >= g.ngrad || slot >= g.slots) return;   // grid is exactly slots * 4; kept for safety
  const int64_t r0 = (int64_t)slot * g.rows_per_slot;
  const int64_t r1 = std::min<int64_t>(r0 + g.rows_per_slot, g.n);
  const T *X = (const T *)g.X, *G = (const T *)g.G[s];

  // staging registers of the next PD steps (a ring, indexed statically by
  // unrolling the step loop PD times); rows go through a buffer resource
  // bounded to the step's rows of the slot, so rows past the slot read as 0
  // (bf16 at D = 256, 1M rows: 2 steps 0.79 ms, 3 steps 0.71, 4 steps 0.69,
  // 5 steps 0.65, and 6 do not fit the registers; at D = 128, 2.4M rows, 6
  // or 8 steps were slower than 4)
  constexpr int PD = D == 256 ? (sizeof(T) == 4 ? 1 : 5) : 4;
  constexpr int RB = D * (int)sizeof(T);
  uint4 st[PD][2 * SU];
  // unit u: operand u / UOP, column group mg, row pair kp of the step
  auto unit = [&](int u, int &op, int &mg, int &kp) {
    const int v = u % UOP;
    op = u / UOP;
    const int lo = v % 4, rest = v / 4;
    mg = rest % (D / AV);
    kp = lo + 4 * (rest / (D / AV));
  };
  auto fetch = [&](uint4 (&dst)[2 * SU], int64_t k0) {
    const int64_t nrow = k0 < r1 ? std::min<int64_t>(WG_KT, r1 - k0) : 0;
    const int64_t kb = k0 < r1 ? k0 : 0;
    const auto rx = __builtin_amdgcn_make_buffer_rsrc((void *)(X + kb * D), 0, (int)(nrow * RB), BUF_WORD3);
    const auto rg = __builtin_amdgcn_make_buffer_rsrc((void *)(G + kb * D), 0, (int)(nrow * RB), BUF_WORD3);
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = tid + i * NT;
      int op, mg, kp;
      unit(u, op, mg, kp);
      // UOP is a multiple of 64, so the operand is the same for a whole
      // wavefront: pick its buffer resource in scalar registers
      const auto r = __builtin_amdgcn_readfirstlane(op) == 0 ? rx : rg;
      const int o = 2 * kp * RB + mg * 16;
      dst[2 * i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
      dst[2 * i + 1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o + RB, 0, 0));
    }
  };
  auto put = [&](const uint4 (&src)[2 * SU]) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = tid + i * NT;
      if (u < 2 * UOP) {
        int op, mg, kp;
        unit(u, op, mg, kp);
        const int k = 2 * kp;
        int off[AV];
#pragma unroll
        for (int c = 0; c < AV; ++c) off[c] = wtile_off<T>(mg * AV + c, k / AV) + k % AV;
        store_pair_t<T>(op == 0 ? Xs : Gs, src[2 * i], src[2 * i + 1], off);
      }
    }
  };

  v16f acc[S::MB][S::NB];
#pragma unroll
  for (int i = 0; i < S::MB; ++i)
#pragma unroll
    for (int j = 0; j < S::NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // steps of WG_KT rows, padded to a multiple of PD (the padding steps read
  // zeros and add nothing)
  const int64_t nsteps = r0 < r1 ? (r1 - r0 + WG_KT - 1) / WG_KT : 0;
#pragma unroll
  for (int q = 0; q < PD; ++q) fetch(st[q], r0 + (int64_t)q * WG_KT);
  for (int64_t i0 = 0; i0 < nsteps; i0 += PD) {
#pragma unroll
    for (int q = 0; q < PD; ++q) {
      __syncthreads();
      put(st[q]);
      __syncthreads();
      fetch(st[q], r0 + (i0 + q + PD) * WG_KT);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        uint4 av[S::MB], bv[S::NB];
#pragma unroll
        for (int i = 0; i < S::MB; ++i)
          av[i] = *reinterpret_cast<const uint4 *>(
              Xs + wtile_off<T>(32 * (wm * S::MB + i) + lane % 32, 2 * c + h));
#pragma unroll
        for (int j = 0; j < S::NB; ++j)
          bv[j] = *reinterpret_cast<const uint4 *>(
              Gs + wtile_off<T>(32 * (wn * S::NB + j) + lane % 32, 2 * c + h));
#pragma unroll
        for (int i = 0; i < S::MB; ++i)
#pragma unroll
          for (int j = 0; j < S::NB; ++j) acc[i][j] = M::mma(av[i], bv[j], acc[i][j]);
      }
    }
  }
  float *P = g.part + ((int64_t)s * g.slots + slot) * D * D;
#pragma unroll
  for (int i = 0; i < S::MB; ++i)
#pragma unroll
    for (int j = 0; j < S::NB; ++j) {
      const int col = 32 * (wn * S::NB + j) + lane % 32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 32 * (wm * S::MB + i) + 8 * (v / 4) + 4 * h + v % 4;
        P[(int64_t)row * D + col] = acc[i][j][v];
      }
    }
}

// dW_s[i] = sum over slots, in slot order, of part[s][slot][i]
__global__ void k_wgrad_reduce(WgradGemm g) {
  const int64_t dd = (int64_t)g.d * g.d;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= dd * g.ngrad) return;
  const int s = (int)(t / dd);
  const int64_t i = t % dd;
  const float *p = g.part + (int64_t)s * g.slots * dd + i;
  float x = 0.f;
  for (int c = 0; c < g.slots; ++c) x += p[c * dd];
  g.dW[s][i] = x;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Slots of the weight gradient: a multiple of 8, no more than the 32-row
// steps of n, and at most 64 (one workgroup per CU at d = 256; and float32,
// whose partial products cost as much to sum as the rows they save) or 128
// (bfloat16 below d = 256).  Measured on 131K x 128 float32: 174 us at 64
// slots against 200 at 128; on 2.4M x 128 bfloat16: 651 at 128 against 763
// at 64.  The workspace is sized for the bfloat16 count, the larger one.
int wgrad_slots(int64_t n, int d, gt_dtype dt) {
  const int64_t cap = (d >= 256 || dt == GT_F32) ? 64 : 128;
  const int64_t steps = cdiv(std::max<int64_t>(n, 1), WG_KT);
  return (int)std::min<int64_t>(cap, cdiv(steps, 8) * 8);
}

int64_t wgrad_rows_per_slot(int64_t n, int slots) {
  return cdiv(cdiv(std::max<int64_t>(n, 1), slots), WG_KT) * WG_KT;
}

template <typename T, bool TRANSB, int NA>
static void launch_rows(const RowsGemm &g, dim3 grid, hipStream_t st) {
  k_gemm_rows<T, 256, TRANSB, NA><<<grid, RG_THREADS, 0, st>>>(g);
}

// Workgroups of a kernel that fit on one CU (registers and LDS), and the
// CU count of the current device, from the runtime; each is queried once
// per process (function-local statics initialise thread-safely).
template <typename K>
static int blocks_per_cu(K kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

static int device_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    return n;
  }();
  return cus;
}

template <typename T, int D, bool RESID, int NZ>
static int resident_per_cu() {
  static const int per_cu = blocks_per_cu(k_rows_resident<T, D, RESID, NZ>, RR_THREADS);
  return per_cu;
}

template <typename T, int D, bool RESID, int NZ>
static void launch_resident_k(const RowsGemm &g, hipStream_t st) {
  // workgroups per (XCD, output split): fill the CUs of the XCD (eight
  // XCDs), but no more than the strips need
  const int nsplit = NZ == 1 ? g.nout : 1;
  const int64_t strips = cdiv(g.n, 32);
  const int64_t cus_per_xcd = std::max(1, device_cus() / 8);
  int64_t groups = std::max<int64_t>(1, (int64_t)resident_per_cu<T, D, RESID, NZ>() * cus_per_xcd / nsplit);
  groups = std::max<int64_t>(1, std::min<int64_t>(groups, cdiv(strips, 8 * RR_WAVES)));
  const dim3 grid((unsigned)(8 * groups * nsplit));
  k_rows_resident<T, D, RESID, NZ><<<grid, RR_THREADS, 0, st>>>(g, (int)groups);
}

template <int D, int NH>
static void launch_staged_out(const RowsGemm &g, hipStream_t st) {
  static const int per_cu = blocks_per_cu(k_rows_staged_out<D, NH>, RR_THREADS);
  const int64_t strips = cdiv(g.n, 32);
  const int64_t cus_per_xcd = std::max(1, device_cus() / 8);
  int64_t groups = std::max<int64_t>(1, (int64_t)per_cu * cus_per_xcd / NH);
  groups = std::max<int64_t>(1, std::min<int64_t>(groups, cdiv(strips, 8 * RR_WAVES)));
  const dim3 grid((unsigned)(8 * groups * NH));
  k_rows_staged_out<D, NH><<<grid, RR_THREADS, 0, st>>>(g, (int)groups);
}

template <int D, int NZ>
static void launch_staged_k(const RowsGemm &g, hipStream_t st) {
  static const int per_cu = blocks_per_cu(k_rows_staged<D, NZ>, RR_THREADS);
  const int nsplit = NZ == 1 ? g.nout : 1;
  const int64_t strips = cdiv(g.n, 32);
  const int64_t cus_per_xcd = std::max(1, device_cus() / 8);
  int64_t groups = std::max<int64_t>(1, (int64_t)per_cu * cus_per_xcd / nsplit);
  groups = std::max<int64_t>(1, std::min<int64_t>(groups, cdiv(strips, 8 * RR_WAVES)));
  const dim3 grid((unsigned)(8 * groups * nsplit));
  k_rows_staged<D, NZ><<<grid, RR_THREADS, 0, st>>>(g, (int)groups);
}

// all three Q/K/V weights stay in LDS together where they fit (128 KB), so
// each strip of X is read once; otherwise workgroups split the outputs.
// bf16 at D = 128 and 256 stages its strips through LDS (the output
// projection with its residual in k_rows_staged_out).
template <typename T, int D>
static void launch_resident(const RowsGemm &g, hipStream_t st) {
  constexpr bool three_fit = 3 * D * D * (int)sizeof(T) <= 128 * 1024;
  constexpr bool staged = sizeof(T) == 2 && (D == 128 || D == 256);
  if constexpr (staged) {
    if (g.R) launch_staged_out<D, D == 256 ? 2 : 1>(g, st);
    else if (g.nout == 3 && three_fit) launch_staged_k<D, three_fit ? 3 : 1>(g, st);
    else launch_staged_k<D, 1>(g, st);
  } else {
    if (g.R) launch_resident_k<T, D, true, 1>(g, st);
    else if (g.nout == 3 && three_fit) launch_resident_k<T, D, false, three_fit ? 3 : 1>(g, st);
    else launch_resident_k<T, D, false, 1>(g, st);
  }
}

// transb = false: one source (NA = 1); transb = true: four (NA = 4)
template <typename T, int D>
static void launch_sum4(const RowsGemm &g, hipStream_t st) {
  const int64_t nblk = cdiv(g.n, S4_ROWS);
  if constexpr (sizeof(T) == 2 && (D == 128 || D == 256)) {
    static const int per_cu = blocks_per_cu(k_rows_sum4_staged<D>, S4_THREADS);
    const int64_t grid = std::min<int64_t>(nblk, (int64_t)per_cu * device_cus());
    k_rows_sum4_staged<D><<<dim3((unsigned)grid), S4_THREADS, 0, st>>>(g);
  } else {
    static const int per_cu = blocks_per_cu(k_rows_sum4<T, D>, S4_THREADS);
    const int64_t grid = std::min<int64_t>(nblk, (int64_t)per_cu * device_cus());
    k_rows_sum4<T, D><<<dim3((unsigned)grid), S4_THREADS, 0, st>>>(g);
  }
}

gt_status launch_rows_gemm(gt_dtype dt, RowsGemm g, int nout, bool transb, hipStream_t st) {
  if (g.n == 0) return GT_OK;
  g.nout = nout;
  if (transb && !(dt == GT_F32 && g.d == 256)) {   // the input gradient: four sources
    // (fp32 at d = 256: a strip and its result do not fit the registers
    // together; that case takes the column-tiled kernel below)
    if (dt == GT_F32) {
      if (g.d == 64) launch_sum4<float, 64>(g, st);
      else launch_sum4<float, 128>(g, st);
    } else {
      if (g.d == 64) launch_sum4<bf16_t, 64>(g, st);
      else if (g.d == 128) launch_sum4<bf16_t, 128>(g, st);
      else launch_sum4<bf16_t, 256>(g, st);
    }
    GT_CHECK_LAUNCH();
    return GT_OK;
  }
  if (!transb && !(dt == GT_F32 && g.d == 256)) {
    if (dt == GT_F32) {
      if (g.d == 64) launch_resident<float, 64>(g, st);
      else launch_resident<float, 128>(g, st);
    } else {
      if (g.d == 64) launch_resident<bf16_t, 64>(g, st);
      else if (g.d == 128) launch_resident<bf16_t, 128>(g, st);
      else launch_resident<bf16_t, 256>(g, st);
    }
    GT_CHECK_LAUNCH();
    return GT_OK;
  }
  // fp32 at d = 256: the column-tiled kernel
  const dim3 grid((unsigned)cdiv(g.n, RG_ROWS));
  if (transb) launch_rows<float, true, 4>(g, grid, st);
  else launch_rows<float, false, 1>(g, grid, st);
  GT_CHECK_LAUNCH();
  return GT_OK;
}

template <typename T>
static gt_status run_wgrad(WgradGemm &g, hipStream_t st) {
  if (g.n > 0) {
    const dim3 grid((unsigned)(g.slots * 4));
    switch (g.d) {
      case 64: k_gemm_wgrad<T, 64><<<grid, 4 * WAVE, 0, st>>>(g); break;
      case 128: k_gemm_wgrad<T, 128><<<grid, 8 * WAVE, 0, st>>>(g); break;
      default: k_gemm_wgrad<T, 256><<<grid, 8 * WAVE, 0, st>>>(g); break;
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
  return (size_t)std::max<int64_t>(4 * (int64_t)wgrad_slots(n, d, GT_BF16) * d * d * 4, 256);
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
  g.slots = n > 0 ? wgrad_slots(n, d, dt) : 0;     // n = 0: the sums are empty, dW = 0
  g.rows_per_slot = n > 0 ? wgrad_rows_per_slot(n, g.slots) : 0;
  g.d = d;
  g.ngrad = 4;
  return launch_wgrad(dt, g, (hipStream_t)stream);
}
