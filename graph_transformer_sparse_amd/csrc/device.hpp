// Device helpers shared by the gfx950 kernels: 16-byte lane vectors of
// float32 / bfloat16 features, cross-lane sums inside a head, exp2.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gt {

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;   // log2(e)
constexpr float LN2 = 0.6931471805599453f;     // ln(2)

struct bf16_t { uint16_t bits; };

// A lane owns one 16-byte slice of a feature row: 4 float32 or 8 bfloat16
// values, widened to float32 in registers.
template <typename T> struct Vec;

template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ static inline void load(const float *p, float (&x)[4]) {
    float4 v = *reinterpret_cast<const float4 *>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  __device__ static inline void store(float *p, const float (&x)[4]) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

// bfloat16 -> float32 is exact (the bf16 bits are the high half).
// float32 -> bfloat16 rounds to nearest, ties to even; NaN stays NaN.
__device__ inline uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ static inline void load(const bf16_t *p, float (&x)[8]) {
    uint4 v = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  __device__ static inline void store(bf16_t *p, const float (&x)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = f32_to_bf16_bits(x[2 * k]) | (f32_to_bf16_bits(x[2 * k + 1]) << 16);
    *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// DPP lane moves inside a row of 16 lanes.
template <int CTRL> __device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;  // lane i <- lane 15-i within 16
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <- lane 7-i within 8

// Sum over each aligned group of L lanes; every lane of the group gets the
// same bits (each step adds a lane's value to its partner's, a commutative
// pair, and after the quad steps the partners of the mirror steps hold
// group-uniform values).
template <int L> __device__ inline float group_sum(float x) {
  static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16 || L == 32 || L == 64, "L");
  if constexpr (L >= 2) x += dpp<DPP_QUAD_XOR1>(x);
  if constexpr (L >= 4) x += dpp<DPP_QUAD_XOR2>(x);
  if constexpr (L >= 8) x += dpp<DPP_HALF_MIRROR>(x);
  if constexpr (L >= 16) x += dpp<DPP_ROW_MIRROR>(x);
  if constexpr (L >= 32) x += __shfl_xor(x, 16);
  if constexpr (L >= 64) x += __shfl_xor(x, 32);
  return x;
}

// The row of CSR edge e (0 <= e < nnz): the last r with indptr[r] <= e,
// which skips empty rows.
__device__ inline int32_t row_of_edge(const int32_t *indptr, int64_t n_rows, int32_t e) {
  int64_t lo = 0, hi = n_rows;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (indptr[mid] <= e) lo = mid;
    else hi = mid;
  }
  return (int32_t)lo;
}

// 2^x on the hardware transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace gt
