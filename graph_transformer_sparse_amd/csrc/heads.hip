// Head repack of graph parallelism with all-to-all ("Scalable and Adaptive
// Parallel Training of Graph Transformer on Large Graphs", Section 3.2 and
// Algorithm 2): [rows, heads, hb] <-> [parts][rows, heads/parts, hb], hb the
// bytes of one head.  Pure data movement, bound by HBM bandwidth.
//
// Each thread moves four vectors (16, 8 or 4 bytes, the widest that the
// chunk size and both pointers allow).  The unpacked side is walked in
// order, so its accesses are fully coalesced; on the packed side the
// vectors of consecutive rows of one part are contiguous too, so a
// wavefront writes (or reads) one run of rows x chunk bytes per part.
#include "device.hpp"
#include "host.hpp"
#include "../../include/gt_heads.h"

namespace gt {

struct HeadRepack {
  const char *src;
  char *dst;
  int64_t rows, total;   // rows; vectors of the unpacked tensor (rows * rv)
  uint32_t rv, cv;       // vectors per row, per part chunk
};

constexpr int HR_THREADS = 256, HR_PER = 4;

template <int VB> struct VecOf;
template <> struct VecOf<4> { typedef uint32_t type; };
template <> struct VecOf<8> { typedef uint2 type; };
template <> struct VecOf<16> { typedef uint4 type; };

// SPLIT: unpacked -> packed; otherwise packed -> unpacked
template <int VB, bool SPLIT>
__global__ __launch_bounds__(HR_THREADS) void k_head_repack(HeadRepack a) {
  typedef typename VecOf<VB>::type V;
  const V *src = reinterpret_cast<const V *>(a.src);
  V *dst = reinterpret_cast<V *>(a.dst);
  const int64_t base = (int64_t)blockIdx.x * (HR_THREADS * HR_PER);
  const int64_t row0 = base / a.rv;
  const uint32_t off0 = (uint32_t)(base - row0 * a.rv);
  V v[HR_PER];
  int64_t flat[HR_PER], packed[HR_PER];
#pragma unroll
  for (int k = 0; k < HR_PER; ++k) {
    const uint32_t local = off0 + threadIdx.x + k * HR_THREADS;
    const int64_t row = row0 + local / a.rv;
    const uint32_t col = local % a.rv, part = col / a.cv, w = col % a.cv;
    flat[k] = base + threadIdx.x + k * HR_THREADS;
    packed[k] = ((int64_t)part * a.rows + row) * a.cv + w;
    if (flat[k] < a.total) v[k] = SPLIT ? src[flat[k]] : src[packed[k]];
  }
#pragma unroll
  for (int k = 0; k < HR_PER; ++k)
    if (flat[k] < a.total) dst[SPLIT ? packed[k] : flat[k]] = v[k];
}

template <bool SPLIT>
static gt_status launch_repack(int64_t rows, int32_t heads, int32_t head_bytes, int32_t parts,
                               const void *src, void *dst, hipStream_t st) {
  const int64_t row_bytes = (int64_t)heads * head_bytes;
  const int64_t chunk = row_bytes / parts;
  const uintptr_t al = (uintptr_t)src | (uintptr_t)dst;
  const int vb = (chunk % 16 == 0 && al % 16 == 0) ? 16 : (chunk % 8 == 0 && al % 8 == 0) ? 8 : 4;
  HeadRepack a;
  a.src = (const char *)src;
  a.dst = (char *)dst;
  a.rows = rows;
  a.rv = (uint32_t)(row_bytes / vb);
  a.cv = (uint32_t)(chunk / vb);
  a.total = rows * a.rv;
  if (a.total == 0) return GT_OK;
  const dim3 grid((unsigned)cdiv(a.total, HR_THREADS * HR_PER));
  switch (vb) {
    case 16: k_head_repack<16, SPLIT><<<grid, HR_THREADS, 0, st>>>(a); break;
    case 8: k_head_repack<8, SPLIT><<<grid, HR_THREADS, 0, st>>>(a); break;
    default: k_head_repack<4, SPLIT><<<grid, HR_THREADS, 0, st>>>(a); break;
  }
  GT_CHECK_LAUNCH();
  return GT_OK;
}

}  // namespace gt

using namespace gt;

namespace {

gt_status check_repack(int64_t rows, int32_t heads, int32_t head_bytes, int32_t parts,
                       const void *src, void *dst) {
  if (parts < 1) return fail(GT_E_ARG, "parts = %d: must be >= 1", parts);
  if (rows < 0) return fail(GT_E_ARG, "rows = %lld is negative", (long long)rows);
  if (heads < 1 || head_bytes < 4 || head_bytes % 4 != 0)
    return fail(GT_E_SHAPE, "heads = %d, head_bytes = %d: need heads >= 1 and head_bytes a "
                "positive multiple of 4", heads, head_bytes);
  if (heads % parts != 0)
    return fail(GT_E_SHAPE, "heads = %d is not divisible by parts = %d", heads, parts);
  if ((int64_t)heads * head_bytes > (int64_t)1 << 30)
    return fail(GT_E_SHAPE, "a row of %d x %d bytes is too long", heads, head_bytes);
  if (rows > 0 && (!src || !dst)) return fail(GT_E_NULL, "src or dst is NULL");
  if ((((uintptr_t)src | (uintptr_t)dst) & 3u) != 0)
    return fail(GT_E_ALIGN, "src and dst must be 4-byte aligned");
  return GT_OK;
}

}  // namespace

extern "C" gt_status gt_head_split(int64_t rows, int32_t heads, int32_t head_bytes, int32_t parts,
                                   const void *src, void *dst, void *stream) {
  clear_error();
  const gt_status s = check_repack(rows, heads, head_bytes, parts, src, dst);
  if (s != GT_OK) return s;
  return launch_repack<true>(rows, heads, head_bytes, parts, src, dst, (hipStream_t)stream);
}

extern "C" gt_status gt_head_merge(int64_t rows, int32_t heads, int32_t head_bytes, int32_t parts,
                                   const void *src, void *dst, void *stream) {
  clear_error();
  const gt_status s = check_repack(rows, heads, head_bytes, parts, src, dst);
  if (s != GT_OK) return s;
  return launch_repack<false>(rows, heads, head_bytes, parts, src, dst, (hipStream_t)stream);
}
