// Graph preparation on the GPU (integer work, once per graph):
//   * a stable CSR transpose (the A^T that the backward's transposed
//     products run on: "Scalable and Adaptive Parallel Training of Graph
//     Transformer on Large Graphs", Section 2.2), built as a stable LSD radix
//     sort of (column, edge id) pairs;
//   * the degree-ordered work schedule over the rows of A and of A^T
//     (load balance by sorting rows by their nonzero count, as the
//     engineering blog page restating the method advises in its section on
//     sparse kernels), also a stable radix sort, on (max_degree - degree);
//   * the debug CSR validator.
// Every result is an integer array that is unique by definition (stable
// sorts, order-independent counts), so it is reproducible bit for bit.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include <vector>

#include "device.hpp"
#include "host.hpp"
#include "layout.hpp"

namespace gt {

// ---------------------------------------------------------------------------
// exclusive prefix sum of uint32 (reduce, scan the block sums, down-sweep)
// ---------------------------------------------------------------------------
constexpr int SCAN_THREADS = 256;
constexpr int SCAN_IPT = 16;
constexpr int SCAN_TILE = SCAN_THREADS * SCAN_IPT;

// Exclusive scan of one value per thread over a 256-thread block.
__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t *total) {
  __shared__ uint32_t wsum[SCAN_THREADS / WAVE];
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == WAVE - 1) wsum[w] = x;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < SCAN_THREADS / WAVE; ++k) {
    if (k < w) pre += wsum[k];
    tot += wsum[k];
  }
  __syncthreads();
  *total = tot;
  return pre + x - v;
}

__global__ __launch_bounds__(SCAN_THREADS) void k_scan_reduce(const uint32_t *in, int64_t n,
                                                              uint32_t *bsum) {
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_IPT;
  uint32_t s = 0;
  for (int k = 0; k < SCAN_IPT; ++k)
    if (base + k < n) s += in[base + k];
  uint32_t tot;
  block_excl_scan(s, &tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

// One block scans the block sums in place; *total gets the grand total.
__global__ __launch_bounds__(SCAN_THREADS) void k_scan_top(uint32_t *bsum, int64_t nb,
                                                           uint32_t *total) {
  uint32_t carry = 0;
  for (int64_t c0 = 0; c0 < nb; c0 += SCAN_THREADS) {
    const int64_t i = c0 + threadIdx.x;
    const uint32_t v = i < nb ? bsum[i] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan(v, &tot);
    if (i < nb) bsum[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0 && total) *total = carry;
}

// out may alias in: every element is read and then written by one thread.
__global__ __launch_bounds__(SCAN_THREADS) void k_scan_down(const uint32_t *in, uint32_t *out,
                                                            int64_t n, const uint32_t *bsum) {
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_IPT;
  uint32_t v[SCAN_IPT];
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < SCAN_IPT; ++k) {
    v[k] = base + k < n ? in[base + k] : 0u;
    s += v[k];
  }
  uint32_t tot;
  uint32_t run = block_excl_scan(s, &tot) + bsum[blockIdx.x];
#pragma unroll
  for (int k = 0; k < SCAN_IPT; ++k) {
    if (base + k < n) out[base + k] = run;
    run += v[k];
  }
}

// out[0..n) = exclusive prefix sums of in[0..n); *total (device, nullable)
// = the sum of all n values.
static gt_status excl_scan(const uint32_t *in, uint32_t *out, int64_t n, uint32_t *bsum,
                           uint32_t *total, hipStream_t s) {
  if (n <= 0) {
    if (total) GT_HIP(hipMemsetAsync(total, 0, sizeof(uint32_t), s));
    return GT_OK;
  }
  const int64_t nb = cdiv(n, SCAN_TILE);
  k_scan_reduce<<<dim3((unsigned)nb), dim3(SCAN_THREADS), 0, s>>>(in, n, bsum);
  GT_CHECK_LAUNCH();
  k_scan_top<<<1, SCAN_THREADS, 0, s>>>(bsum, nb, total);
  GT_CHECK_LAUNCH();
  k_scan_down<<<dim3((unsigned)nb), dim3(SCAN_THREADS), 0, s>>>(in, out, n, bsum);
  GT_CHECK_LAUNCH();
  return GT_OK;
}

// ---------------------------------------------------------------------------
// stable LSD radix sort of (uint32 key, uint32 value) pairs, 8 bits a pass
// ---------------------------------------------------------------------------
constexpr int SORT_THREADS = 256;
constexpr int SORT_ROUNDS = 16;                      // rounds of 256 items per tile
constexpr int SORT_TILE = SORT_THREADS * SORT_ROUNDS;  // 4096 items per block
constexpr int RADIX = 256;

// hist[digit * nblk + block] = count of the digit in the block's tile.
__global__ __launch_bounds__(SORT_THREADS) void k_sort_hist(const uint32_t *keys, int64_t n,
                                                            int shift, uint32_t *hist,
                                                            int64_t nblk) {
  __shared__ uint32_t h[RADIX];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
  for (int r = 0; r < SORT_ROUNDS; ++r) {
    const int64_t i = base + (int64_t)r * SORT_THREADS + threadIdx.x;
    if (i < n) atomicAdd(&h[(keys[i] >> shift) & (RADIX - 1)], 1u);
  }
  __syncthreads();
  hist[(int64_t)threadIdx.x * nblk + blockIdx.x] = h[threadIdx.x];
}

// Scatter a tile to its sorted positions.  offs = exclusive scan of hist
// (digit-major), so offs[d * nblk + b] is where the digit-d items of tile b
// start.  The tile is first sorted by digit in LDS: an item's place is the
// start of its digit in the tile plus its rank among equal digits, which
// keeps the items' order (rounds go in order, and within a round the rank
// counts the earlier waves and the lower lanes of its own wave, found by
// matching the 8 digit bits with ballots).  Then consecutive threads copy
// consecutive LDS slots out, so each digit's run leaves as contiguous
// stores.  vin == nullptr means value = item index.
__global__ __launch_bounds__(SORT_THREADS) void k_sort_scatter(
    const uint32_t *kin, const uint32_t *vin, uint32_t *kout, uint32_t *vout, int64_t n,
    int shift, const uint32_t *offs, int64_t nblk) {
  __shared__ uint32_t sk[SORT_TILE], sv[SORT_TILE];
  __shared__ uint32_t tstart[RADIX], run[RADIX], gstart[RADIX];
  __shared__ uint32_t wc[SORT_THREADS / WAVE][RADIX];
  const int t = threadIdx.x, wv = t / WAVE;
  const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
  const int64_t tile_n = std::min<int64_t>(SORT_TILE, n - base);
  // this tile's count of digit t, from consecutive entries of the
  // digit-major offsets (the last entry ends at n)
  const int64_t o = (int64_t)t * nblk + blockIdx.x;
  const uint32_t g0 = offs[o];
  const uint32_t g1 = (o + 1 < RADIX * nblk) ? offs[o + 1] : (uint32_t)n;
  uint32_t total;
  const uint32_t ts = block_excl_scan(g1 - g0, &total);
  tstart[t] = ts;
  run[t] = ts;
  gstart[t] = g0;
  const uint64_t lt = (1ull << (t & (WAVE - 1))) - 1ull;
  for (int r = 0; r < SORT_ROUNDS; ++r) {
#pragma unroll
    for (int w = 0; w < SORT_THREADS / WAVE; ++w) wc[w][t] = 0;
    __syncthreads();
    const int64_t i = base + (int64_t)r * SORT_THREADS + t;
    const bool valid = i < n;
    const uint32_t key = valid ? kin[i] : 0u;
    const uint32_t d = (key >> shift) & (RADIX - 1);
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const int rank = __popcll(peers & lt);
    if (valid && rank == 0) wc[wv][d] = (uint32_t)__popcll(peers);
    __syncthreads();
    if (valid) {
      uint32_t pos = run[d] + (uint32_t)rank;
      for (int w = 0; w < wv; ++w) pos += wc[w][d];
      sk[pos] = key;
      sv[pos] = vin ? vin[i] : (uint32_t)i;
    }
    __syncthreads();
    uint32_t add = 0;
#pragma unroll
    for (int w = 0; w < SORT_THREADS / WAVE; ++w) add += wc[w][t];
    run[t] += add;
  }
  __syncthreads();
  for (int j = t; j < tile_n; j += SORT_THREADS) {
    const uint32_t key = sk[j];
    const uint32_t d = (key >> shift) & (RADIX - 1);
    const uint32_t pos = gstart[d] + ((uint32_t)j - tstart[d]);
    kout[pos] = key;
    vout[pos] = sv[j];
  }
}

struct SortBufs {
  uint32_t *kA, *vA, *kB, *vB, *hist, *bsum;
};

// Stable sort of n pairs by the low `bits` bits of the keys.  kin may alias
// b.kA (pass 0 writes b.kB).  The sorted pairs end in (*kres, *vres), one of
// the A/B buffers.
static gt_status radix_sort(const uint32_t *kin, const uint32_t *vin, int64_t n, int bits,
                            const SortBufs &b, hipStream_t s, uint32_t **kres, uint32_t **vres) {
  bits = std::max(bits, 1);
  const int64_t nblk = std::max<int64_t>(cdiv(n, SORT_TILE), 1);
  const uint32_t *kc = kin, *vc = vin;
  uint32_t *kn = b.kB, *vn = b.vB;
  for (int shift = 0; shift < bits; shift += 8) {
    if (n > 0) {
      k_sort_hist<<<dim3((unsigned)nblk), dim3(SORT_THREADS), 0, s>>>(kc, n, shift, b.hist, nblk);
      GT_CHECK_LAUNCH();
      gt_status st = excl_scan(b.hist, b.hist, nblk * RADIX, b.bsum, nullptr, s);
      if (st != GT_OK) return st;
      k_sort_scatter<<<dim3((unsigned)nblk), dim3(SORT_THREADS), 0, s>>>(kc, vc, kn, vn, n, shift,
                                                                         b.hist, nblk);
      GT_CHECK_LAUNCH();
    }
    kc = kn;
    vc = vn;
    kn = (kn == b.kB) ? b.kA : b.kB;
    vn = (vn == b.vB) ? b.vA : b.vB;
  }
  *kres = const_cast<uint32_t *>(kc);
  *vres = const_cast<uint32_t *>(vc);
  return GT_OK;
}

// Bits needed for keys in [0, maxval]; keys are < 2^31 here.
static int bits_for(int64_t maxval) {
  int b = 0;
  while (b < 32 && maxval > 0 && (maxval >> b) != 0) ++b;
  return b;
}

// ---------------------------------------------------------------------------
// transpose
// ---------------------------------------------------------------------------
// indptr_t[c] = number of edges with column < c, found by binary search in
// the column keys sorted by the radix sort (c = 0 .. n_cols).
__global__ void k_col_ptr(const uint32_t *sorted_cols, int64_t nnz, int64_t n_cols,
                          int32_t *indptr_t) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c > n_cols) return;
  int64_t lo = 0, hi = nnz;  // first position with key >= c
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if ((int64_t)sorted_cols[mid] < c) lo = mid + 1;
    else hi = mid;
  }
  indptr_t[c] = (int32_t)lo;
}

// Row of a CSR edge: the last r with indptr[r] <= e (indptr non-decreasing).
// The row of every CSR edge, in edge order.  A workgroup takes ER_TILE
// consecutive edges: two searches give the rows of its first and last edge,
// the indptr entries between them go to LDS, and each edge then searches
// only those (the global search per edge stays as the fallback for a tile
// that spans more rows than fit, which takes many empty rows).
constexpr int ER_THREADS = 256, ER_TILE = 4096, ER_ROWS = 4096;

__global__ __launch_bounds__(ER_THREADS) void k_edge_rows(const int32_t *indptr, int64_t n_rows,
                                                          int64_t nnz, int32_t *row_of) {
  __shared__ int32_t ip[ER_ROWS + 1];
  __shared__ int32_t r01[2];
  const int64_t e0 = (int64_t)blockIdx.x * ER_TILE;
  const int64_t e1 = std::min<int64_t>(e0 + ER_TILE, nnz);   // exclusive
  if (threadIdx.x < 2)
    r01[threadIdx.x] = row_of_edge(indptr, n_rows, (int32_t)(threadIdx.x == 0 ? e0 : e1 - 1));
  __syncthreads();
  const int32_t r0 = r01[0], r1 = r01[1];
  const int64_t nr = (int64_t)r1 - r0 + 1;                   // rows r0 .. r1
  if (nr <= ER_ROWS) {
    for (int64_t k = threadIdx.x; k <= nr; k += ER_THREADS) ip[k] = indptr[r0 + k];
    __syncthreads();
    for (int64_t e = e0 + threadIdx.x; e < e1; e += ER_THREADS) {
      int lo = 0, hi = (int)nr;            // last k with ip[k] <= e, in [lo, hi)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ip[mid] <= e) lo = mid;
        else hi = mid;
      }
      row_of[e] = r0 + lo;
    }
  } else {
    for (int64_t e = e0 + threadIdx.x; e < e1; e += ER_THREADS)
      row_of[e] = row_of_edge(indptr, n_rows, (int32_t)e);
  }
}

// indices_t[t] = the row of edge perm[t]
__global__ void k_source_rows(const int32_t *row_of, const int32_t *perm, int64_t nnz,
                              int32_t *indices_t) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < nnz) indices_t[t] = row_of[perm[t]];
}

// ---------------------------------------------------------------------------
// degree-ordered schedule
// ---------------------------------------------------------------------------
struct Misc {  // device counters in the meta buffer
  uint32_t max_degree;
  uint32_t n_big, n_mid, n_small;
  uint32_t n_items, n_merges;
  uint32_t csr_flags, csr_first;
};

// Maximum degree and tier counts: each thread walks segments grid-strided,
// wavefronts reduce with shuffles, workgroups through LDS, and one thread
// per workgroup updates the counters (few enough workgroups that the
// atomics on the four counters do not queue up).
constexpr int DS_THREADS = 256, DS_MAX_BLOCKS = 1024;

__global__ __launch_bounds__(DS_THREADS) void k_degree_stats(const int32_t *ptr, int64_t n,
                                                             int32_t t_small, int32_t t_mid,
                                                             Misc *m) {
  __shared__ uint32_t red[DS_THREADS / WAVE][4];
  uint32_t d = 0, big = 0, mid = 0, small = 0;
  for (int64_t s = (int64_t)blockIdx.x * DS_THREADS + threadIdx.x; s < n;
       s += (int64_t)gridDim.x * DS_THREADS) {
    const int32_t dd = ptr[s + 1] - ptr[s];
    d = max(d, (uint32_t)dd);
    const bool b = dd > t_mid, md = !b && dd > t_small;
    big += b;
    mid += md;
    small += !b && !md;
  }
#pragma unroll
  for (int o = WAVE / 2; o > 0; o >>= 1) {
    d = max(d, (uint32_t)__shfl_xor((int)d, o));
    big += __shfl_xor((int)big, o);
    mid += __shfl_xor((int)mid, o);
    small += __shfl_xor((int)small, o);
  }
  const int w = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == 0) {
    red[w][0] = d;
    red[w][1] = big;
    red[w][2] = mid;
    red[w][3] = small;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < DS_THREADS / WAVE; ++k) {
      d = max(d, red[k][0]);
      big += red[k][1];
      mid += red[k][2];
      small += red[k][3];
    }
    atomicMax(&m->max_degree, d);
    if (big) atomicAdd(&m->n_big, big);
    if (mid) atomicAdd(&m->n_mid, mid);
    if (small) atomicAdd(&m->n_small, small);
  }
}

// Sort keys of the degree order: maxd minus the degree, a small segment's
// degree (at most t_small) rounded down to a multiple of cls; the stable sort
// then breaks ties by id.
__global__ void k_degree_keys(const int32_t *ptr, int64_t n, uint32_t maxd, int32_t t_small,
                              int32_t cls, uint32_t *key) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n) return;
  const int32_t d = ptr[s + 1] - ptr[s];
  key[s] = maxd - (uint32_t)(d <= t_small ? d - d % cls : d);
}

__global__ void k_piece_counts(const int32_t *ptr, const int32_t *order, int64_t nb,
                               int32_t chunk, uint32_t *nch, uint32_t *split) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= nb) return;
  const int32_t sg = order[k];
  const int64_t d = ptr[sg + 1] - ptr[sg];
  const uint32_t c = (uint32_t)((d + chunk - 1) / chunk);
  nch[k] = c;
  split[k] = c > 1 ? 1u : 0u;
}

// One wavefront per big segment; its lanes write the segment's pieces.
constexpr int WI_THREADS = 256;

__global__ __launch_bounds__(WI_THREADS) void k_write_items(
    const int32_t *ptr, const int32_t *order, int64_t nb, const uint32_t *item_off,
    const uint32_t *merge_off, int32_t chunk, int32_t *items, int32_t *merges) {
  const int64_t k = (int64_t)blockIdx.x * (WI_THREADS / WAVE) + threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  if (k >= nb) return;
  const int32_t sg = order[k];
  const int64_t p0 = ptr[sg], d = ptr[sg + 1] - p0;
  const int64_t nch = (d + chunk - 1) / chunk;
  const int64_t off = item_off[k];
  for (int64_t c = lane; c < nch; c += WAVE) {
    int32_t *it = items + 4 * (off + c);
    it[0] = sg;
    it[1] = (int32_t)(p0 + (c * d) / nch);
    it[2] = (int32_t)(p0 + ((c + 1) * d) / nch);
    it[3] = nch > 1 ? (int32_t)(off + c) : -1;
  }
  if (nch > 1 && lane == 0) {
    int32_t *mg = merges + 3 * (int64_t)merge_off[k];
    mg[0] = sg;
    mg[1] = (int32_t)off;
    mg[2] = (int32_t)nch;
  }
}

// spans[k] = (ptr[order[k]], ptr[order[k] + 1])
__global__ void k_spans(const int32_t *ptr, const int32_t *order, int64_t n, int32_t *spans) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int32_t sg = order[k];
  *reinterpret_cast<int2 *>(spans + 2 * k) = make_int2(ptr[sg], ptr[sg + 1]);
}

// The two schedules (rows of A and of A^T) are built side by side, so that
// the host reads their sizes back twice in all (after the degree statistics
// and after the piece lists) instead of twice per schedule.
struct SchedJob {
  const int32_t *ptr;   // segment pointer (indptr or indptr_t)
  int64_t n;            // segments
  Misc *misc_d;         // this schedule's device counters
  gt_sched *out;
  int32_t small_class;  // small segments ordered by degree rounded down to a multiple of this
  Misc m;               // host copy of the counters
};

// Piece order (the definition is in gt_attn.h): the pieces of the big
// segments, written segment after segment, are dealt to the XCDs by their
// position in their segment.  Workgroups go to the XCDs in turn and hold
// four wavefronts each, so block k of the list (items 4k .. 4k + 3) runs on
// XCD k mod 8; queue x holds the pieces in the x-th eighth of their
// segments, in position order, so each XCD works on one eighth of every big
// segment's range (of columns for the rows of A, of source rows for the
// columns of A^T) at a time, and the rows those pieces gather are shared in
// its L2.  Slots stay the segment-major indices, so the merges are
// unchanged.  The list is short (about nnz / chunk items), so it is dealt on
// the host, which prepare synchronises with anyway.
static gt_status deal_items(gt_sched *out, hipStream_t s) {
  const int64_t n = out->n_items;
  std::vector<int32_t> it((size_t)n * 4), dealt((size_t)n * 4);
  GT_HIP(hipMemcpyAsync(it.data(), out->items, sizeof(int32_t) * 4 * (size_t)n,
                        hipMemcpyDeviceToHost, s));
  GT_HIP(hipStreamSynchronize(s));
  // bucket q of every piece, then the pieces of each bucket in list order
  std::vector<int64_t> byq[64];
  for (int64_t i = 0; i < n;) {
    int64_t e = i;
    while (e < n && it[4 * e] == it[4 * i]) ++e;   // the pieces of one segment
    const int64_t nch = e - i;
    for (int64_t c = 0; c < nch; ++c) byq[(64 * (2 * c + 1)) / (2 * nch)].push_back(i + c);
    i = e;
  }
  std::vector<int64_t> q[8];
  for (int b = 0; b < 64; ++b) q[b / 8].insert(q[b / 8].end(), byq[b].begin(), byq[b].end());
  size_t head[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int64_t pos = 0;
  for (int64_t k = 0; pos < n; ++k) {
    for (int t = 0; t < 4 && pos < n; ++t) {
      int x = (int)(k % 8);
      while (head[x] == q[x].size()) x = (x + 1) % 8;
      const int64_t src = q[x][head[x]++];
      for (int f = 0; f < 4; ++f) dealt[4 * pos + f] = it[4 * src + f];
      ++pos;
    }
  }
  GT_HIP(hipMemcpyAsync(out->items, dealt.data(), sizeof(int32_t) * 4 * (size_t)n,
                        hipMemcpyHostToDevice, s));
  GT_HIP(hipStreamSynchronize(s));
  return GT_OK;
}

static gt_status build_schedules(SchedJob (&jobs)[2], int32_t t_small, int32_t t_mid,
                                 int32_t chunk, const SortBufs &b, hipStream_t s) {
  const int TB = 256;
  // phase 1: degree statistics of both
  for (SchedJob &j : jobs) {
    GT_HIP(hipMemsetAsync(j.misc_d, 0, sizeof(Misc), s));
    if (j.n > 0) {
      const int64_t nblk = std::min<int64_t>(cdiv(j.n, DS_THREADS), DS_MAX_BLOCKS);
      k_degree_stats<<<dim3((unsigned)nblk), dim3(DS_THREADS), 0, s>>>(j.ptr, j.n, t_small, t_mid,
                                                                       j.misc_d);
      GT_CHECK_LAUNCH();
    }
  }
  for (SchedJob &j : jobs)
    GT_HIP(hipMemcpyAsync(&j.m, j.misc_d, sizeof(Misc), hipMemcpyDeviceToHost, s));
  GT_HIP(hipStreamSynchronize(s));
  // phase 2: degree order, extents and piece lists of each (the sort
  // scratch is reused in stream order)
  for (SchedJob &j : jobs) {
    gt_sched *out = j.out;
    const int64_t n = j.n;
    if (n > 0) {
      k_degree_keys<<<dim3((unsigned)cdiv(n, TB)), dim3(TB), 0, s>>>(j.ptr, n, j.m.max_degree,
                                                                     t_small, j.small_class, b.kA);
      GT_CHECK_LAUNCH();
    }
    uint32_t *ks, *vs;
    gt_status st = radix_sort(b.kA, nullptr, n, bits_for(j.m.max_degree), b, s, &ks, &vs);
    if (st != GT_OK) return st;
    if (n > 0) {
      GT_HIP(hipMemcpyAsync(out->order, vs, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToDevice,
                            s));
      k_spans<<<dim3((unsigned)cdiv(n, TB)), dim3(TB), 0, s>>>(j.ptr, out->order, n, out->spans);
      GT_CHECK_LAUNCH();
    }
    const int64_t nb = j.m.n_big;
    if (nb > 0) {
      // piece counts and split flags of the big segments, then their offsets
      uint32_t *nch = b.kA, *split = b.kB, *ioff = b.vA, *moff = b.vB;
      k_piece_counts<<<dim3((unsigned)cdiv(nb, TB)), dim3(TB), 0, s>>>(j.ptr, out->order, nb,
                                                                        chunk, nch, split);
      GT_CHECK_LAUNCH();
      st = excl_scan(nch, ioff, nb, b.bsum, &j.misc_d->n_items, s);
      if (st != GT_OK) return st;
      st = excl_scan(split, moff, nb, b.bsum, &j.misc_d->n_merges, s);
      if (st != GT_OK) return st;
      k_write_items<<<dim3((unsigned)cdiv(nb, WI_THREADS / WAVE)), dim3(WI_THREADS), 0, s>>>(
          j.ptr, out->order, nb, ioff, moff, chunk, out->items, out->merges);
      GT_CHECK_LAUNCH();
    }
  }
  for (SchedJob &j : jobs)
    if (j.m.n_big > 0)
      GT_HIP(hipMemcpyAsync(&j.m, j.misc_d, sizeof(Misc), hipMemcpyDeviceToHost, s));
  GT_HIP(hipStreamSynchronize(s));
  for (SchedJob &j : jobs) {
    gt_sched *out = j.out;
    out->n_seg = j.n;
    out->n_big = j.m.n_big;
    out->n_mid = j.m.n_mid;
    out->n_small = j.m.n_small;
    out->n_items = j.m.n_big > 0 ? j.m.n_items : 0;
    out->n_merges = j.m.n_big > 0 ? j.m.n_merges : 0;
    out->max_degree = j.m.max_degree;
    if (out->n_items > 1) {
      const gt_status st2 = deal_items(out, s);
      if (st2 != GT_OK) return st2;
    }
  }
  return GT_OK;
}

// ---------------------------------------------------------------------------
// validator
// ---------------------------------------------------------------------------
__global__ void k_val_ptr(const int32_t *indptr, int64_t n_rows, int64_t nnz, Misc *m) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r == 0 && (indptr[0] != 0 || (int64_t)indptr[n_rows] != nnz)) atomicOr(&m->csr_flags, 1u);
  if (r < n_rows && indptr[r + 1] < indptr[r]) atomicOr(&m->csr_flags, 2u);
}

// Every edge: its column in range, and above the previous edge's column
// unless it starts its row.  Runs once the row pointer has passed k_val_ptr
// (so it is non-decreasing from 0 to nnz).  The first bad edge e is kept as
// 2e (column out of range) or 2e + 1 (columns not increasing).  Rows are
// found as in k_edge_rows: per tile of consecutive edges, in an LDS copy of
// the row pointer between the tile's first and last row.
__global__ __launch_bounds__(ER_THREADS) void k_val_edges(const int32_t *indptr,
                                                          const int32_t *indices, int64_t n_rows,
                                                          int64_t n_cols, int64_t nnz, Misc *m) {
  __shared__ int32_t ip[ER_ROWS + 1];
  __shared__ int32_t r01[2];
  const int64_t e0 = (int64_t)blockIdx.x * ER_TILE;
  const int64_t e1 = std::min<int64_t>(e0 + ER_TILE, nnz);   // exclusive
  if (threadIdx.x < 2)
    r01[threadIdx.x] = row_of_edge(indptr, n_rows, (int32_t)(threadIdx.x == 0 ? e0 : e1 - 1));
  __syncthreads();
  const int32_t r0 = r01[0];
  const int64_t nr = (int64_t)r01[1] - r0 + 1;               // rows r0 .. r1
  const bool local = nr <= ER_ROWS;
  if (local)
    for (int64_t k = threadIdx.x; k <= nr; k += ER_THREADS) ip[k] = indptr[r0 + k];
  __syncthreads();
  for (int64_t e = e0 + threadIdx.x; e < e1; e += ER_THREADS) {
    const int32_t c = indices[e];
    if (c < 0 || (int64_t)c >= n_cols) {
      atomicMin(&m->csr_first, (uint32_t)(2 * e));
      continue;
    }
    int32_t start;                       // the first edge of e's row
    if (local) {
      int lo = 0, hi = (int)nr;          // last k with ip[k] <= e, in [lo, hi)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ip[mid] <= e) lo = mid;
        else hi = mid;
      }
      start = ip[lo];
    } else {
      start = indptr[row_of_edge(indptr, n_rows, (int32_t)e)];
    }
    if (e > start && c <= indices[e - 1]) atomicMin(&m->csr_first, (uint32_t)(2 * e + 1));
  }
}

}  // namespace gt

using namespace gt;

extern "C" size_t gt_graph_meta_bytes(int64_t n_rows, int64_t n_cols, int64_t nnz,
                                      int32_t chunk) {
  MetaLayout L;
  if (!meta_layout(n_rows, n_cols, nnz, chunk, &L)) return 0;
  return L.total;
}

extern "C" void gt_default_thresholds(int32_t *t_small, int32_t *t_mid, int32_t *chunk) {
  if (t_small) *t_small = DEFAULT_T_SMALL;
  if (t_mid) *t_mid = DEFAULT_CHUNK;
  if (chunk) *chunk = DEFAULT_CHUNK;
}

extern "C" void gt_graph_thresholds(int64_t nnz, int32_t *t_small, int32_t *t_mid,
                                    int32_t *chunk) {
  const int32_t c = chunk_for(nnz);
  if (t_small) *t_small = DEFAULT_T_SMALL;
  if (t_mid) *t_mid = c;
  if (chunk) *chunk = c;
}

extern "C" gt_status gt_graph_prepare(const int32_t *indptr, const int32_t *indices,
                                      int64_t n_rows, int64_t n_cols, int64_t nnz,
                                      int32_t t_small, int32_t t_mid, int32_t chunk, void *meta,
                                      size_t meta_bytes, gt_graph *out, void *stream) {
  clear_error();
  if (!out) return fail(GT_E_NULL, "out is NULL");
  if (!indptr) return fail(GT_E_NULL, "indptr is NULL");
  if (nnz > 0 && !indices) return fail(GT_E_NULL, "indices is NULL");
  if (!meta) return fail(GT_E_NULL, "meta is NULL");
  if (t_small < 0 || t_mid < t_small || chunk < 1)
    return fail(GT_E_ARG, "thresholds need 0 <= t_small <= t_mid and chunk >= 1");
  MetaLayout L;
  if (!meta_layout(n_rows, n_cols, nnz, chunk, &L))
    return fail(GT_E_ARG, "sizes out of range (n_rows %lld, n_cols %lld, nnz %lld)",
                (long long)n_rows, (long long)n_cols, (long long)nnz);
  if (meta_bytes < L.total)
    return fail(GT_E_WORKSPACE, "meta has %zu bytes, needs %zu", meta_bytes, L.total);
  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)meta;
  auto at = [&](size_t off) { return (void *)(base + off); };
  gt_graph g;
  memset(&g, 0, sizeof(g));
  g.n_rows = n_rows;
  g.n_cols = n_cols;
  g.nnz = nnz;
  g.indptr = indptr;
  g.indices = indices;
  g.indptr_t = (int32_t *)at(L.indptr_t);
  g.indices_t = (int32_t *)at(L.indices_t);
  g.perm = (int32_t *)at(L.perm);
  g.rows.order = (int32_t *)at(L.row_order);
  g.rows.items = (int32_t *)at(L.row_items);
  g.rows.merges = (int32_t *)at(L.row_merges);
  g.rows.spans = (int32_t *)at(L.row_spans);
  g.cols.order = (int32_t *)at(L.col_order);
  g.cols.items = (int32_t *)at(L.col_items);
  g.cols.merges = (int32_t *)at(L.col_merges);
  g.cols.spans = (int32_t *)at(L.col_spans);
  g.t_small = t_small;
  g.t_mid = t_mid;
  g.chunk = chunk;
  SortBufs b{(uint32_t *)at(L.kA), (uint32_t *)at(L.vA), (uint32_t *)at(L.kB),
             (uint32_t *)at(L.vB), (uint32_t *)at(L.hist), (uint32_t *)at(L.bsum)};
  static_assert(2 * sizeof(Misc) <= 64 * sizeof(int32_t), "meta holds two Misc");
  Misc *misc = (Misc *)at(L.misc);   // [0] rows of A, [1] rows of A^T
  const int TB = 256;

  // perm: edge ids stably sorted by column; indptr_t: where each column's
  // run starts in the sorted keys; indices_t: the source rows of perm
  uint32_t *ks, *vs;
  gt_status st = radix_sort((const uint32_t *)indices, nullptr, nnz, bits_for(n_cols - 1), b, s,
                            &ks, &vs);
  if (st != GT_OK) return st;
  k_col_ptr<<<dim3((unsigned)cdiv(n_cols + 1, TB)), dim3(TB), 0, s>>>(ks, nnz, n_cols, g.indptr_t);
  GT_CHECK_LAUNCH();
  if (nnz > 0) {
    GT_HIP(hipMemcpyAsync(g.perm, vs, sizeof(int32_t) * (size_t)nnz, hipMemcpyDeviceToDevice, s));
    // the sort buffers are free again (stream order): rows of the edges in
    // edge order into one of them, then gathered through perm
    int32_t *row_of = (int32_t *)(vs == b.vA ? b.vB : b.vA);
    k_edge_rows<<<dim3((unsigned)cdiv(nnz, ER_TILE)), dim3(ER_THREADS), 0, s>>>(indptr, n_rows,
                                                                               nnz, row_of);
    GT_CHECK_LAUNCH();
    k_source_rows<<<dim3((unsigned)cdiv(nnz, TB)), dim3(TB), 0, s>>>(row_of, g.perm, nnz,
                                                                      g.indices_t);
    GT_CHECK_LAUNCH();
  }
  SchedJob jobs[2] = {{indptr, n_rows, misc, &g.rows, ROW_SMALL_CLASS, {}},
                      {g.indptr_t, n_cols, misc + 1, &g.cols, 1, {}}};
  st = build_schedules(jobs, t_small, t_mid, chunk, b, s);
  if (st != GT_OK) return st;
  GT_HIP(hipStreamSynchronize(s));
  *out = g;
  return GT_OK;
}

extern "C" gt_status gt_csr_validate(const int32_t *indptr, const int32_t *indices,
                                     int64_t n_rows, int64_t n_cols, int64_t nnz, void *work,
                                     size_t work_bytes, int32_t *code, void *stream) {
  clear_error();
  if (!indptr || !code || !work || (nnz > 0 && !indices)) return fail(GT_E_NULL, "NULL argument");
  if (n_rows < 0 || n_cols < 0 || nnz < 0 || n_rows >= INT32_MAX || n_cols >= INT32_MAX ||
      nnz >= INT32_MAX)
    return fail(GT_E_ARG, "sizes out of range");
  if (work_bytes < GT_VALIDATE_WORK_BYTES)
    return fail(GT_E_WORKSPACE, "work has %zu bytes, needs %d", work_bytes,
                (int)GT_VALIDATE_WORK_BYTES);
  static_assert(sizeof(Misc) <= GT_VALIDATE_WORK_BYTES, "validator scratch");
  hipStream_t s = (hipStream_t)stream;
  Misc *m = (Misc *)work;
  Misc h;
  memset(&h, 0, sizeof(h));
  h.csr_first = 0xffffffffu;
  const int TB = 256;
  GT_HIP(hipMemcpyAsync(m, &h, sizeof(Misc), hipMemcpyHostToDevice, s));
  k_val_ptr<<<dim3((unsigned)cdiv(n_rows + 1, TB)), dim3(TB), 0, s>>>(indptr, n_rows, nnz, m);
  GT_CHECK_LAUNCH();
  GT_HIP(hipMemcpyAsync(&h, m, sizeof(Misc), hipMemcpyDeviceToHost, s));
  GT_HIP(hipStreamSynchronize(s));
  int32_t c = 0;
  if (h.csr_flags & 1u) {
    c = 1;
  } else if (h.csr_flags & 2u) {
    c = 2;
  } else if (nnz > 0) {
    k_val_edges<<<dim3((unsigned)cdiv(nnz, ER_TILE)), dim3(ER_THREADS), 0, s>>>(indptr, indices,
                                                                               n_rows, n_cols, nnz, m);
    GT_CHECK_LAUNCH();
    GT_HIP(hipMemcpyAsync(&h, m, sizeof(Misc), hipMemcpyDeviceToHost, s));
    GT_HIP(hipStreamSynchronize(s));
    if (h.csr_first != 0xffffffffu) c = (h.csr_first & 1u) ? 4 : 3;
  }
  *code = c;
  if (c != 0) return fail(GT_E_CSR, "malformed CSR (code %d)", c);
  return GT_OK;
}
