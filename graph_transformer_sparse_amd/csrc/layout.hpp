// Layout of the caller's `meta` buffer of a prepared graph, and the
// default thresholds of the degree-ordered schedule.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace gt {

// Segments (rows of A or of A^T) with at most DEFAULT_T_SMALL nonzeros are
// handled by a lane group inside a wavefront; longer ones by whole
// wavefronts, in pieces of at most DEFAULT_CHUNK nonzeros.
constexpr int32_t DEFAULT_T_SMALL = 32;
constexpr int32_t DEFAULT_CHUNK = 256;

// In the schedule over the rows of A, small rows are ordered by their degree
// rounded down to a multiple of ROW_SMALL_CLASS (descending), then by id:
// the four rows of a wavefront still have nearly equal lengths, and rows
// with neighbouring ids, which share staged dbias lines (and, in graphs
// whose ids carry locality, neighbours), run together.  Measured per step
// against exact degrees: Hub 12.24 -> 12.13 ms, Mid 0.624 -> 0.619 ms,
// Large 6.38 -> 6.36 ms, Shard unchanged.  The transpose's schedule keeps
// exact degrees: there the same classes cost Shard, whose columns are 61 %
// empty, 0.17 ms in the column pass.
constexpr int32_t ROW_SMALL_CLASS = 4;

// Pieces are dealt to the XCDs by their position in their segment, so the
// shorter the pieces, the narrower the range of rows each XCD gathers at a
// time (and the more merge work).  Measured with the dealt order, per step
// (2048 / 512 / 256-nonzero pieces): Hub 12.86 / 12.26 / 12.15 ms, Large
// 6.63 / 6.42 / 6.35 ms, Mid (512 / 256) 0.625 / 0.623 ms.  Before the
// dealing, pieces of 2048 were the better choice from 8M nonzeros on; now
// one size serves every graph.
inline int32_t chunk_for(int64_t) { return DEFAULT_CHUNK; }

constexpr int SORT_TILE_ITEMS = 4096;   // items per radix-sort block
constexpr int SCAN_TILE_ITEMS = 4096;   // items per scan block

// Capacity of a schedule's piece list: sum over big segments of
// ceil(d / chunk) <= floor(nnz / chunk) + n_seg.
inline int64_t sched_cap(int64_t n_seg, int64_t nnz, int32_t chunk) {
  return n_seg + nnz / chunk + 1;
}

// Floats per piece slot of a split segment, for each pass (D = heads *
// head_dim, H = heads; a multiple of 4 so slots stay 16-byte aligned):
//   forward   [acc D][m H][l H]
//   row pass  [A1 D][A2 D][S H][L H][c H]
//   column    [dK D][dV D]
constexpr int64_t round4(int64_t x) { return (x + 3) / 4 * 4; }
constexpr int64_t fwd_slot_floats(int64_t D, int64_t H) { return round4(D + 2 * H); }
constexpr int64_t rows_slot_floats(int64_t D, int64_t H) { return round4(2 * D + 3 * H); }
constexpr int64_t cols_slot_floats(int64_t D, int64_t) { return 2 * D; }

struct MetaLayout {
  size_t indptr_t, indices_t, perm;
  size_t row_order, row_items, row_merges, row_spans;
  size_t col_order, col_items, col_merges, col_spans;
  size_t kA, vA, kB, vB, hist, bsum, misc;
  size_t total;
};

inline bool meta_layout(int64_t R, int64_t M, int64_t E, int32_t chunk, MetaLayout *L) {
  const int64_t LIM = INT32_MAX - 1;
  if (R < 0 || M < 0 || E < 0 || R > LIM || M > LIM || E > LIM || chunk < 1) return false;
  size_t off = 0;
  auto take = [&](int64_t words) {
    size_t at = off;
    off += ((size_t)std::max<int64_t>(words, 1) * 4 + 255) / 256 * 256;
    return at;
  };
  const int64_t capR = sched_cap(R, E, chunk), capM = sched_cap(M, E, chunk);
  L->indptr_t = take(M + 1);
  L->indices_t = take(E);
  L->perm = take(E);
  L->row_order = take(R);
  L->row_items = take(4 * capR);
  L->row_merges = take(3 * capR);
  L->row_spans = take(2 * R);
  L->col_order = take(M);
  L->col_items = take(4 * capM);
  L->col_merges = take(3 * capM);
  L->col_spans = take(2 * M);
  const int64_t nmax = std::max<int64_t>({E, R, M, 1});
  const int64_t nblk = (nmax + SORT_TILE_ITEMS - 1) / SORT_TILE_ITEMS;
  const int64_t scan_len = std::max<int64_t>({256 * nblk, M + 1, R + 1});
  L->kA = take(nmax);
  L->vA = take(nmax);
  L->kB = take(nmax);
  L->vB = take(nmax);
  L->hist = take(256 * nblk);
  L->bsum = take((scan_len + SCAN_TILE_ITEMS - 1) / SCAN_TILE_ITEMS + 1);
  L->misc = take(64);
  L->total = off;
  return true;
}

}  // namespace gt
