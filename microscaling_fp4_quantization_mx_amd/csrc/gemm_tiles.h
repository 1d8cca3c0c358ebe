// Output tile of a workgroup in the dense and grouped GEMMs.
//
// Grouped form: rows [off[g], off[g+1]) of A and C use weight matrix g; tiles
// of BM x BN never straddle a group's rows, so every group has
// ceil(rows_g / BM) tile rows (the last one ragged).  Offsets are clamped to
// [0, M] on the device, so malformed offsets cannot index out of bounds.
//
// Workgroup -> tile mapping: consecutive workgroup ids run on different XCDs
// (round-robin dispatch), so workgroup b takes tile (b % 8) * per_xcd + b / 8:
// each XCD walks a contiguous run of tiles and shares their A/B panels in its
// own L2.  Within a group, GM tile rows at a time walk all tile columns.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

struct GemmTile {
  int g;          // weight matrix (0 when dense)
  int m_begin;    // first row of the group
  int m_end;      // end of the group's rows (M when dense)
  int m0, n0;     // first row and column of the tile
};

// Tiles of the product: every group adds ceil(rows_g / BM) tile rows of
// ceil(N / BN) tiles.
template <int BM, int BN>
__device__ __forceinline__ int gemm_tile_count(int M, int N, int groups, const int32_t* offsets) {
  const int tn_count = (N + BN - 1) / BN;
  if (groups == 0) return ((M + BM - 1) / BM) * tn_count;
  int total = 0;
  for (int i = 0; i < groups; ++i) {
    const int o0 = min(max(offsets[i], 0), M), o1 = min(max(offsets[i + 1], 0), M);
    const int rows = o1 > o0 ? o1 - o0 : 0;
    total += ((rows + BM - 1) / BM) * tn_count;
  }
  return total;
}

// Geometry of tile t (0 <= t < gemm_tile_count) in raster order: groups in
// turn; within a group, GM tile rows at a time walk all tile columns.
template <int BM, int BN, int GM>
__device__ __forceinline__ void gemm_tile_at(int t, int M, int N, int groups, const int32_t* offsets, GemmTile& o) {
  const int tn_count = (N + BN - 1) / BN;
  o.g = 0;
  o.m_begin = 0;
  o.m_end = M;
  int tl = t;  // tile index within its group
  if (groups != 0) {
    for (int i = 0; i < groups; ++i) {
      const int o0 = min(max(offsets[i], 0), M), o1 = min(max(offsets[i + 1], 0), M);
      const int rows = o1 > o0 ? o1 - o0 : 0;
      const int nt = ((rows + BM - 1) / BM) * tn_count;
      if (tl < nt) {
        o.g = i;
        o.m_begin = o0;
        o.m_end = o1;
        break;
      }
      tl -= nt;
    }
  }
  const int tm_count = (o.m_end - o.m_begin + BM - 1) / BM;
  const int per_group = GM * tn_count;
  const int first_m = (tl / per_group) * GM;
  const int gm = min(tm_count - first_m, GM);
  const int in_grp = tl % per_group;
  o.m0 = o.m_begin + (first_m + in_grp % gm) * BM;
  o.n0 = (in_grp / gm) * BN;
}

// Workgroup bid of a grid of ceil(total / 8) * 8: its tile, XCD-remapped
// (false: no tile; the grid is rounded up to whole XCD runs).
__device__ __forceinline__ int gemm_tile_remap(int bid, int total) {
  const int per_xcd = (total + 7) / 8;
  const int local = bid / 8;
  if (local >= per_xcd) return -1;
  const int t = (bid % 8) * per_xcd + local;
  return t < total ? t : -1;
}

// false: this workgroup has no tile (the grid is rounded up to whole XCD runs)
template <int BM, int BN, int GM>
__device__ __forceinline__ bool gemm_tile(int bid, int M, int N, int groups, const int32_t* offsets, GemmTile& o) {
  const int t = gemm_tile_remap(bid, gemm_tile_count<BM, BN>(M, N, groups, offsets));
  if (t < 0) return false;
  gemm_tile_at<BM, BN, GM>(t, M, N, groups, offsets, o);
  return true;
}

// Split of the last, partly filled round of tiles along K.  With T tiles on
// `cus` workgroup slots (one workgroup per CU), the last r = T % cus tiles
// would run alone for a whole tile's time; instead each is cut into S K-parts
// (S <= split_max, r * S <= cus, at most `parts` pieces of K), computed by
// r * S workgroups that follow the T - r whole tiles.  S = 1: no split.
struct GemmSplit {
  int full;   // whole tiles (the first `full` in raster order)
  int r;      // split tiles (the rest)
  int S;      // K parts per split tile
};
__device__ __forceinline__ GemmSplit gemm_split(int T, int cus, int split_max, int parts) {
  GemmSplit o{T, 0, 1};
  if (split_max < 2 || cus < 2 || T <= 0) return o;
  const int r = T % cus;
  if (r == 0) return o;
  const int S = min(min(split_max, cus / r), parts);
  if (S < 2) return o;
  o.full = T - r;
  o.r = r;
  o.S = S;
  return o;
}

// Upper bound of the tile count for the launch grid: every group adds at
// most one ragged tile row.
inline int64_t gemm_tile_bound(int64_t M, int64_t N, int BM, int BN, int groups) {
  return ((M + BM - 1) / BM + (groups > 0 ? groups : 0)) * ((N + BN - 1) / BN);
}

}  // namespace mxk
