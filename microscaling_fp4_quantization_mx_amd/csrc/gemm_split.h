// The last, partly filled round of 256 x 256 tiles split along K: the K-part
// partial tiles of the block-scaled GEMMs and their in-order sum.
//
// A partial tile is stored in the accumulators' own layout: float4 slot
// ((wave * TI + i) * TJ + j) * 4 + q) * 64 + lane holds registers 4q .. 4q+3
// of 32 x 32 tile (i, j) of the wave's 128 x 128 block, i.e. rows
// 8q + 4 (lane / 32) + 0..3 of that 32 x 32 tile, column lane % 32 (the
// v_mfma 32x32 output layout), so every store and load is 16 coalesced bytes
// per lane.
#pragma once
#include "gemm_tiles.h"
#include "mx_device.h"

namespace mxk {

constexpr int kGemmSplitMax = 4;            // K parts per split tile
constexpr int kSplitTileFloats = 256 * 256; // one fp32 partial tile

// The K parts of split tile u, part `part` of S, into partial tile u * S + part.
template <int TI, int TJ>
__device__ __forceinline__ void gemm_split_store_partial(const f32x16 (&acc)[TI][TJ], float* part, int u, int S,
                                                         int partno) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4* mine = reinterpret_cast<f32x4*>(part) + (size_t)(u * S + partno) * (kSplitTileFloats / 4);
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_nontemporal_store(f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]},
                                    mine + (((wave * TI + i) * TJ + j) * 4 + q) * 64 + lane);
}

struct GemmSplitReduce {
  const float* part;
  void* c;
  int64_t ldc;
  int c_bf16;
  int M, N, groups;
  const int32_t* offsets;
  int cus, split_max, parts;   // as given to gemm_split by the GEMM
  const float* ga;             // C = (sum of parts) * (*ga) * (*gb) when both are given
  const float* gb;
};

// C of the split tiles: the S partials of each added in part order (so C does
// not depend on which part finished first), times the global scales if any,
// rounded as the whole-tile epilogues round.  WGT workgroups per tile, each
// a 1/WGT share of the slots, consecutive threads consecutive slots, a part's
// loads all in flight before the adds.  Tile geometry as the GEMM's (raster
// group GM).
constexpr int kSplitReduceWgPerTile = 16;
template <int GM>
__global__ __launch_bounds__(256) void k_gemm_split_reduce(GemmSplitReduce p) {
  constexpr int TI = 4, TJ = 4, WM = 128, WN = 128, NWX = 2;
  constexpr int SLOTS = kSplitTileFloats / 4;
  constexpr int WGT = kSplitReduceWgPerTile;
  constexpr int PER_T = SLOTS / WGT / 256;
  const int total = gemm_tile_count<256, 256>(p.M, p.N, p.groups, p.offsets);
  const GemmSplit sp = gemm_split(total, p.cus, p.split_max, p.parts);
  const int u = blockIdx.x / WGT;
  if (u >= sp.r) return;
  const int base = (blockIdx.x % WGT) * (SLOTS / WGT) + threadIdx.x;
  const f32x4* src = reinterpret_cast<const f32x4*>(p.part) + (size_t)u * sp.S * SLOTS + base;
  f32x4 v[PER_T];
#pragma unroll
  for (int k = 0; k < PER_T; ++k) v[k] = __builtin_nontemporal_load(src + 256 * k);
  for (int q = 1; q < sp.S; ++q) {
    f32x4 w[PER_T];
#pragma unroll
    for (int k = 0; k < PER_T; ++k) w[k] = __builtin_nontemporal_load(src + (size_t)q * SLOTS + 256 * k);
    __builtin_amdgcn_sched_barrier(0);   // all of this part's loads in flight before the first add
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      v[k][0] += w[k][0];
      v[k][1] += w[k][1];
      v[k][2] += w[k][2];
      v[k][3] += w[k][3];
    }
  }
  const float gg = (p.ga && p.gb) ? (*p.ga) * (*p.gb) : 1.0f;
  GemmTile tile;
  gemm_tile_at<256, 256, GM>(sp.full + u, p.M, p.N, p.groups, p.offsets, tile);
#pragma unroll
  for (int k = 0; k < PER_T; ++k) {
    const int idx = base + 256 * k;
    const int lane = idx & 63, rest = idx >> 6;
    const int q = rest & 3, j = (rest >> 2) % TJ, i = (rest >> 2) / TJ % TI, wave = (rest >> 2) / (TJ * TI);
    const int wy = wave / NWX, wx = wave % NWX;
    const int col = tile.n0 + wx * WN + j * 32 + (lane & 31);
    const int row0 = tile.m0 + wy * WM + i * 32 + 8 * q + 4 * (lane >> 5);
    if (col >= p.N) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = row0 + e;
      if (row >= tile.m_end) break;
      const float y = (p.ga && p.gb) ? v[k][e] * gg : v[k][e];
      if (p.c_bf16)
        reinterpret_cast<uint16_t*>(p.c)[(size_t)row * p.ldc + col] = (uint16_t)f32_to_bf16_rne(y);
      else
        reinterpret_cast<float*>(p.c)[(size_t)row * p.ldc + col] = y;
    }
  }
}

// Scratch for the partials: r split tiles x S parts <= min(cus, tiles x
// kGemmSplitMax) partial tiles; 0 when no split can occur (a dense product
// that fills whole rounds, or fewer than 2 K parts).
inline size_t gemm_split_bytes(int64_t M, int64_t N, int groups, int cus, int parts) {
  if (M <= 0 || N <= 0 || cus < 2 || parts < 2) return 0;
  const int64_t bound = gemm_tile_bound(M, N, 256, 256, groups);
  if (groups == 0 && bound % cus == 0) return 0;
  const int64_t tiles = bound * kGemmSplitMax < cus ? bound * kGemmSplitMax : cus;
  return (size_t)tiles * kSplitTileFloats * sizeof(float);
}

}  // namespace mxk
