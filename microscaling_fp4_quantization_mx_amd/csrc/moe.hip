// Mixture-of-experts data movement around the grouped W4A4 GEMM, for gfx950.
//
// Routed expert weights are where block-scaled FP4 pays most ("NVFP4
// Architecture", section "Strategic Recommendations: Adopting NVFP4 in 2026";
// the "MXFP4" card, section "Core Facts", lists grouped GEMM and TopK among
// the operations of an MXFP4 serving stack).  A routed layer is
//   route   : (token, slot) pairs -> expert-sorted rows (stable counting sort)
//   gather  : quantize the routed tokens' activations in that order (quantize.hip)
//   GEMM    : grouped W4A4 over the per-expert row ranges (gemm_mxfp4.hip)
//   combine : out[t] = sum_s w[t, s] * y[row(t, s)]
// Every step is deterministic: the sort is stable (pairs of one expert keep
// their flat order t * topk + s) and the combine sums the slots in order.
#include <algorithm>

#include "mx_device.h"
#include "mx_kernels.h"

namespace mxk {

constexpr int RT = 256;   // threads per workgroup of the counting kernels

// The pairs are cut into C chunks of `ch` consecutive pairs (ch a multiple of
// 64, at least kRouteChunkMin unless there are fewer pairs), with
// C * experts <= kRouteTable, so that the per-chunk counts fit a workspace
// whose size depends on the expert count only.  Every pass is linear in the
// pairs plus C * experts: one counting pass over the pairs, a scan over the
// counts, one assignment pass over the pairs.
constexpr int kRouteTable = 1 << 16;
constexpr int kRouteChunkMin = 1024;

int route_max_chunks(int experts) { return experts >= kRouteTable ? 1 : kRouteTable / experts; }

// Workgroup c counts the pairs of chunk c per expert: hist[c][e].
__global__ __launch_bounds__(RT) void k_route_hist(const int32_t* __restrict__ ids, int npairs, int experts, int ch,
                                                   int32_t* __restrict__ hist) {
  const int c = blockIdx.x;
  int32_t* row = hist + (size_t)c * experts;
  for (int e = threadIdx.x; e < experts; e += RT) row[e] = 0;
  __threadfence();   // the zeros are in memory before any lane's increment
  __syncthreads();
  const int64_t p0 = (int64_t)c * ch, p1 = min((int64_t)npairs, p0 + ch);
  for (int64_t p = p0 + threadIdx.x; p < p1; p += RT) {
    const int e = ids[p];
    if (e >= 0 && e < experts) atomicAdd(&row[e], 1);
  }
}

// Thread e: hist[c][e] <- pairs of expert e in chunks before c (exclusive
// prefix down the column), tot[e] <- all pairs of expert e.
__global__ __launch_bounds__(RT) void k_route_colscan(int chunks, int experts, int32_t* __restrict__ hist,
                                                      int32_t* __restrict__ tot) {
  const int e = blockIdx.x * RT + threadIdx.x;
  if (e >= experts) return;
  int run = 0;
  for (int c = 0; c < chunks; ++c) {
    const int h = hist[(size_t)c * experts + e];
    hist[(size_t)c * experts + e] = run;
    run += h;
  }
  tot[e] = run;
}

// One workgroup: offsets[g] = sum_{e < g} tot[e] for g = 0 .. experts.
constexpr int RO_T = 1024;
__global__ __launch_bounds__(RO_T) void k_route_offsets(int experts, const int32_t* __restrict__ tot,
                                                        int32_t* __restrict__ offsets) {
  __shared__ int part[RO_T];
  const int t = threadIdx.x;
  const int per = (experts + RO_T - 1) / RO_T;
  const int e0 = min(experts, t * per), e1 = min(experts, e0 + per);
  int s = 0;
  for (int e = e0; e < e1; ++e) s += tot[e];
  part[t] = s;
  __syncthreads();
  // inclusive scan of the per-thread sums (Hillis-Steele)
  for (int d = 1; d < RO_T; d <<= 1) {
    const int v = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = t ? part[t - 1] : 0;
  for (int e = e0; e < e1; ++e) {
    offsets[e] = run;
    run += tot[e];
  }
  if (t == RO_T - 1) offsets[experts] = part[RO_T - 1];
}

// One wave per chunk walks its pairs in order, 64 at a time.  The lanes
// holding the same expert v form a ballot mask; their rows are
// offsets[v] + (pairs of v before this chunk and before these 64 pairs)
// + the lane's rank in the mask, so every expert's pairs keep their flat
// order.  hist[c][v] (the count before this chunk) advances by the mask's
// popcount as the chunk proceeds; only this wave touches row c.
__global__ __launch_bounds__(64) void k_route_assign(const int32_t* __restrict__ ids, int npairs, int topk, int experts,
                                                     int ch, const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ hist, int32_t* __restrict__ dest_row,
                                                     int32_t* __restrict__ src_token) {
  const int c = blockIdx.x, lane = threadIdx.x;
  int32_t* row = hist + (size_t)c * experts;
  const int64_t p0 = (int64_t)c * ch, p1 = min((int64_t)npairs, p0 + ch);
  for (int64_t q = p0; q < p1; q += 64) {
    const int64_t p = q + lane;
    const bool in = p < p1;
    const int e = in ? ids[p] : -1;
    const bool valid = in && e >= 0 && e < experts;
    if (in && !valid) dest_row[p] = -1;
    uint64_t todo = __ballot(valid);
    while (todo) {
      const int leader = __builtin_ctzll(todo);
      const int v = __shfl(e, leader, 64);
      const uint64_t mask = __ballot(valid && e == v);
      int before = 0;
      if (lane == leader) before = atomicAdd(&row[v], __popcll(mask));
      before = __shfl(before, leader, 64);
      if ((mask >> lane) & 1) {
        const int r = offsets[v] + before + __popcll(mask & ((uint64_t(1) << lane) - 1));
        dest_row[p] = r;
        src_token[r] = (int)(p / topk);
      }
      todo &= ~mask;
    }
  }
}

size_t route_workspace_bytes(int experts) {
  return ((size_t)experts + (size_t)route_max_chunks(experts) * experts) * sizeof(int32_t);
}

hipError_t launch_moe_route(const int32_t* ids, int64_t npairs, int topk, int experts, int32_t* offsets,
                            int32_t* dest_row, int32_t* src_token, int32_t* ws, hipStream_t st) {
  const int np = (int)npairs;
  int chunks = 0, ch = 64;
  if (np > 0) {
    chunks = (int)std::min<int64_t>((npairs + kRouteChunkMin - 1) / kRouteChunkMin, route_max_chunks(experts));
    ch = (int)(((npairs + chunks - 1) / chunks + 63) / 64 * 64);
    chunks = (int)((npairs + ch - 1) / ch);
  }
  int32_t* tot = ws;
  int32_t* hist = ws + experts;
  if (chunks > 0) hipLaunchKernelGGL(k_route_hist, dim3(chunks), dim3(RT), 0, st, ids, np, experts, ch, hist);
  hipLaunchKernelGGL(k_route_colscan, dim3((experts + RT - 1) / RT), dim3(RT), 0, st, chunks, experts, hist, tot);
  hipLaunchKernelGGL(k_route_offsets, dim3(1), dim3(RO_T), 0, st, experts, tot, offsets);
  if (chunks > 0)
    hipLaunchKernelGGL(k_route_assign, dim3(chunks), dim3(64), 0, st, ids, np, topk, experts, ch, offsets, hist,
                       dest_row, src_token);
  return hipGetLastError();
}

// out[t, n] = sum_s w[t, s] * y[dest_row[t, s], n] in fp32, slots in order;
// a pair whose row is outside [0, y_rows) contributes nothing.  A thread owns
// 8 consecutive columns of one token.
template <bool Y_BF16, bool O_BF16>
__global__ __launch_bounds__(256) void k_moe_combine(const void* __restrict__ y, int64_t ldy, int64_t y_rows,
                                                     const int32_t* __restrict__ dest_row, const float* __restrict__ w,
                                                     int64_t tokens, int topk, int64_t N, void* __restrict__ out,
                                                     int64_t ldo) {
  const int64_t vpr = N / 8;
  const int64_t total = tokens * vpr;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < total; v += (int64_t)gridDim.x * 256) {
    const int64_t t = v / vpr, c = (v - t * vpr) * 8;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int s = 0; s < topk; ++s) {
      const int32_t r = dest_row[t * topk + s];
      if (r < 0 || r >= y_rows) continue;
      const float ws = w[t * topk + s];
      if (Y_BF16) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(y) + (size_t)r * ldy + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = __builtin_fmaf(ws, bf16_lo(q[i]), acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(ws, bf16_hi(q[i]), acc[2 * i + 1]);
        }
      } else {
        const float* src = reinterpret_cast<const float*>(y) + (size_t)r * ldy + c;
        const f32x4 a = *reinterpret_cast<const f32x4*>(src), b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] = __builtin_fmaf(ws, a[i], acc[i]);
          acc[4 + i] = __builtin_fmaf(ws, b[i], acc[4 + i]);
        }
      }
    }
    if (O_BF16) {
      const u32x4 o = {pack_bf16x2_rne(acc[0], acc[1]), pack_bf16x2_rne(acc[2], acc[3]),
                       pack_bf16x2_rne(acc[4], acc[5]), pack_bf16x2_rne(acc[6], acc[7])};
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * ldo + c) = o;
    } else {
      float* dst = reinterpret_cast<float*>(out) + (size_t)t * ldo + c;
      *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
  }
}

hipError_t launch_moe_combine(const void* y, int y_bf16, int64_t ldy, int64_t y_rows, const int32_t* dest_row,
                              const float* w, int64_t tokens, int topk, int64_t N, void* out, int o_bf16, int64_t ldo,
                              hipStream_t st) {
  const int64_t total = tokens * (N / 8);
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 256 * 16) grid = 256 * 16;
#define MX_CMB(YB, OB)                                                                                         \
  hipLaunchKernelGGL((k_moe_combine<YB, OB>), dim3((unsigned)grid), dim3(256), 0, st, y, ldy, y_rows, dest_row, \
                     w, tokens, topk, N, out, ldo)
  if (y_bf16 && o_bf16) MX_CMB(true, true);
  else if (y_bf16) MX_CMB(true, false);
  else if (o_bf16) MX_CMB(false, true);
  else MX_CMB(false, false);
#undef MX_CMB
  return hipGetLastError();
}

}  // namespace mxk
