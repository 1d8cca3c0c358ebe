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
#include "mx_device.h"
#include "mx_kernels.h"

namespace mxk {

constexpr int RT = 256;   // threads per workgroup of the routing kernels

// Workgroup g counts the pairs routed to expert g.
__global__ __launch_bounds__(RT) void k_route_count(const int32_t* __restrict__ ids, int npairs, int32_t* __restrict__ cnt) {
  __shared__ int red[RT / 64];
  const int g = blockIdx.x;
  int c = 0;
  for (int p = threadIdx.x; p < npairs; p += RT) c += ids[p] == g;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) c += __shfl_xor(c, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < RT / 64; ++w) t += red[w];
    cnt[g] = t;
  }
}

// Workgroup g < experts: offsets[g] = sum of the counts before g, then the
// pairs of expert g in flat order get rows offsets[g], offsets[g] + 1, ...
// (chunks of 256 pairs; a pair's rank inside a chunk is a ballot popcount
// plus the counts of the waves before it).  Workgroup `experts` marks pairs
// whose expert id is out of range with row -1 and writes offsets[experts].
__global__ __launch_bounds__(RT) void k_route_assign(const int32_t* __restrict__ ids, int npairs, int topk, int experts,
                                                     const int32_t* __restrict__ cnt, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token) {
  __shared__ int wsum[RT / 64];
  __shared__ int base_sh;
  const int g = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (g == experts) {
    int total = 0;
    for (int e = 0; e < experts; ++e) total += cnt[e];
    if (tid == 0) offsets[experts] = total;
    for (int p = tid; p < npairs; p += RT) {
      const int e = ids[p];
      if (e < 0 || e >= experts) dest_row[p] = -1;
    }
    return;
  }
  if (tid == 0) {
    int off = 0;
    for (int e = 0; e < g; ++e) off += cnt[e];
    base_sh = off;
    offsets[g] = off;
  }
  __syncthreads();
  int base = base_sh;
  for (int p0 = 0; p0 < npairs; p0 += RT) {
    const int p = p0 + tid;
    const bool hit = p < npairs && ids[p] == g;
    const uint64_t bal = __ballot(hit);
    const int before = __popcll(bal & ((uint64_t(1) << lane) - 1));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < RT / 64; ++w) {
      woff += w < wave ? wsum[w] : 0;
      tot += wsum[w];
    }
    if (hit) {
      const int row = base + woff + before;
      dest_row[p] = row;
      src_token[row] = p / topk;
    }
    base += tot;
    __syncthreads();   // wsum is rewritten by the next chunk
  }
}

hipError_t launch_moe_route(const int32_t* ids, int64_t npairs, int topk, int experts, int32_t* offsets,
                            int32_t* dest_row, int32_t* src_token, int32_t* cnt, hipStream_t st) {
  hipLaunchKernelGGL(k_route_count, dim3(experts), dim3(RT), 0, st, ids, (int)npairs, cnt);
  hipLaunchKernelGGL(k_route_assign, dim3(experts + 1), dim3(RT), 0, st, ids, (int)npairs, topk, experts, cnt, offsets,
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
