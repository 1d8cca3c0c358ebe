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

constexpr int RT = 256;   // threads per workgroup of the counting kernel

// The pairs are cut into C chunks of `ch` consecutive pairs (ch a multiple of
// 64, at least kRouteChunk unless there are fewer pairs), with
// C * experts <= kRouteTable, so that the per-chunk counts fit a workspace
// whose size depends on the expert count only.  Each pass is linear in the
// pairs plus C * experts: per-chunk counts, one scan over the counts, one
// assignment pass over the pairs.  Counts live in LDS for up to
// kRouteLdsExperts experts (global atomics beyond).
constexpr int kRouteTable = 1 << 16;
constexpr int kRouteChunk = 256;
constexpr int kRouteLdsExperts = 8192;

int route_max_chunks(int experts) { return experts >= kRouteTable ? 1 : kRouteTable / experts; }

// Workgroup c: hist[c][e] = pairs of chunk c routed to expert e.
template <bool LDS>
__global__ __launch_bounds__(RT) void k_route_hist(const int32_t* __restrict__ ids, int npairs, int experts, int ch,
                                                   int32_t* __restrict__ hist) {
  __shared__ int cnt[LDS ? kRouteLdsExperts : 1];
  const int c = blockIdx.x;
  int32_t* row = hist + (size_t)c * experts;
  int* ctr = LDS ? cnt : row;
  for (int e = threadIdx.x; e < experts; e += RT) ctr[e] = 0;
  if (!LDS) __threadfence();   // the zeros are in memory before any lane's increment
  __syncthreads();
  const int64_t p0 = (int64_t)c * ch, p1 = min((int64_t)npairs, p0 + ch);
  for (int64_t p = p0 + threadIdx.x; p < p1; p += RT) {
    const int e = ids[p];
    if (e >= 0 && e < experts) atomicAdd(&ctr[e], 1);
  }
  if (LDS) {
    __syncthreads();
    for (int e = threadIdx.x; e < experts; e += RT) row[e] = cnt[e];
  }
}

// One workgroup: exclusive prefix of the counts taken expert by expert and,
// within an expert, chunk by chunk; hist[c][e] becomes the first row of the
// pairs of expert e in chunk c, offsets[e] the first row of expert e, and
// offsets[experts] the number of routed pairs.
constexpr int RS_T = 1024;
__global__ __launch_bounds__(RS_T) void k_route_scan(int chunks, int experts, int32_t* __restrict__ hist,
                                                     int32_t* __restrict__ offsets) {
  __shared__ int part[RS_T];
  const int t = threadIdx.x;
  const int n = chunks * experts;
  if (n == 0) {   // no pairs: every expert is empty
    for (int e = t; e <= experts; e += RS_T) offsets[e] = 0;
    return;
  }
  const int per = (n + RS_T - 1) / RS_T;
  const int i0 = min(n, t * per), i1 = min(n, i0 + per);
  auto at = [&](int i) -> int32_t& { return hist[(size_t)(i % chunks) * experts + i / chunks]; };   // i = e * C + c
  int s = 0;
  for (int i = i0; i < i1; ++i) s += at(i);
  part[t] = s;
  __syncthreads();
  for (int d = 1; d < RS_T; d <<= 1) {   // inclusive scan of the per-thread sums
    const int v = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = t ? part[t - 1] : 0;
  for (int i = i0; i < i1; ++i) {
    const int h = at(i);
    at(i) = run;
    if (i % chunks == 0) offsets[i / chunks] = run;
    run += h;
  }
  if (t == RS_T - 1) offsets[experts] = part[RS_T - 1];
}

// One wave per chunk walks its pairs in order, 64 at a time.  The lanes
// holding the same expert v form a ballot mask; their rows are the next
// free row of v in this chunk plus the lane's rank in the mask, so every
// expert's pairs keep their flat order.  The chunk's next free rows start
// from the scanned counts and advance by the masks' popcounts (in LDS, or
// in the chunk's own workspace row with atomics beyond kRouteLdsExperts
// experts).
template <bool LDS>
__global__ __launch_bounds__(64) void k_route_assign(const int32_t* __restrict__ ids, int npairs, int topk, int experts,
                                                     int ch, int32_t* __restrict__ hist, int32_t* __restrict__ dest_row,
                                                     int32_t* __restrict__ src_token) {
  __shared__ int nxt[LDS ? kRouteLdsExperts : 1];
  const int c = blockIdx.x, lane = threadIdx.x;
  int32_t* row = hist + (size_t)c * experts;
  if (LDS) {
    for (int e = lane; e < experts; e += 64) nxt[e] = row[e];
    __syncthreads();
  }
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
      int first = 0;
      if (lane == leader) {
        if (LDS) {
          first = nxt[v];
          nxt[v] = first + __popcll(mask);
        } else {
          first = atomicAdd(&row[v], __popcll(mask));
        }
      }
      first = __shfl(first, leader, 64);
      if ((mask >> lane) & 1) {
        const int r = first + __popcll(mask & ((uint64_t(1) << lane) - 1));
        dest_row[p] = r;
        src_token[r] = (int)(p / topk);
      }
      todo &= ~mask;
    }
  }
}

size_t route_workspace_bytes(int experts) {
  return (size_t)route_max_chunks(experts) * experts * sizeof(int32_t);
}

hipError_t launch_moe_route(const int32_t* ids, int64_t npairs, int topk, int experts, int32_t* offsets,
                            int32_t* dest_row, int32_t* src_token, int32_t* ws, hipStream_t st) {
  const int np = (int)npairs;
  int chunks = 0, ch = 64;
  if (np > 0) {
    chunks = (int)std::min<int64_t>((npairs + kRouteChunk - 1) / kRouteChunk, route_max_chunks(experts));
    ch = (int)(((npairs + chunks - 1) / chunks + 63) / 64 * 64);
    chunks = (int)((npairs + ch - 1) / ch);
  }
  const bool lds = experts <= kRouteLdsExperts;
  if (chunks > 0) {
    if (lds) hipLaunchKernelGGL(k_route_hist<true>, dim3(chunks), dim3(RT), 0, st, ids, np, experts, ch, ws);
    else hipLaunchKernelGGL(k_route_hist<false>, dim3(chunks), dim3(RT), 0, st, ids, np, experts, ch, ws);
  }
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(RS_T), 0, st, chunks, experts, ws, offsets);
  if (chunks > 0) {
    if (lds)
      hipLaunchKernelGGL(k_route_assign<true>, dim3(chunks), dim3(64), 0, st, ids, np, topk, experts, ch, ws, dest_row,
                         src_token);
    else
      hipLaunchKernelGGL(k_route_assign<false>, dim3(chunks), dim3(64), 0, st, ids, np, topk, experts, ch, ws,
                         dest_row, src_token);
  }
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
