// RMSNorm fused with block-scaled FP4 quantization of its output, for gfx950.
//
// Dynamic activation quantization costs a pass over the activations at every
// layer ("NVFP4 Architecture", section "The Problem": the re-quantization
// overhead of prior formats); doing it in the epilogue of the producing
// normalization removes that pass (RMSNorm is among the operations of an
// MXFP4 serving stack: "MXFP4" card, section "Core Facts").  With a static
// (calibrated) per-tensor scale, NVFP4 needs no tensor-wide max either.
//
// Definition (fixed so that the codes are reproducible bit for bit):
//   s   = sum of x_k^2 in fp32 -- thread t owns the 32-element chunks
//         t, t + 256, ... of the row and adds their squares in element order
//         (bf16 squares are exact in fp32); the 256 partial sums are added as
//         a pairwise tree over thread index (within each wave of 64, then
//         (w0 + w1) + (w2 + w3));
//   r   = fp32(1 / sqrt(s / K + eps)), evaluated in fp64;
//   y_k = fp32(fp32(x_k * r) * gamma_k);
//   y is then quantized exactly as mx_quantize quantizes an fp32 tensor
//   (MXFP4, or NVFP4 with the caller's per-tensor scale).
// A workgroup walks rows with the next row's loads in flight; a row is read
// with coalesced loads, reaches its chunk-owning threads through LDS and stays
// in registers between the two passes; gamma is loaded once per workgroup.
#include "mx_device.h"
#include "nv_codes.h"
#include "mx_kernels.h"

namespace mxk {

constexpr int NQ_T = 256;

constexpr int NQ_MAXCH = 4;   // chunks of 32 per thread: K <= 256 * 32 * 4

template <bool NV, bool G_BF16, int CH>
__global__ __launch_bounds__(NQ_T) void k_rmsnorm_quant(const uint16_t* __restrict__ x, int64_t ldx, int64_t rows, int K,
                                                        const void* __restrict__ gamma, float eps,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                        const float* __restrict__ gscale) {
  static_assert(CH >= 1 && CH <= NQ_MAXCH, "chunks per thread");
  constexpr int GV = G_BF16 ? 4 : 8;               // 16-byte gamma vectors per 32-element chunk
  __shared__ float wsum[NQ_T / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = K / 32;
  const float g = NV ? *gscale : 1.0f;
  const double six_g = 6.0 * (double)g;
  // Loads are buffer loads whose out-of-range offsets (chunks past the row)
  // return zeros, so none is conditional and the counted waits below are exact.
  constexpr uint32_t FAR = 0x40000000u;
  auto chunk_off = [&](int j) -> uint32_t {
    const int c = tid + j * NQ_T;
    return c < nch ? (uint32_t)c * 64 : FAR;       // 32 bf16 = 64 bytes per chunk
  };
  // gamma of this thread's chunks, the same for every row: loaded once
  u32x4 gm[CH][GV];
  {
    const __amdgpu_buffer_rsrc_t rg =
        __builtin_amdgcn_make_buffer_rsrc((void*)gamma, 0, K * (G_BF16 ? 2 : 4), 0x00020000);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t o = chunk_off(j) * (G_BF16 ? 1 : 2);
#pragma unroll
      for (int q = 0; q < GV; ++q)
        gm[j][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, o + q * 16, 0, 0));
    }
  }
  // Row loads are coalesced: load s of thread t is the row's 16-byte vector
  // 256 s + t, so each load instruction reads 1 KiB of contiguous memory.
  // The vectors reach their chunk's thread through LDS (piece p of chunk c
  // in slot 4 c + (p ^ ((c >> 2) & 3)), conflict-free for both sides).  Two
  // register sets alternate: while one row is staged, reduced and coded, the
  // next row's loads are in flight in the other.
  __shared__ u32x4 stage[NQ_T * CH * 4];
  auto slot = [](int c, int p) { return 4 * c + (p ^ ((c >> 2) & 3)); };
  auto load_row = [&](u32x4 (&dst)[CH * 4], int64_t row) {
    // rows past the end load zeros (an empty range)
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + (size_t)(row < rows ? row : 0) * ldx), 0, row < rows ? K * 2 : 0, 0x00020000);
#pragma unroll
    for (int v = 0; v < CH * 4; ++v) {
      const int vec = v * NQ_T + tid;
      dst[v] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, vec < nch * 4 ? (uint32_t)vec * 16 : FAR, 0, 2));
    }
  };
  u32x4 xa[CH * 4], xb[CH * 4];
  auto do_row = [&](const u32x4 (&cur)[CH * 4], u32x4 (&nxt)[CH * 4], int64_t row) {
    load_row(nxt, row + gridDim.x);
    wait_vmcnt<CH * 4>();                          // this row (and gamma) landed; the next is in flight
#pragma unroll
    for (int v = 0; v < CH * 4; ++v) {
      const int vec = v * NQ_T + tid;
      stage[slot(vec >> 2, vec & 3)] = cur[v];
    }
    __syncthreads();
    u32x4 xv[CH][4];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = tid + j * NQ_T;
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[j][q] = stage[slot(c, q)];
    }
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {              // chunks past the row are zeros
          const float a = bf16_lo(xv[j][q][i]), b = bf16_hi(xv[j][q][i]);
          part = part + a * a;
          part = part + b * b;
        }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) part = fadd_xor(part, m);
    if (lane == 0) wsum[wave] = part;
    // (the stage reads above finished before the sums used them, so after this
    // barrier the stage may be rewritten; wsum is rewritten only after the next
    // row's first barrier, which every thread reaches after reading it)
    __syncthreads();
    const float total = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    const float r = (float)(1.0 / sqrt((double)total / (double)K + (double)eps));
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = tid + j * NQ_T;
      if (c >= nch) continue;
      float y[32];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float gf[8];
        if (G_BF16) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            gf[2 * i] = bf16_lo(gm[j][q][i]);
            gf[2 * i + 1] = bf16_hi(gm[j][q][i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            gf[i] = ffrom(gm[j][2 * q][i]);
            gf[4 + i] = ffrom(gm[j][2 * q + 1][i]);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = bf16_lo(xv[j][q][i]) * r, b = bf16_hi(xv[j][q][i]) * r;
          y[q * 8 + 2 * i] = a * gf[2 * i];
          y[q * 8 + 2 * i + 1] = b * gf[2 * i + 1];
        }
      }
      uint8_t* crow = codes + (size_t)row * (K / 2) + c * 16;
      if (!NV) {
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) am = max(am, fbits(y[i]) & 0x7fffffffu);
        const int e = mx_block_exp(am);
        const float s = pow2f(e);
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t o = 0;
          o = cvt_fp4x2<0>(o, y[q * 8 + 0], y[q * 8 + 1], s);
          o = cvt_fp4x2<1>(o, y[q * 8 + 2], y[q * 8 + 3], s);
          o = cvt_fp4x2<2>(o, y[q * 8 + 4], y[q * 8 + 5], s);
          o = cvt_fp4x2<3>(o, y[q * 8 + 6], y[q * 8 + 7], s);
          w[q] = o;
        }
        *reinterpret_cast<u32x4*>(crow) = u32x4{w[0], w[1], w[2], w[3]};
        scales[(size_t)row * (K / 32) + c] = (uint8_t)(e + 127);
      } else {
        uint32_t w[4];
        uint32_t sc2 = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {          // two 16-element NVFP4 blocks
          uint32_t am = 0;
#pragma unroll
          for (int i = 0; i < 16; ++i) am = max(am, fbits(y[h * 16 + i]) & 0x7fffffffu);
          const uint32_t sc = e4m3_rne_sat((double)ffrom(am) / six_g);
          const double unit = (double)e4m3_to_f32(sc) * (double)g;
          uint32_t yb[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) yb[i] = fbits(y[h * 16 + i]);
          const NvFast nf = nv_fast_setup(unit, am);
          const bool f0 = nv_fast_codes8(yb, nf, w[h * 2]), f1 = nv_fast_codes8(yb + 8, nf, w[h * 2 + 1]);
          if (!(nf.ok && f0 && f1)) {          // an element within 2^-20 of a boundary: exact test
            uint32_t U[7];
            nv_boundaries(unit, U);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              uint32_t o = 0;
#pragma unroll
              for (int i = 0; i < 8; ++i) o |= nv_code_sel(yb[q * 8 + i], U) << (4 * i);
              w[h * 2 + q] = o;
            }
          }
          sc2 |= sc << (8 * h);
        }
        *reinterpret_cast<u32x4*>(crow) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<uint16_t*>(scales + (size_t)row * (K / 16) + c * 2) = (uint16_t)sc2;
      }
    }
  };
  load_row(xa, blockIdx.x);
  for (int64_t row = blockIdx.x; row < rows; row += 2 * (int64_t)gridDim.x) {
    do_row(xa, xb, row);
    if (row + gridDim.x >= rows) break;
    do_row(xb, xa, row + gridDim.x);
  }
}

hipError_t launch_rmsnorm_quant(const void* x, int64_t ldx, int64_t rows, int64_t K, const void* gamma, int g_bf16,
                                float eps, bool nv, uint8_t* codes, uint8_t* scales, const float* gscale,
                                hipStream_t st) {
  if (rows == 0) return hipSuccess;
  // about two resident workgroups per CU, each walking many rows with the next
  // row in flight
  const int grid = (int)(rows < 256 * 2 ? rows : 256 * 2);
#define MX_RNQ3(NVB, GB, C)                                                                                        \
  hipLaunchKernelGGL((k_rmsnorm_quant<NVB, GB, C>), dim3(grid), dim3(NQ_T), 0, st, (const uint16_t*)x, ldx, rows, \
                     (int)K, gamma, eps, codes, scales, gscale)
#define MX_RNQ(NVB, GB) \
  if (ch <= 1) MX_RNQ3(NVB, GB, 1); else if (ch <= 2) MX_RNQ3(NVB, GB, 2); else MX_RNQ3(NVB, GB, 4)
  // registers for the row: the fewest chunks per thread that cover it
  const int64_t ch = (K / 32 + NQ_T - 1) / NQ_T;
  if (nv) {
    if (g_bf16) { MX_RNQ(true, true); } else { MX_RNQ(true, false); }
  } else {
    if (g_bf16) { MX_RNQ(false, true); } else { MX_RNQ(false, false); }
  }
#undef MX_RNQ3
#undef MX_RNQ
  return hipGetLastError();
}

}  // namespace mxk
