// W4A16 decode GEMV / skinny GEMM for gfx950: y[m, n] = sum_k x[m, k] W_hat[n, k]
// with bf16 activations and MXFP4 weights (weights compressed, arithmetic in
// 16-bit: "Extreme Quantization and Precision Engineering", section "Key
// points"; decode is bound by streaming weight bytes: "NVFP4 Architecture",
// section "The Problem", and the same page's "Hardware-Managed Tensor Core
// Dot-Products" for why 4-bit weights halve those bytes).
//
// The weights are streamed once from HBM and dequantized in registers; the
// matrix cores are not used.  Each lane owns one 32-element MX block (16
// bytes of codes + its E8M0 byte) of R rows at a time.  The 16 code bytes
// expand with v_cvt_scalef32_pk_bf16_fp4 into 32 bf16 weights equal to
// q * 2^e exactly (2 significant bits), and v_dot2_f32_bf16 multiplies pairs
// of them with the matching bf16 activation pairs into fp32 accumulators.
// The activations are staged in LDS (all M rows, a K chunk at a time) and
// read once per block for all R rows.  At the end every wave reduces its
// R x M partial sums across the 64 lanes.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mxk {

constexpr int GV_T = 256;              // 4 waves
constexpr int GV_R = 4;                // weight rows per wave
constexpr int GV_LDS = 64 * 1024;      // bytes of activations staged per chunk
constexpr int GV_WIN = 64 * 32;        // K elements per wave step (64 lanes x 1 block)

template <int M>
__global__ __launch_bounds__(GV_T) void k_gemv(const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wc,
                                               const uint8_t* __restrict__ ws, int N, int K,
                                               uint16_t* __restrict__ y, int64_t ldy) {
  constexpr int KC_MAX = GV_LDS / (2 * M) / GV_WIN * GV_WIN;  // K elements per staged chunk
  __shared__ __attribute__((aligned(16))) uint16_t sx[M * KC_MAX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = (blockIdx.x * (GV_T / 64) + wave) * GV_R;
  const int KB = K / 2, KS = K / 32;
  const int kc = K < KC_MAX ? K : KC_MAX;

  float acc[GV_R][M];
#pragma unroll
  for (int r = 0; r < GV_R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += kc) {
    const int klen = min(kc, K - k0);
    __syncthreads();
    // stage x[:, k0:k0+klen] (klen % 8 == 0; 16-byte vectors)
    const int vpr = klen / 8;
    for (int v = tid; v < M * vpr; v += GV_T) {
      const int m = v / vpr, c = v - m * vpr;
      *reinterpret_cast<u32x4*>(&sx[m * KC_MAX + c * 8]) =
          *reinterpret_cast<const u32x4*>(x + (size_t)m * ldx + k0 + c * 8);
    }
    __syncthreads();
    for (int w0 = 0; w0 < klen; w0 += GV_WIN) {
      const int kl = w0 + lane * 32;       // lane's block start within the chunk
      const bool kok = kl < klen;
      const int kb = (k0 + kl) / 32;       // global block index
      u32x4 cw[GV_R];
      uint32_t se[GV_R];
#pragma unroll
      for (int r = 0; r < GV_R; ++r) {
        const int n = n0 + r;
        const bool ok = kok && n < N;
        cw[r] = ok ? *reinterpret_cast<const u32x4*>(wc + (size_t)n * KB + (size_t)kb * 16) : u32x4{0, 0, 0, 0};
        se[r] = ok ? ws[(size_t)n * KS + kb] : 127u;
      }
      if (!kok) continue;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        u32x4 xv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[q] = *reinterpret_cast<const u32x4*>(&sx[m * KC_MAX + kl + q * 8]);
#pragma unroll
        for (int r = 0; r < GV_R; ++r) {
          const float s = pow2f((int)se[r] - 127);
          float a = acc[r][m];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t c = cw[r][q];   // 8 codes = elements 8q .. 8q+7 of the block
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              bf16x2 wv;
              switch (b) {
                case 0: wv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 0); break;
                case 1: wv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 1); break;
                case 2: wv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 2); break;
                default: wv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 3); break;
              }
              bf16x2 xx;
              const uint32_t xw = xv[q][b];
              __builtin_memcpy(&xx, &xw, 4);
              a = __builtin_amdgcn_fdot2_f32_bf16(wv, xx, a, false);
            }
          }
          acc[r][m] = a;
        }
      }
    }
  }
  // reduce across the wave; lane 0 writes
#pragma unroll
  for (int r = 0; r < GV_R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[r][m];
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) v = fadd_xor(v, msk);
      if (lane == 0 && n0 + r < N) y[(size_t)m * ldy + n0 + r] = (uint16_t)f32_to_bf16_rne(v);
    }
}

hipError_t launch_gemv(const void* x, int64_t ldx, int64_t M, const uint8_t* wc, const uint8_t* ws, int64_t N,
                       int64_t K, void* y, int64_t ldy, hipStream_t st) {
  const int grid = (int)((N + (GV_T / 64) * GV_R - 1) / ((GV_T / 64) * GV_R));
  if (grid == 0) return hipSuccess;
#define MX_GV(MM) case MM: hipLaunchKernelGGL((k_gemv<MM>), dim3(grid), dim3(GV_T), 0, st, (const uint16_t*)x, ldx, wc, ws, (int)N, (int)K, (uint16_t*)y, ldy); break;
  switch ((int)M) {
    MX_GV(1) MX_GV(2) MX_GV(3) MX_GV(4) MX_GV(5) MX_GV(6) MX_GV(7) MX_GV(8)
    MX_GV(9) MX_GV(10) MX_GV(11) MX_GV(12) MX_GV(13) MX_GV(14) MX_GV(15) MX_GV(16)
    default: return hipErrorInvalidValue;
  }
#undef MX_GV
  return hipGetLastError();
}

}  // namespace mxk
