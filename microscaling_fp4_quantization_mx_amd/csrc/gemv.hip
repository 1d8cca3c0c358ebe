// W4A16 decode GEMV / skinny GEMM for gfx950: y[m, n] = sum_k x[m, k] W_hat[n, k]
// with bf16 activations and MXFP4 weights (weights compressed, arithmetic in
// 16-bit: "Extreme Quantization and Precision Engineering", section "Key
// points"; decode is bound by streaming weight bytes: "NVFP4 Architecture",
// section "The Problem").
//
// The weights are streamed once from HBM and dequantized in registers; the
// matrix cores are not used.  A lane owns one 32-element MX block of a weight
// row per 2048-element window of K (64 lanes x 32): its 16 code bytes expand
// with v_cvt_scalef32_pk_bf16_fp4 into 32 bf16 weights equal to q * 2^e
// exactly (at most 2 significant bits), and v_dot2_f32_bf16 multiplies pairs
// of them with the matching bf16 activation pairs into fp32 accumulators, so
// every product is exact and only the fp32 summation order differs from the
// plain definition.  Partial sums are reduced across the 64 lanes at the end.
//
// Two kernels:
//  * M <= 4 is bound by HBM: many small workgroups, split-K across waves.
//  * M >= 5 is bound by the VALU (one dot2 per weight pair and activation
//    row): each weight pair is converted once and used for all M rows, and
//    the activations come from LDS, staged once per workgroup and window.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mxk {

// Weight codes and scales are read once per call: non-temporal loads (cache
// policy bit NT) keep the weight stream from displacing the activations.
constexpr int GV_NT = 2;

constexpr int GV_T = 256;              // 4 waves
constexpr int GV_WIN = 64 * 32;        // K elements per window (64 lanes x 1 block)
constexpr int GV_SK_RB = 4;            // weight rows per workgroup of the small-M kernel

// Sum each of V values (V a power of two, at most 64) over the 64 lanes of a
// wave with V - 1 + (6 - log2 V) * 1 exchanges instead of 6 V: at each of
// the first log2 V steps a lane keeps half of its values, sends the other
// half to its partner (lane ^ mask) and adds what it receives.  Afterwards
// lane l holds the partial sum of value index sum_t bit(l, 5 - t) * 2^t over
// the lanes that share its top log2 V bits; plain xor steps finish the sum.
// Returns that total; *idx receives the value index.
template <int V>
__device__ __forceinline__ float wave_transpose_sum(float (&v)[V], int lane, int* idx) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
  int id = 0;
  int n = V;
#pragma unroll
  for (int t = 0; (1 << t) < V; ++t) {
    const int mask = 32 >> t;
    const bool hi = (lane & mask) != 0;
    id |= (hi ? 1 : 0) << t;
    n >>= 1;
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      if (i < n) {
        const float send = hi ? v[2 * i] : v[2 * i + 1];
        const float keep = hi ? v[2 * i + 1] : v[2 * i];
        v[i] = keep + __shfl_xor(send, mask, 64);
      }
    }
  }
  float r = v[0];
#pragma unroll
  for (int mask = 32 / V; mask >= 1; mask >>= 1) r += __shfl_xor(r, mask, 64);
  *idx = id;
  return r;
}

// Small M (memory-bound): split-K inside the workgroup.  A workgroup owns RB
// weight rows; its four waves take the 2048-element windows of K in turn
// (wave w: windows w, w+4, ...), so each wave streams RB x 1 KiB of codes per
// window while reading only its own 4 KiB slice of each activation row.  The
// loads of a window go out in the order they are consumed (scale bytes,
// activations, codes) so the counted waits let arithmetic start on the first
// row while later rows are still in flight.  The four per-wave partial sums
// of every output meet in LDS at the end.
template <int M, int RB>
__global__ __launch_bounds__(GV_T) void k_gemv_sk(const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wc,
                                                  const uint8_t* __restrict__ ws, int N, int K,
                                                  uint16_t* __restrict__ y, int64_t ldy) {
  __shared__ float red[GV_T / 64][RB * M];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * RB;                 // < N: the grid is ceil(N / RB)
  const int KB = K / 2, KS = K / 32;
  const int rows_ok = __builtin_amdgcn_readfirstlane(min(RB, N - n0));
  const __amdgpu_buffer_rsrc_t rwc = __builtin_amdgcn_make_buffer_rsrc((void*)(wc + (size_t)n0 * KB), 0, rows_ok * KB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc((void*)(ws + (size_t)n0 * KS), 0, rows_ok * KS, 0x00020000);
  const int nwin = (K + GV_WIN - 1) / GV_WIN;

  float acc[RB][M];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  for (int win = wave; win < nwin; win += GV_T / 64) {
    const int kb = win * 64 + lane;               // the lane's block of K
    const bool kok = kb < KS;                     // blocks past K read as zero
    uint32_t sc[RB];
    u32x4 xv[M][4], cw[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) sc[r] = __builtin_amdgcn_raw_buffer_load_b8(rws, kok ? r * KS + kb : 0x7ffffff0, 0, GV_NT);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)(x + (size_t)m * ldx), 0, K * 2, 0x00020000);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[m][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, kok ? kb * 64 + q * 16 : 0x7ffffff0, 0, 0));
    }
#pragma unroll
    for (int r = 0; r < RB; ++r)
      cw[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwc, kok ? r * KB + kb * 16 : 0x7ffffff0, 0, GV_NT));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const float s = pow2f((int)sc[r] - 127);   // byte 0 (zero block past K) gives +0.0
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t c = cw[r][q];              // 8 codes = elements 8q .. 8q+7 of the block
        bf16x2 wv[4];
        wv[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 0);
        wv[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 1);
        wv[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 2);
        wv[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 3);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float a = acc[r][m];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t xj = xv[m][q][j];
            bf16x2 xp;
            __builtin_memcpy(&xp, &xj, 4);
            a = __builtin_amdgcn_fdot2_f32_bf16(wv[j], xp, a, false);
          }
          acc[r][m] = a;
        }
      }
    }
  }
  {
    constexpr int V = (RB * M <= 4) ? 4 : (RB * M <= 8) ? 8 : 16;
    static_assert(RB * M <= 16, "at most 16 sums per wave");
    float v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = i < RB * M ? acc[i / M][i % M] : 0.0f;
    int id;
    const float tot = wave_transpose_sum<V>(v, lane, &id);
    if ((lane & (64 / V - 1)) == 0 && id < RB * M) red[wave][id] = tot;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < RB * M) {
    const int r = t / M, m = t - r * M;
    float v = red[0][t];
#pragma unroll
    for (int w = 1; w < GV_T / 64; ++w) v += red[w][t];
    if (n0 + r < N) y[(size_t)m * ldy + n0 + r] = (uint16_t)f32_to_bf16_rne(v);
  }
}

// Larger M (VALU-bound).  A workgroup of 8 waves owns 8 x RB weight rows
// (RB per wave) and walks the windows of K together.  Per window:
//  * the activations of all M rows (M x 4 KiB) are copied into LDS by the
//    LDS-DMA path (buffer_load ... lds), one buffer ahead, in a layout where
//    chunk q (16 bytes) of lane l's block sits at (q * 64 + l) * 16, so the
//    ds_read_b128 of a given q across the wave is conflict-free;
//  * each wave loads its RB code vectors and scale bytes one window ahead;
//  * each lane converts its RB blocks once (RB x 16 bf16 pairs in registers)
//    and then, per activation row m, reads its 64 activation bytes from LDS
//    and issues RB x 16 dot2.
// Two barriers per window: after the counted wait that covers this window's
// copy, and after the arithmetic (before the buffer is refilled).
constexpr int GL_T = 512;              // 8 waves
constexpr int GV_LG_RB = 4;            // weight rows per wave of the large-M kernel
constexpr int GV_LG_MIN_M = 2;         // smallest M that takes the large-M kernel



template <int M, int RB>
__global__ __launch_bounds__(GL_T) void k_gemv_lg(const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wc,
                                                  const uint8_t* __restrict__ ws, int N, int K,
                                                  uint16_t* __restrict__ y, int64_t ldy) {
  constexpr int MP = (M + 1) & ~1;                 // staged rows, even: every wave issues MP / 2 copies
  constexpr int XCH = MP * 4;                      // 1 KiB copies per window (4 per activation row)
  constexpr int XPW = XCH / 8;                     // copies per wave
  __shared__ __attribute__((aligned(16))) uint8_t sx[2][MP * 4096];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * (8 * RB) + wave * RB;
  const int KB = K / 2, KS = K / 32;
  const int nwin = (K + GV_WIN - 1) / GV_WIN;
  const int rows_ok = __builtin_amdgcn_readfirstlane(max(0, min(RB, N - n0)));
  const size_t nb = n0 < N ? (size_t)n0 : 0;
  const __amdgpu_buffer_rsrc_t rwc = __builtin_amdgcn_make_buffer_rsrc((void*)(wc + nb * KB), 0, rows_ok * KB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc((void*)(ws + nb * KS), 0, rows_ok * KS, 0x00020000);
  const int oob = max(0x7ffffff0, KS);             // beyond every range: the load returns zero

  // copy window w of the activations into LDS buffer b
  auto stage = [&](int b, int w) {
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
      const int c = wave * XPW + i;                // uniform
      const int m = c >> 2, q = c & 3;
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(x + (size_t)(m < M ? m : 0) * ldx), 0, m < M ? K * 2 : 0, 0x00020000);
      // LDS chunk q * 64 + lane holds window chunk 4 * lane + q
      const int k = w * GV_WIN + (4 * lane + q) * 8;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(&sx[b][(m * 256 + q * 64) * 16]), 16,
                                               k < K ? k * 2 : oob, 0, 0, 0);
    }
  };
  uint32_t sc[2][RB];
  u32x4 cw[2][RB];
  auto issue = [&](int b, int w) {
    const int kb = w * 64 + lane;
    const bool kok = kb < KS;
#pragma unroll
    for (int r = 0; r < RB; ++r) sc[b][r] = __builtin_amdgcn_raw_buffer_load_b8(rws, kok ? r * KS + kb : oob, 0, GV_NT);
#pragma unroll
    for (int r = 0; r < RB; ++r)
      cw[b][r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwc, kok ? r * KB + kb * 16 : oob, 0, GV_NT));
  };
  constexpr int LOADS = XPW + 2 * RB;              // vector-memory ops per window and wave

  float acc[RB][M];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  auto compute = [&](int b) {
    bf16x2 wv[RB][16];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const float s = pow2f((int)sc[b][r] - 127);   // byte 0 (zero block) gives +0.0
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wv[r][q * 4 + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[b][r][q], s, 0);
        wv[r][q * 4 + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[b][r][q], s, 1);
        wv[r][q * 4 + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[b][r][q], s, 2);
        wv[r][q * 4 + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[b][r][q], s, 3);
      }
    }
    // activation rows one at a time, the next one's LDS reads in flight
    // (the barriers below keep the compiler from hoisting all of them)
    u32x4 xq[2][4];
    auto read_x = [&](int slot, int m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) xq[slot][q] = *reinterpret_cast<const u32x4*>(&sx[b][((m * 256) + q * 64 + lane) * 16]);
    };
    read_x(0, 0);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (m + 1 < M) read_x((m + 1) & 1, m + 1);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float a = acc[r][m];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t xt = xq[m & 1][q][t];
            bf16x2 xp;
            __builtin_memcpy(&xp, &xt, 4);
            a = __builtin_amdgcn_fdot2_f32_bf16(wv[r][q * 4 + t], xp, a, false);
          }
        asm volatile("" : "+v"(a));   // row m's sums are complete here ...
        acc[r][m] = a;
      }
      asm volatile("" ::: "memory");   // ... and later rows' LDS reads stay below
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Windows go in pairs (buffers 0 and 1); a window past the end copies and
  // loads zeros and is computed on zeros, so no load is ever conditional.
  stage(0, 0);
  issue(0, 0);
  for (int w = 0; w < nwin; w += 2) {              // uniform trip count
    stage(1, w + 1);
    issue(1, w + 1);
    wait_vmcnt<LOADS>();                           // window w is in LDS and registers
    block_barrier();
    compute(0);
    block_barrier();                               // buffer 0 is free again
    stage(0, w + 2);
    issue(0, w + 2);
    wait_vmcnt<LOADS>();
    block_barrier();
    compute(1);
    block_barrier();
  }
  wait_vmcnt<0>();

  // reduce the RB x M sums over the wave; lane l ends up owning one of them
  constexpr int V = (RB * M <= 8) ? 8 : (RB * M <= 16) ? 16 : (RB * M <= 32) ? 32 : 64;
  static_assert(RB * M <= 64, "at most 64 sums per wave");
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = i < RB * M ? acc[i / M][i % M] : 0.0f;
  int id;
  const float tot = wave_transpose_sum<V>(v, lane, &id);
  const int r = id / M, m = id - r * M;
  if ((lane & (64 / V - 1)) == 0 && id < RB * M && n0 + r < N)
    y[(size_t)m * ldy + n0 + r] = (uint16_t)f32_to_bf16_rne(tot);
}

hipError_t launch_gemv(const void* x, int64_t ldx, int64_t M, const uint8_t* wc, const uint8_t* ws, int64_t N,
                       int64_t K, void* y, int64_t ldy, hipStream_t st) {
  if (N == 0) return hipSuccess;
  if (M < GV_LG_MIN_M) {
    constexpr int RB = GV_SK_RB;
    const int grid = (int)((N + RB - 1) / RB);
#define MX_GVS(MM) case MM: hipLaunchKernelGGL((k_gemv_sk<MM, RB>), dim3(grid), dim3(GV_T), 0, st, (const uint16_t*)x, ldx, wc, ws, (int)N, (int)K, (uint16_t*)y, ldy); break;
    switch ((int)M) {
      MX_GVS(1) MX_GVS(2) MX_GVS(3) MX_GVS(4)
      default: return hipErrorInvalidValue;
    }
#undef MX_GVS
    return hipGetLastError();
  }
  constexpr int RB = GV_LG_RB;
  const int grid = (int)((N + 8 * RB - 1) / (8 * RB));
#define MX_GVL(MM) case MM: hipLaunchKernelGGL((k_gemv_lg<MM, RB>), dim3(grid), dim3(GL_T), 0, st, (const uint16_t*)x, ldx, wc, ws, (int)N, (int)K, (uint16_t*)y, ldy); break;
  switch ((int)M) {
    MX_GVL(2) MX_GVL(3) MX_GVL(4) MX_GVL(5) MX_GVL(6) MX_GVL(7) MX_GVL(8)
    MX_GVL(9) MX_GVL(10) MX_GVL(11) MX_GVL(12) MX_GVL(13) MX_GVL(14) MX_GVL(15) MX_GVL(16)
    default: return hipErrorInvalidValue;
  }
#undef MX_GVL
  return hipGetLastError();
}

}  // namespace mxk
