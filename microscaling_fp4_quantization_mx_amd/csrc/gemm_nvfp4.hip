// NVFP4 x NVFP4 GEMM for gfx950.
//
// C[m, n] = gA gB sum_b sA[m,b] sB[n,b] sum_{k in b} qA qB over 16-element
// blocks with fp32 accumulation (dual-level scaling, "NVFP4 Architecture",
// section "1. The Dual-Level Mathematical Formulation"; block dot products
// scaled by both block scales, section "2. Hardware-Managed Tensor Core
// Dot-Products").
//
// CDNA4's block-scaled MFMA takes one power-of-two (E8M0) scale per 32 K
// values per lane, which cannot carry an E4M3 scale (3 mantissa bits) per 16
// values.  The block scale is therefore applied to the operands: every code is
// expanded once per workgroup, while staging into LDS, to the fp16 value
// q * s_b, which is exact (q has 2 significant bits, s_b 4, and the product
// lies in [2^-10, 2880], inside fp16's normal range).  Summing these exact
// products in fp32 is the same sum as scaling each 16-element partial sum by
// sA * sB; the two per-tensor scales multiply the fp32 result in the epilogue.
// The expansion uses v_cvt_scalef32_pk_f16_fp4 (exact q * 2^E for the
// exponent of s_b) and one packed fp16 multiply by s_b's significand.
// HBM traffic stays at 4.5 bits per element; the arithmetic runs on the fp16
// matrix cores (v_mfma_f32_32x32x16_f16).
//
// Tiling as in the MXFP4 kernel: 4 waves, 256 x 256 workgroup tile, 128 x 128
// per wave, K = 64 per stage, double-buffered LDS (fp16 rows of 128 B whose
// eight 16-byte chunks are XOR-swizzled), XCD-aware tile order.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mxk {

constexpr int NV_BK = 64;             // K elements per stage (4 NVFP4 blocks)
constexpr int NV_ROWB = NV_BK * 2;    // LDS bytes per fp16 row per stage
constexpr int NV_GROUP_M = 4;

__device__ __forceinline__ int swz8(int row) { return (row & 7) ^ ((row >> 3) & 1); }

struct NvGemmParams {
  const uint8_t* a_codes;  // [M, K/2]
  const uint8_t* a_scales; // [M, K/16] E4M3
  const float* a_global;
  const uint8_t* b_codes;  // [N, K/2]
  const uint8_t* b_scales; // [N, K/16]
  const float* b_global;
  void* c;
  int64_t ldc;
  int M, N, K;
  int c_bf16;
};

// E4M3 byte -> (power of two of its exponent, fp16 significand) with
// s = pow2 * sig exactly: normal 2^(e-7) * (1 + m/8), subnormal 2^-9 * m.
__device__ __forceinline__ void e4m3_split(uint32_t c, float& pow2, _Float16& sig) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e) {
    pow2 = ffrom((e + 120u) << 23);
    sig = (_Float16)(1.0f + (float)m * 0.125f);
  } else {
    pow2 = 0.001953125f;
    sig = (_Float16)(float)m;
  }
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_gemm_nv(NvGemmParams p) {
  constexpr int NWX = BN / WN;
  constexpr int NT = (BM / WM) * NWX * 64;
  constexpr int TI = WM / 32, TJ = WN / 32;
  constexpr int A_CH = BM * 2 / NT;  // 16-byte code chunks (32 elements) per thread per stage
  constexpr int B_CH = BN * 2 / NT;
  static_assert(BM * 2 % NT == 0 && BN * 2 % NT == 0, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * NV_ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * NV_ROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wy = wave / NWX, wx = wave % NWX;

  const int tn_count = (p.N + BN - 1) / BN;
  const int tm_count = (p.M + BM - 1) / BM;
  int tm, tn;
  {
    const int total = tm_count * tn_count;
    const int per_xcd = (total + 7) / 8;
    const int bid = blockIdx.x;
    const int local = bid / 8;
    if (local >= per_xcd) return;
    const int t = (bid % 8) * per_xcd + local;
    if (t >= total) return;
    const int per_group = NV_GROUP_M * tn_count;
    const int grp = t / per_group;
    const int first_m = grp * NV_GROUP_M;
    const int gm = min(tm_count - first_m, NV_GROUP_M);
    const int in_grp = t % per_group;
    tm = first_m + in_grp % gm;
    tn = in_grp / gm;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int KB = p.K / 2, KS = p.K / 16;

  u32x4 ra[A_CH], rb[B_CH];
  uint32_t rsa[A_CH], rsb[B_CH];  // the two E4M3 bytes of each chunk
  auto load_stage = [&](int s) {
    const int kb0 = s * (NV_BK / 2), ks0 = s * 4;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = tid + i * NT, row = q >> 1, seg = q & 1;
      const int gr = m0 + row;
      const bool ok = gr < p.M && kb0 + seg * 16 < KB;
      ra[i] = ok ? *reinterpret_cast<const u32x4*>(p.a_codes + (size_t)gr * KB + kb0 + seg * 16) : u32x4{0, 0, 0, 0};
      const uint8_t* sp = p.a_scales + (size_t)gr * KS + ks0 + seg * 2;
      rsa[i] = ok ? ((uint32_t)sp[0] | ((uint32_t)sp[1] << 8)) : 0u;
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int q = tid + i * NT, row = q >> 1, seg = q & 1;
      const int gr = n0 + row;
      const bool ok = gr < p.N && kb0 + seg * 16 < KB;
      rb[i] = ok ? *reinterpret_cast<const u32x4*>(p.b_codes + (size_t)gr * KB + kb0 + seg * 16) : u32x4{0, 0, 0, 0};
      const uint8_t* sp = p.b_scales + (size_t)gr * KS + ks0 + seg * 2;
      rsb[i] = ok ? ((uint32_t)sp[0] | ((uint32_t)sp[1] << 8)) : 0u;
    }
  };
  // expand 32 codes to 32 exact fp16 values q * s and write 4 swizzled chunks
  auto expand = [&](uint8_t* dst, int row, int seg, const u32x4& w, uint32_t sc2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {        // two 16-element blocks
      float pw;
      _Float16 sg;
      e4m3_split((sc2 >> (8 * h)) & 0xffu, pw, sg);
      const f16x2 sg2 = {sg, sg};
#pragma unroll
      for (int d = 0; d < 2; ++d) {      // two code words per block
        const uint32_t cw = w[h * 2 + d];
        f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, pw, 0) * sg2;
        f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, pw, 1) * sg2;
        f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, pw, 2) * sg2;
        f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, pw, 3) * sg2;
        uint32_t w0, w1, w2, w3;
        __builtin_memcpy(&w0, &v0, 4);
        __builtin_memcpy(&w1, &v1, 4);
        __builtin_memcpy(&w2, &v2, 4);
        __builtin_memcpy(&w3, &v3, 4);
        const u32x4 o = {w0, w1, w2, w3};
        const int c = seg * 4 + h * 2 + d;  // 16-byte chunk (8 fp16) within the 128-byte row
        *reinterpret_cast<u32x4*>(dst + row * NV_ROWB + ((c ^ swz8(row)) << 4)) = o;
      }
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = tid + i * NT;
      expand(sA[buf], q >> 1, q & 1, ra[i], rsa[i]);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int q = tid + i * NT;
      expand(sB[buf], q >> 1, q & 1, rb[i], rsb[i]);
    }
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nstages = (p.K + NV_BK - 1) / NV_BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  const int lrow = lane & 31, khalf = lane >> 5;
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstages) load_stage(s + 1);
#pragma unroll
    for (int kk = 0; kk < NV_BK / 16; ++kk) {
      const int c = kk * 2 + khalf;  // lane holds K = 16*kk + 8*khalf + (0..7)
      f16x8 fa[TI], fb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int row = wy * WM + i * 32 + lrow;
        fa[i] = *reinterpret_cast<const f16x8*>(&sA[buf][row * NV_ROWB + ((c ^ swz8(row)) << 4)]);
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int row = wx * WN + j * 32 + lrow;
        fb[j] = *reinterpret_cast<const f16x8*>(&sB[buf][row * NV_ROWB + ((c ^ swz8(row)) << 4)]);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nstages) store_stage(buf ^ 1);
    __syncthreads();
  }

  const float gg = (*p.a_global) * (*p.b_global);
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = n0 + wx * WN + j * 32 + lrow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wy * WM + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
        if (row < p.M && col < p.N) {
          const float v = acc[i][j][r] * gg;
          if (p.c_bf16)
            reinterpret_cast<uint16_t*>(p.c)[(size_t)row * p.ldc + col] = (uint16_t)f32_to_bf16_rne(v);
          else
            reinterpret_cast<float*>(p.c)[(size_t)row * p.ldc + col] = v;
        }
      }
    }
}

constexpr int NBM = 256, NBN = 256, NWM = 128, NWN = 128;

hipError_t launch_gemm_nv(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                          const uint8_t* b_codes, const uint8_t* b_scales, const float* b_global, void* c, int c_bf16,
                          int64_t ldc, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  NvGemmParams p;
  p.a_codes = a_codes; p.a_scales = a_scales; p.a_global = a_global;
  p.b_codes = b_codes; p.b_scales = b_scales; p.b_global = b_global;
  p.c = c; p.ldc = ldc; p.M = (int)M; p.N = (int)N; p.K = (int)K; p.c_bf16 = c_bf16;
  const int64_t tiles = ((M + NBM - 1) / NBM) * ((N + NBN - 1) / NBN);
  const int64_t grid = (tiles + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  constexpr int NT = (NBM / NWM) * (NBN / NWN) * 64;
  hipLaunchKernelGGL((k_gemm_nv<NBM, NBN, NWM, NWN>), dim3((unsigned)grid), dim3(NT), 0, st, p);
  return hipGetLastError();
}

}  // namespace mxk
