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
#include "gemm_split.h"

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
  // split of the last round along K (k_gemm_nv_k256 only; split_max < 2: none)
  int split_max;
  int cus;                 // workgroup slots of the device (one per CU)
  float* part;             // fp32 partial tiles
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

// ---------------------------------------------------------------------------
// Main path for K % 256 == 0: the operands stay 4-bit in LDS.  Stages of
// K = 256 go HBM -> LDS by the direct-to-LDS path exactly as in the MXFP4
// kernel (128-byte code rows with XOR-swizzled 16-byte chunks) together with
// each row's 16 E4M3 bytes, two slots of 72 KiB.  Every wave then expands its
// own fragments in registers to the exact fp16 values q * s_b right before
// the fp16 MFMAs, so the matrix cores, not LDS bandwidth, set the pace; the
// expansion (two VALU ops per element pair) overlaps the MFMAs.
//
// K order inside a stage: a lane of half h (lanes 32h..32h+31) owns, for the
// K = 64 sub-stage kk, the 32 codes 64kk + 32h .. +31 (one 16-byte chunk, the
// same chunk the MXFP4 kernel feeds to one FP4 MFMA).  The fp16 MFMA
// 32x32x16 takes 8 K values per lane, so dword d of that chunk (codes
// 64kk + 32h + 8d .. +7, NVFP4 block 4kk + 2h + d/2) is one MFMA's operand;
// A and B use the same order, so each MFMA still pairs equal K indices.
//
// One barrier per stage: the counted wait for this stage's loads, the
// barrier (all waves' copies landed, all waves done with the other slot),
// then the next stage's loads into the other slot, interleaved with the
// first sub-stage's MFMAs.
// ---------------------------------------------------------------------------
constexpr int NVK_BK = 256, NVK_BKB = 128, NVK_BKS = 16;

// 8 codes (one dword) -> 8 fp16 values q * s: v_cvt_scalef32_pk_f16_fp4 with
// scale 1 gives q exactly, and one packed multiply by the block scale (an
// E4M3 value, exact in fp16) gives q * s exactly (at most 6 significant bits,
// magnitudes in [2^-10, 2688]).
__device__ __forceinline__ f16x8 nv_expand8(uint32_t w, f16x2 s2) {
  const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_gemm_nv_k256(NvGemmParams p) {
  constexpr int NWX = BN / WN;
  constexpr int TI = WM / 32, TJ = WN / 32;
  static_assert(BM == 256 && BN == 256 && WM == 128 && WN == 128, "load mapping assumes 256x256 tiles, 4 waves");
  constexpr int SLOT_A = BM * NVK_BKB;           // 32 KiB of codes
  constexpr int SLOT_B = BN * NVK_BKB;
  constexpr int OFF_SA = SLOT_A + SLOT_B;        // [BM][16] E4M3 bytes
  constexpr int OFF_SB = OFF_SA + BM * NVK_BKS;  // [BN][16]
  constexpr int SLOT = OFF_SB + BN * NVK_BKS;    // 73728
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wy = wave / NWX, wx = wave % NWX;

  // Whole tiles take workgroups [0, nfull) (XCD-remapped, tile rows in
  // raster groups of NV_GROUP_M); with a split of the last round, the K parts
  // of its tiles follow, part-major within a tile.
  const int nst = p.K / NVK_BK;
  const GemmSplit sp = gemm_split(gemm_tile_count<BM, BN>(p.M, p.N, 0, nullptr), p.cus, p.split_max, nst);
  const int nfull = (sp.full + 7) / 8 * 8;
  const int bid = blockIdx.x;
  int t, u = 0, part = 0;
  if (bid < nfull) {
    t = gemm_tile_remap(bid, sp.full);
    if (t < 0) return;
  } else {
    const int j = bid - nfull;
    if (j >= sp.r * sp.S) return;
    u = j / sp.S;
    part = j % sp.S;
    t = sp.full + u;
  }
  GemmTile tile;
  gemm_tile_at<BM, BN, NV_GROUP_M>(t, p.M, p.N, 0, nullptr, tile);
  const int m0 = tile.m0, n0 = tile.n0;
  // stages [s0, s1): all of K, or K part `part` of S
  const int s0 = bid < nfull ? 0 : part * nst / sp.S;
  const int s1 = bid < nfull ? nst : (part + 1) * nst / sp.S;
  const int KB = p.K / 2, KS = p.K / 16;
  const int a_rows = min(BM, p.M - m0), b_rows = min(BN, p.N - n0);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a_codes + (size_t)m0 * KB), 0, a_rows * KB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.b_codes + (size_t)n0 * KB), 0, b_rows * KB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a_scales + (size_t)m0 * KS), 0, a_rows * KS, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.b_scales + (size_t)n0 * KS), 0, b_rows * KS, 0x00020000);

  // codes: LDS 16-byte position q = (wave*8 + j)*64 + lane holds row q/8,
  // swizzled chunk q%8 (global chunk (q%8) ^ swz8r(row))
  int voff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = (wave * 8 + j) * 64 + lane;
    const int row = q >> 3, cs = q & 7;
    voff[j] = row * KB + ((cs ^ swz8r(row)) << 4);
  }
  // scales: LDS dword 64t + lane (t = 4*wave + u) holds row (64t + lane)/4,
  // bytes 4*(lane%4) .. +3 of the row's 16 scale bytes of the stage
  int soff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) soff[u] = (64 * wave + 16 * u + (lane >> 2)) * KS + (lane & 3) * 4;

  // The 24 loads of a stage per wave (16 code copies, 8 scale copies), in
  // four parts of six: the refill of a slot goes out over four MFMA steps, so
  // the four waves never ask the texture unit for a whole stage at once.
  auto issue_part = [&](int st, int piece) {
    uint8_t* slot = smem + (st & 1) * SLOT;
    const bool in = st < s1;
    const int kb0 = st * NVK_BKB, ks0 = st * NVK_BKS;
#pragma unroll
    for (int idx = 6 * piece; idx < 6 * piece + 6; ++idx) {
      if (idx < 8) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(slot + (wave * 8 + idx) * 1024), 16,
                                                 in ? voff[idx] + kb0 : 0x7ffffff0, 0, 0, 0);
      } else if (idx < 16) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(slot + SLOT_A + (wave * 8 + idx - 8) * 1024), 16,
                                                 in ? voff[idx - 8] + kb0 : 0x7ffffff0, 0, 0, 0);
      } else {
        const int u = (idx - 16) >> 1;
        if ((idx & 1) == 0)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(slot + OFF_SA + (wave * 4 + u) * 256), 4,
                                                   in ? soff[u] + ks0 : 0x7ffffff0, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(slot + OFF_SB + (wave * 4 + u) * 256), 4,
                                                   in ? soff[u] + ks0 : 0x7ffffff0, 0, 0, 0);
      }
    }
  };
  auto issue = [&](int st) {
#pragma unroll
    for (int piece = 0; piece < 4; ++piece) issue_part(st, piece);
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int lrow = lane & 31;
  const int khalf = lane >> 5;
  // rows wy*128 + 32i + lrow (A) and wx*128 + 32j + lrow (B): the swizzle of
  // a row does not depend on i or j (32 rows apart), so one value serves all
  const int swz = swz8r(lrow);
  const int rowa = (wy * WM + lrow) * NVK_BKB, rowb = SLOT_A + (wx * WN + lrow) * NVK_BKB;
  const int srowa = OFF_SA + (wy * WM + lrow) * NVK_BKS, srowb = OFF_SB + (wx * WN + lrow) * NVK_BKS;
  const int sshift = 16 * khalf;                 // this half's two blocks of a scale dword

  // Fragment set of one K = 64 sub-stage: 16 code bytes per A/B row group
  // and the scale dword holding its blocks; two sets rotate (the next
  // sub-stage's set is read while the current one is expanded).
  u32x4 fa[2][TI], fb[2][TJ];
  uint32_t fsa[2][TI], fsb[2][TJ];
  auto read_kk = [&](int set, const uint8_t* slot, int kk) {
    const int ch = ((kk * 2 + khalf) ^ swz) << 4;
#pragma unroll
    for (int i = 0; i < TI; ++i) fa[set][i] = *reinterpret_cast<const u32x4*>(slot + rowa + i * 32 * NVK_BKB + ch);
#pragma unroll
    for (int j = 0; j < TJ; ++j) fb[set][j] = *reinterpret_cast<const u32x4*>(slot + rowb + j * 32 * NVK_BKB + ch);
#pragma unroll
    for (int i = 0; i < TI; ++i) fsa[set][i] = *reinterpret_cast<const uint32_t*>(slot + srowa + i * 32 * NVK_BKS + kk * 4);
#pragma unroll
    for (int j = 0; j < TJ; ++j) fsb[set][j] = *reinterpret_cast<const uint32_t*>(slot + srowb + j * 32 * NVK_BKS + kk * 4);
  };
  // expanded MFMA operands of one step (8 K per lane), double-buffered
  f16x8 oa[2][TI], ob[2][TJ];
  f16x2 s2a[TI], s2b[TJ];   // this lane's two block scales (fp16) of the current sub-stage
  auto expand_step = [&](int ob_i, int set, int d) {
    if (d == 0) {
#pragma unroll
      for (int i = 0; i < TI; ++i) s2a[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(fsa[set][i] >> sshift, 1.0f, false);
#pragma unroll
      for (int j = 0; j < TJ; ++j) s2b[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(fsb[set][j] >> sshift, 1.0f, false);
    }
    const int e = d >> 1;
#pragma unroll
    for (int i = 0; i < TI; ++i) oa[ob_i][i] = nv_expand8(fa[set][i][d], f16x2{s2a[i][e], s2a[i][e]});
#pragma unroll
    for (int j = 0; j < TJ; ++j) ob[ob_i][j] = nv_expand8(fb[set][j][d], f16x2{s2b[j][e], s2b[j][e]});
  };

  // Pipeline: stages s and s+1 are in LDS; a stage is 16 steps t = 4kk + d of
  // 16 MFMAs each.  During step t the wave expands step t+1 and, at t = 4kk,
  // reads the fragments of sub-stage kk+1.  At t = 12 (all of stage s read):
  // counted wait for stage s+1, barrier, refill of this slot with stage s+2
  // (interleaved with steps 12-15), read of stage s+1's first sub-stage.
  issue(s0);
  issue(s0 + 1);
  asm volatile("s_waitcnt vmcnt(24)" ::: "memory");   // stage s0 landed (stage s0+1's 24 loads may be in flight)
  block_barrier();
  read_kk(0, smem + (s0 & 1) * SLOT, 0);
  read_kk(1, smem + (s0 & 1) * SLOT, 1);
  expand_step(0, 0, 0);
  for (int s = s0; s < s1; ++s) {
    const uint8_t* cur = smem + (s & 1) * SLOT;
    const uint8_t* nxt = smem + ((s + 1) & 1) * SLOT;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int kk = t >> 2, d = t & 3;
      if (t == 12) {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");   // stage s+1 landed; reads of `cur` done
        block_barrier();
        issue_part(s + 2, 0);
        read_kk(0, nxt, 0);
      } else if (t > 12) {
        issue_part(s + 2, t - 12);
      } else if (d == 0 && kk < 3) {
        read_kk((kk + 1) & 1, cur, kk + 1);
      }
      // operands of the next step (for t = 15: step 0 of stage s+1)
      if (t < 15)
        expand_step((t + 1) & 1, ((t + 1) >> 2) & 1, (t + 1) & 3);
      else
        expand_step(0, 0, 0);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(oa[t & 1][i], ob[t & 1][j], acc[i][j], 0, 0, 0);
      // one MFMA, then a quarter of the next step's conversions, and the
      // step's LDS reads / refill loads spread between the MFMAs (a refill
      // load after every other MFMA)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (q & 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (bid >= nfull) {   // a K part: its partial tile (gA * gB is applied to the sum)
    gemm_split_store_partial<TI, TJ>(acc, p.part, u, sp.S, part);
    return;
  }

  // ---- epilogue through LDS (as in the MXFP4 kernel), times gA * gB
  const float gg = (*p.a_global) * (*p.b_global);
  block_barrier();   // every wave is done reading the slots
  constexpr int EP_PITCH = WN + 8;
  float* ep = reinterpret_cast<float*>(smem) + wave * (WM / 2) * EP_PITCH;
  const bool vec_ok = (p.ldc % 4) == 0;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int ii = 0; ii < TI / 2; ++ii)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = ii * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
          ep[lr * EP_PITCH + j * 32 + lrow] = acc[half * (TI / 2) + ii][j][r] * gg;
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
    const int cl = (lane & 31) * 4;
    const int col = n0 + wx * WN + cl;
#pragma unroll 4
    for (int t = 0; t < WM / 4; ++t) {
      const int lr = 2 * t + khalf;
      const int row = m0 + wy * WM + half * (WM / 2) + lr;
      const f32x4 v = *reinterpret_cast<const f32x4*>(&ep[lr * EP_PITCH + cl]);
      if (row < p.M) {
        if (p.c_bf16) {
          uint16_t* dst = reinterpret_cast<uint16_t*>(p.c) + (size_t)row * p.ldc + col;
          if (vec_ok && col + 3 < p.N) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            // non-temporal: C is not read again here, and the L2 keeps the A/B panels
            __builtin_nontemporal_store(u32x2{pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3])},
                                        reinterpret_cast<u32x2*>(dst));
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (col + q < p.N) dst[q] = (uint16_t)f32_to_bf16_rne(v[q]);
          }
        } else {
          float* dst = reinterpret_cast<float*>(p.c) + (size_t)row * p.ldc + col;
          if (vec_ok && col + 3 < p.N) {
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (col + q < p.N) dst[q] = v[q];
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
  }
}

constexpr int NBM = 256, NBN = 256, NWM = 128, NWN = 128;

size_t gemm_nv_split_bytes(int64_t M, int64_t N, int64_t K, int cus) {
  return K % NVK_BK == 0 ? gemm_split_bytes(M, N, 0, cus, (int)(K / NVK_BK)) : 0;
}

hipError_t launch_gemm_nv(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                          const uint8_t* b_codes, const uint8_t* b_scales, const float* b_global, void* c, int c_bf16,
                          int64_t ldc, int64_t M, int64_t N, int64_t K, hipStream_t st, float* part, size_t part_bytes,
                          int cus) {
  NvGemmParams p;
  p.a_codes = a_codes; p.a_scales = a_scales; p.a_global = a_global;
  p.b_codes = b_codes; p.b_scales = b_scales; p.b_global = b_global;
  p.c = c; p.ldc = ldc; p.M = (int)M; p.N = (int)N; p.K = (int)K; p.c_bf16 = c_bf16;
  const int64_t tiles = ((M + NBM - 1) / NBM) * ((N + NBN - 1) / NBN);
  const int64_t grid = (tiles + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  // the last round's K parts (see gemm_split.h), when the scratch holds them
  const size_t need = gemm_nv_split_bytes(M, N, K, cus);
  const bool split = part && need > 0 && part_bytes >= need;
  const int64_t nparts = (int64_t)(need / (kSplitTileFloats * sizeof(float)));
  p.split_max = split ? kGemmSplitMax : 1;
  p.cus = cus;
  p.part = split ? part : nullptr;
  constexpr int NT = (NBM / NWM) * (NBN / NWN) * 64;
  if (K % NVK_BK == 0) {
    hipLaunchKernelGGL((k_gemm_nv_k256<NBM, NBN, NWM, NWN>), dim3((unsigned)(grid + (split ? nparts : 0))), dim3(NT), 0,
                       st, p);
    if (split) {
      const int64_t rmax = tiles < cus ? tiles : cus;
      GemmSplitReduce r{part, c, ldc, c_bf16, (int)M, (int)N, 0, nullptr, cus, kGemmSplitMax, (int)(K / NVK_BK),
                        a_global, b_global};
      hipLaunchKernelGGL((k_gemm_split_reduce<NV_GROUP_M>), dim3((unsigned)(rmax * kSplitReduceWgPerTile)), dim3(256), 0,
                         st, r);
    }
  } else {
    hipLaunchKernelGGL((k_gemm_nv<NBM, NBN, NWM, NWN>), dim3((unsigned)grid), dim3(NT), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace mxk
