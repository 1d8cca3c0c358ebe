// MXFP4 x MXFP4 GEMM on CDNA4 block-scaled matrix cores.
//
// C[m, n] = sum_b 2^(eA[m,b] + eB[n,b]) * sum_{k in b} qA[m,k] qB[n,k], fp32
// accumulation: the block-scaled dot product of "NVFP4 Architecture", section
// "2. Hardware-Managed Tensor Core Dot-Products" (k-element FP4 dot products
// multiplied by the two block scales and accumulated in fp32) and the silicon
// execution of "How Microscaling FP4 (MXFP4) Halves Memory Bandwidth",
// section "Silicon Execution".  On gfx950 this is
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands: every lane feeds 32
// consecutive K values of one row (exactly one MX block) plus that block's
// E8M0 byte, so the hardware applies the two block scales itself.
//
// Tiling: a workgroup of 4 waves computes a BM x BN tile; each wave a
// WM x WN sub-tile of 32x32 MFMA tiles.  K advances 128 per stage; packed
// codes (64 B per row per stage) and the four scale bytes of each row are
// staged through LDS (double buffered, one barrier per stage).  Rows are
// stored with their four 16-byte chunks XOR-swizzled so that the 16-byte
// fragment reads of 8 or 16 consecutive rows hit distinct LDS banks.
//
// Grouped (mixture-of-experts) form: row ranges [off[g], off[g+1]) of A use
// the g-th [N, K] matrix of B; tiles never straddle groups.
//
// Workgroup -> tile mapping is XCD-aware: consecutive workgroup ids go to
// different XCDs round-robin, so id i is remapped to logical tile
// (i % 8) * ceil(T/8) + i / 8 and each XCD walks a contiguous range of tiles,
// rasterized in groups of GROUP_M tile rows so that concurrently running
// tiles on one XCD share A and B panels in that XCD's L2.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mxk {

constexpr int MX_BK = 128;          // K elements per stage
constexpr int MX_BKB = MX_BK / 2;   // bytes of packed codes per row per stage
constexpr int GROUP_M = 4;

__device__ __forceinline__ int swz4(int row) { return ((row >> 1) & 3) ^ ((row >> 2) & 3); }

struct MxGemmParams {
  const uint8_t* a_codes;  // [M, K/2]
  const uint8_t* a_scales; // [M, K/32]
  const uint8_t* b_codes;  // [G*N, K/2] (G = 1 dense)
  const uint8_t* b_scales; // [G*N, K/32]
  void* c;
  int64_t ldc;
  int M, N, K;
  int groups;              // 0 = dense
  const int32_t* offsets;  // [groups + 1]
  int c_bf16;
};

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_gemm_mx(MxGemmParams p) {
  constexpr int NWX = BN / WN;
  constexpr int NT = (BM / WM) * NWX * 64;
  constexpr int TI = WM / 32, TJ = WN / 32;
  constexpr int A_CH = BM * 4 / NT;  // 16-byte chunks per thread per stage
  constexpr int B_CH = BN * 4 / NT;
  static_assert(BM * 4 % NT == 0 && BN * 4 % NT == 0, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * MX_BKB];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * MX_BKB];
  __shared__ uint32_t sSA[2][BM];
  __shared__ uint32_t sSB[2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wy = wave / NWX, wx = wave % NWX;

  // ---- tile selection
  const int tn_count = (p.N + BN - 1) / BN;
  int g = 0, m_begin = 0, m_end = p.M, tm, tn;
  {
    int total;
    if (p.groups == 0) {
      total = ((p.M + BM - 1) / BM) * tn_count;
    } else {
      total = 0;
      for (int i = 0; i < p.groups; ++i) {
        int o0 = min(max(p.offsets[i], 0), p.M), o1 = min(max(p.offsets[i + 1], 0), p.M);
        int rows = o1 > o0 ? o1 - o0 : 0;
        total += ((rows + BM - 1) / BM) * tn_count;
      }
    }
    const int per_xcd = (total + 7) / 8;
    const int bid = blockIdx.x;
    const int local = bid / 8;
    if (local >= per_xcd) return;
    const int t = (bid % 8) * per_xcd + local;
    if (t >= total) return;
    int tl = t;  // tile index within its group
    if (p.groups != 0) {
      for (int i = 0; i < p.groups; ++i) {
        int o0 = min(max(p.offsets[i], 0), p.M), o1 = min(max(p.offsets[i + 1], 0), p.M);
        int rows = o1 > o0 ? o1 - o0 : 0;
        int nt = ((rows + BM - 1) / BM) * tn_count;
        if (tl < nt) { g = i; m_begin = o0; m_end = o1; break; }
        tl -= nt;
      }
    }
    const int tm_count = (m_end - m_begin + BM - 1) / BM;
    // grouped raster: GROUP_M tile rows at a time, walking all tile columns
    const int per_group = GROUP_M * tn_count;
    const int grp = tl / per_group;
    const int first_m = grp * GROUP_M;
    const int gm = min(tm_count - first_m, GROUP_M);
    const int in_grp = tl % per_group;
    tm = first_m + in_grp % gm;
    tn = in_grp / gm;
  }
  const int m0 = m_begin + tm * BM;
  const int n0 = tn * BN;
  const int KB = p.K / 2;          // bytes per code row
  const int KS = p.K / 32;         // scale bytes per row
  const uint8_t* Ac = p.a_codes;
  const uint8_t* As = p.a_scales;
  const uint8_t* Bc = p.b_codes + (size_t)g * p.N * KB;
  const uint8_t* Bs = p.b_scales + (size_t)g * p.N * KS;
  const bool scale_dword = (KS % 4) == 0;

  // ---- global -> register staging
  u32x4 ra[A_CH], rb[B_CH];
  uint32_t rsa = 0x7f7f7f7fu, rsb = 0x7f7f7f7fu;
  auto load_stage = [&](int s) {
    const int kb0 = s * MX_BKB;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = tid + i * NT, row = q >> 2, c = q & 3;
      const int gr = m0 + row;
      const bool ok = (gr < m_end) && (kb0 + c * 16 < KB);
      ra[i] = ok ? *reinterpret_cast<const u32x4*>(Ac + (size_t)gr * KB + kb0 + c * 16) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int q = tid + i * NT, row = q >> 2, c = q & 3;
      const int gr = n0 + row;
      const bool ok = (gr < p.N) && (kb0 + c * 16 < KB);
      rb[i] = ok ? *reinterpret_cast<const u32x4*>(Bc + (size_t)gr * KB + kb0 + c * 16) : u32x4{0, 0, 0, 0};
    }
    const int ks0 = s * 4;
    auto load_sc = [&](const uint8_t* base, int gr, bool rowok) -> uint32_t {
      if (!rowok) return 0x7f7f7f7fu;
      const uint8_t* src = base + (size_t)gr * KS + ks0;
      if (scale_dword && ks0 + 4 <= KS) return *reinterpret_cast<const uint32_t*>(src);
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) v |= (uint32_t)((ks0 + j < KS) ? src[j] : 0x7f) << (8 * j);
      return v;
    };
    if (tid < BM) rsa = load_sc(As, m0 + tid, m0 + tid < m_end);
    if (tid < BN) rsb = load_sc(Bs, n0 + tid, n0 + tid < p.N);
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = tid + i * NT, row = q >> 2, c = q & 3;
      *reinterpret_cast<u32x4*>(&sA[buf][row * MX_BKB + ((c ^ swz4(row)) << 4)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int q = tid + i * NT, row = q >> 2, c = q & 3;
      *reinterpret_cast<u32x4*>(&sB[buf][row * MX_BKB + ((c ^ swz4(row)) << 4)]) = rb[i];
    }
    if (tid < BM) sSA[buf][tid] = rsa;
    if (tid < BN) sSB[buf][tid] = rsb;
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nstages = (p.K + MX_BK - 1) / MX_BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int lrow = lane & 31;
  const int khalf = lane >> 5;  // which 32-element block of a 64-K MFMA step
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstages) load_stage(s + 1);

    uint32_t sa[TI], sb[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) sa[i] = sSA[buf][wy * WM + i * 32 + lrow] >> (8 * khalf);
#pragma unroll
    for (int j = 0; j < TJ; ++j) sb[j] = sSB[buf][wx * WN + j * 32 + lrow] >> (8 * khalf);

#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      i32x8 fa[TI], fb[TJ];
      const int c = kk * 2 + khalf;
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int row = wy * WM + i * 32 + lrow;
        i32x4 v = *reinterpret_cast<const i32x4*>(&sA[buf][row * MX_BKB + ((c ^ swz4(row)) << 4)]);
        fa[i] = i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int row = wx * WN + j * 32 + lrow;
        i32x4 v = *reinterpret_cast<const i32x4*>(&sB[buf][row * MX_BKB + ((c ^ swz4(row)) << 4)]);
        fb[j] = i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          if (kk == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 4, 4, 2, sa[i], 2, sb[j]);
        }
    }
    if (s + 1 < nstages) store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: the 32x32 output layout puts row 8*(r/4) + 4*(lane/32) + r%4,
  // column lane%32 of each tile in accumulator element r.
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = n0 + wx * WN + j * 32 + lrow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wy * WM + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
        if (row < m_end && col < p.N) {
          if (p.c_bf16)
            reinterpret_cast<uint16_t*>(p.c)[(size_t)row * p.ldc + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
          else
            reinterpret_cast<float*>(p.c)[(size_t)row * p.ldc + col] = acc[i][j][r];
        }
      }
    }
}

// Tile configuration used for every MXFP4 product.
constexpr int GBM = 256, GBN = 256, GWM = 128, GWN = 128;

hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, void* c, int c_bf16, int64_t ldc, int64_t M, int64_t N, int64_t K,
                          int groups, const int32_t* offsets, hipStream_t st) {
  MxGemmParams p;
  p.a_codes = a_codes; p.a_scales = a_scales; p.b_codes = b_codes; p.b_scales = b_scales;
  p.c = c; p.ldc = ldc; p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.groups = groups; p.offsets = offsets; p.c_bf16 = c_bf16;
  const int64_t tn = (N + GBN - 1) / GBN;
  const int64_t tm_upper = (M + GBM - 1) / GBM + (groups > 0 ? groups : 0);
  int64_t tiles = tm_upper * tn;
  int64_t grid = (tiles + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  constexpr int NT = (GBM / GWM) * (GBN / GWN) * 64;
  hipLaunchKernelGGL((k_gemm_mx<GBM, GBN, GWM, GWN>), dim3((unsigned)grid), dim3(NT), 0, st, p);
  return hipGetLastError();
}

}  // namespace mxk
