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
// the g-th [N, K] matrix of B; tiles never straddle groups.  The
// workgroup -> tile mapping (XCD-aware, GROUP_M tile rows at a time) is
// gemm_tiles.h's.
#include "mx_device.h"
#include "gemm_mx_tile.h"
#include "gemm_tiles.h"
#include "gemm_split.h"
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
  // split of the last round along K (k_gemm_mx_k256 only; split_max < 2: none)
  int split_max;
  int cus;                 // workgroup slots of the device (one per CU)
  float* part;             // fp32 partial tiles, cus x 65536 floats
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
  GemmTile tile;
  if (!gemm_tile<BM, BN, GROUP_M>(blockIdx.x, p.M, p.N, p.groups, p.offsets, tile)) return;
  const int g = tile.g, m_end = tile.m_end, m0 = tile.m0, n0 = tile.n0;
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

// ---------------------------------------------------------------------------
// Main path (K % 128 == 0): a 4-slot LDS ring filled by direct-to-LDS buffer
// loads (buffer_load_dwordx4 ... lds), three stages in flight.  Each wave
// waits only for its own loads of the stage it is about to use
// (s_waitcnt vmcnt(n) with n = loads issued after that stage), then a bare
// s_barrier publishes the slot to the whole workgroup; no register staging,
// so the 256 accumulators stay in AGPRs and the loads never stall the MFMA
// stream.  Rows past the matrix edge read as zero through the buffer range
// check (the tile's buffer descriptor covers only its valid rows).
// ---------------------------------------------------------------------------
constexpr int RING = 4;
constexpr int LOADS_PER_STAGE = 10;  // per wave: 4 A chunks, 4 B chunks, 1 A scale, 1 B scale

__device__ __forceinline__ void wait_vm(int n) {
  // n is one of the three pipeline depths; s_waitcnt needs an immediate.
  if (n >= 2 * LOADS_PER_STAGE)
    asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
  else if (n >= LOADS_PER_STAGE)
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_gemm_mx_ring(MxGemmParams p) {
  constexpr int NWX = BN / WN;
  constexpr int NT = (BM / WM) * NWX * 64;
  constexpr int NW = NT / 64;
  constexpr int TI = WM / 32, TJ = WN / 32;
  static_assert(BM == 256 && BN == 256 && NW == 4, "load mapping assumes a 256x256 tile and 4 waves");
  constexpr int SLOT_A = BM * MX_BKB;             // 16 KiB
  constexpr int SLOT_B = BN * MX_BKB;
  constexpr int SLOT = SLOT_A + SLOT_B + 4 * BM + 4 * BN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[RING * SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wy = wave / NWX, wx = wave % NWX;

  // ---- tile selection
  GemmTile tile;
  if (!gemm_tile<BM, BN, GROUP_M>(blockIdx.x, p.M, p.N, p.groups, p.offsets, tile)) return;
  const int g = tile.g, m_end = tile.m_end, m0 = tile.m0, n0 = tile.n0;
  const int KB = p.K / 2, KS = p.K / 32;
  const int a_rows = min(BM, m_end - m0), b_rows = min(BN, p.N - n0);

  // Buffer descriptors over this tile's valid rows (reads past them return 0).
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a_codes + (size_t)m0 * KB), 0, a_rows * KB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.b_codes + ((size_t)g * p.N + n0) * KB), 0, b_rows * KB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a_scales + (size_t)m0 * KS), 0, a_rows * KS, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.b_scales + ((size_t)g * p.N + n0) * KS), 0, b_rows * KS, 0x00020000);

  // Per-lane byte offsets (stage 0); the stage offset goes in soffset.  LDS
  // chunk position q = (wave*4 + j)*64 + lane holds row q/4, swizzled chunk
  // q%4, i.e. global chunk (q%4) ^ swz4(row).
  int voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = (wave * 4 + j) * 64 + lane;
    const int row = q >> 2, cs = q & 3;
    voff[j] = row * KB + ((cs ^ swz4(row)) << 4);
  }
  const int soff_row = (wave * 64 + lane) * KS;   // scale dword of row wave*64+lane

  // All offsets go in the per-lane voffset, which the raw-buffer range check
  // covers; soffset stays 0.  A stage past the end gets an offset beyond
  // every descriptor's range (the host keeps K <= 2^23, so tile ranges stay
  // below 2^30 bytes) and therefore loads zeros.
  const int nst = p.K / MX_BK;
  auto issue = [&](int st) {
    uint8_t* slot = smem + (st % RING) * SLOT;
    const bool in = st < nst;
    const int kb0 = st * MX_BKB;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(slot + (wave * 4 + j) * 1024), 16,
                                               in ? voff[j] + kb0 : 0x7ffffff0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(slot + SLOT_A + (wave * 4 + j) * 1024), 16,
                                               in ? voff[j] + kb0 : 0x7ffffff0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(slot + SLOT_A + SLOT_B + wave * 256), 4,
                                             in ? soff_row + st * 4 : 0x7ffffff0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(slot + SLOT_A + SLOT_B + 4 * BM + wave * 256), 4,
                                             in ? soff_row + st * 4 : 0x7ffffff0, 0, 0, 0);
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Prefetch is issued unconditionally: a stage past the end lies outside
  // the buffer range (soffset beyond num_records) and loads zeros, so every
  // iteration waits for the same count and the loop body is one basic block.
  const int nstages = p.K / MX_BK;
  issue(0);
  issue(1);
  issue(2);

  const int lrow = lane & 31;
  const int khalf = lane >> 5;
  // LDS byte offsets (within a slot) of this lane's fragments: A row
  // wy*WM + i*32 + lrow, B row wx*WN + j*32 + lrow, 16-byte chunk kk*2+khalf.
  int offa[2][TI], offb[2][TJ];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = wy * WM + i * 32 + lrow;
      offa[kk][i] = row * MX_BKB + (((kk * 2 + khalf) ^ swz4(row)) << 4);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int row = wx * WN + j * 32 + lrow;
      offb[kk][j] = SLOT_A + row * MX_BKB + (((kk * 2 + khalf) ^ swz4(row)) << 4);
    }
  }
  const int offsa = SLOT_A + SLOT_B + (wy * WM + lrow) * 4;
  const int offsb = SLOT_A + SLOT_B + 4 * BM + (wx * WN + lrow) * 4;
  const int sshift = 8 * khalf;

  i32x4 fa0[TI], fb0[TJ], fa1[TI], fb1[TJ];
  uint32_t sa[TI], sb[TJ];
  auto read_k0 = [&](const uint8_t* slot) {
#pragma unroll
    for (int i = 0; i < TI; ++i) fa0[i] = *reinterpret_cast<const i32x4*>(slot + offa[0][i]);
#pragma unroll
    for (int j = 0; j < TJ; ++j) fb0[j] = *reinterpret_cast<const i32x4*>(slot + offb[0][j]);
#pragma unroll
    for (int i = 0; i < TI; ++i) sa[i] = *reinterpret_cast<const uint32_t*>(slot + offsa + i * 128);
#pragma unroll
    for (int j = 0; j < TJ; ++j) sb[j] = *reinterpret_cast<const uint32_t*>(slot + offsb + j * 128);
  };
  auto read_k1 = [&](const uint8_t* slot) {
#pragma unroll
    for (int i = 0; i < TI; ++i) fa1[i] = *reinterpret_cast<const i32x4*>(slot + offa[1][i]);
#pragma unroll
    for (int j = 0; j < TJ; ++j) fb1[j] = *reinterpret_cast<const i32x4*>(slot + offb[1][j]);
  };

  asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
  block_barrier();
  read_k0(smem);
  for (int s = 0; s < nstages; ++s) {
    const uint8_t* slot = smem + (s % RING) * SLOT;
    uint32_t sa_s[TI], sb_s[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) sa_s[i] = sa[i] >> sshift;
#pragma unroll
    for (int j = 0; j < TJ; ++j) sb_s[j] = sb[j] >> sshift;
    // segment 1: K 0..63 of stage s; read this stage's second-half fragments
    read_k1(slot);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const i32x8 a8 = {fa0[i][0], fa0[i][1], fa0[i][2], fa0[i][3], 0, 0, 0, 0};
        const i32x8 b8 = {fb0[j][0], fb0[j][1], fb0[j][2], fb0[j][3], 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][j], 4, 4, 0, sa_s[i], 0, sb_s[j]);
      }
#pragma unroll
    for (int q = 0; q < TI + TJ; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ - TI - TJ, 0);
    __builtin_amdgcn_sched_barrier(0);
    // segment 2: stage s+1 is complete in LDS once every wave has seen its
    // own loads land; then refill the slot stage s-1 used.
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    block_barrier();
    issue(s + RING - 1);
    __builtin_amdgcn_sched_barrier(0);
    // segment 3: K 64..127 of stage s; read stage s+1's first-half fragments
    read_k0(smem + ((s + 1) % RING) * SLOT);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const i32x8 a8 = {fa1[i][0], fa1[i][1], fa1[i][2], fa1[i][3], 0, 0, 0, 0};
        const i32x8 b8 = {fb1[j][0], fb1[j][1], fb1[j][2], fb1[j][3], 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][j], 4, 4, 2, sa_s[i], 2, sb_s[j]);
      }
#pragma unroll
    for (int q = 0; q < TI + TJ + 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ - TI - TJ - 4, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue through LDS: each wave stages half of its 128 x 128 fp32
  // tile (64 rows, row pitch 136 floats so the two half-waves' writes fall
  // in different banks), then writes whole rows with 8- or 16-byte stores.
  block_barrier();   // every wave is done reading the ring
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
          ep[lr * EP_PITCH + j * 32 + lrow] = acc[half * (TI / 2) + ii][j][r];
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
    const int cl = (lane & 31) * 4;
    const int col = n0 + wx * WN + cl;
#pragma unroll 4
    for (int t = 0; t < WM / 4; ++t) {
      const int lr = 2 * t + khalf;
      const int row = m0 + wy * WM + half * (WM / 2) + lr;
      const f32x4 v = *reinterpret_cast<const f32x4*>(&ep[lr * EP_PITCH + cl]);
      if (row < m_end) {
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

// ---------------------------------------------------------------------------
// Main path for K % 256 == 0: one 256 x 256 tile per workgroup, the K loop
// and the store of gemm_mx_tile.h.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, bool SP>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_gemm_mx_k256(MxGemmParams p) {
  using T = MxTile<SP>;
  static_assert(BM == T::BM && BN == T::BN && WM == T::WM && WN == T::WN, "one tile shape");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::SMEM];

  // Whole tiles take workgroups [0, nfull) (XCD-remapped); with a split, the
  // K parts of the last round's tiles follow, part-major within a tile.
  const int nst = p.K / BK2;
  const int total = gemm_tile_count<BM, BN>(p.M, p.N, p.groups, p.offsets);
  const GemmSplit sp = gemm_split(total, p.cus, p.split_max, SP ? nst / 2 : nst);
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
  gemm_tile_at<BM, BN, GROUP_M>(t, p.M, p.N, p.groups, p.offsets, tile);
  const int g = tile.g, m_end = tile.m_end, m0 = tile.m0, n0 = tile.n0;
  const MxTileSrc src = mx_tile_src(p.a_codes, p.a_scales, p.b_codes, p.b_scales, p.K, (size_t)m0,
                                    min(BM, m_end - m0), (size_t)g * p.N + n0, min(BN, p.N - n0));
  f32x16 acc[T::TI][T::TJ];
#pragma unroll
  for (int i = 0; i < T::TI; ++i)
#pragma unroll
    for (int j = 0; j < T::TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // a whole tile: all stages; K part `part` of S: stages [s0, s1) (SP: whole
  // stage pairs)
  int s0 = 0, s1 = nst;
  if (bid >= nfull) {
    if (SP) {
      const int np = nst / 2;
      s0 = 2 * (part * np / sp.S);
      s1 = 2 * ((part + 1) * np / sp.S);
    } else {
      s0 = part * nst / sp.S;
      s1 = (part + 1) * nst / sp.S;
    }
  }
  mx_tile_mainloop<SP>(smem, src, s0, s1, acc);
  if (bid < nfull) {
    mx_tile_store<SP>(smem, p.c, p.ldc, p.c_bf16, p.N, m0, m_end, n0, acc);
    return;
  }
  gemm_split_store_partial<T::TI, T::TJ>(acc, p.part, u, sp.S, part);
}

// Tile configuration used for every MXFP4 product.
constexpr int GBM = 256, GBN = 256, GWM = 128, GWN = 128;

// K parts available to a split tile of the K = 256-stage kernel (paired
// scale stages when K % 512 == 0)
static int gemm_mx_parts(int64_t K) {
  if (K % BK2 != 0) return 0;
  return (int)(K % (2 * BK2) == 0 ? K / (2 * BK2) : K / BK2);
}

size_t gemm_mx_split_bytes(int64_t M, int64_t N, int64_t K, int groups, int cus) {
  return gemm_split_bytes(M, N, groups, cus, gemm_mx_parts(K));
}

hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, void* c, int c_bf16, int64_t ldc, int64_t M, int64_t N, int64_t K,
                          int groups, const int32_t* offsets, hipStream_t st, float* part, size_t part_bytes,
                          int cus) {
  MxGemmParams p;
  p.a_codes = a_codes; p.a_scales = a_scales; p.b_codes = b_codes; p.b_scales = b_scales;
  p.c = c; p.ldc = ldc; p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.groups = groups; p.offsets = offsets; p.c_bf16 = c_bf16;
  const int64_t tiles = gemm_tile_bound(M, N, GBM, GBN, groups);
  int64_t grid = (tiles + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  // The split needs a partial tile for each part: at most min(cus, tiles x
  // kGemmSplitMax) of them (r split tiles x S parts, r * S <= cus).
  const size_t need = gemm_mx_split_bytes(M, N, K, groups, cus);
  const bool split = part && need > 0 && part_bytes >= need;
  const int64_t nparts = (int64_t)(need / (kSplitTileFloats * sizeof(float)));   // workgroups for the parts
  const int64_t rmax = tiles < cus ? tiles : cus;                                // split tiles at most
  p.split_max = split ? kGemmSplitMax : 1;
  p.cus = cus;
  p.part = split ? part : nullptr;
  constexpr int NT = (GBM / GWM) * (GBN / GWN) * 64;
  if (K % (2 * BK2) == 0)
    hipLaunchKernelGGL((k_gemm_mx_k256<GBM, GBN, GWM, GWN, true>), dim3((unsigned)(grid + (split ? nparts : 0))),
                       dim3(NT), 0, st, p);
  else if (K % BK2 == 0)
    hipLaunchKernelGGL((k_gemm_mx_k256<GBM, GBN, GWM, GWN, false>), dim3((unsigned)(grid + (split ? nparts : 0))),
                       dim3(NT), 0, st, p);
  if (K % BK2 == 0) {
    if (split) {
      GemmSplitReduce r{part, c, ldc, c_bf16, (int)M, (int)N, groups, offsets, cus, kGemmSplitMax,
                        gemm_mx_parts(K), nullptr, nullptr};
      hipLaunchKernelGGL((k_gemm_split_reduce<GROUP_M>), dim3((unsigned)(rmax * kSplitReduceWgPerTile)), dim3(256), 0,
                         st, r);
    }
  } else if (K % MX_BK == 0) {
    hipLaunchKernelGGL((k_gemm_mx_ring<GBM, GBN, GWM, GWN>), dim3((unsigned)grid), dim3(NT), 0, st, p);
  } else {
    hipLaunchKernelGGL((k_gemm_mx<GBM, GBN, GWM, GWN>), dim3((unsigned)grid), dim3(NT), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace mxk
