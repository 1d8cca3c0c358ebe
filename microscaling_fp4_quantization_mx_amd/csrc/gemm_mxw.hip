// Block-scaled GEMM for every pair of MX element formats (MXFP8 E4M3 / E5M2,
// MXFP6 E2M3 / E3M2, MXFP4 E2M1), mixed pairs included, on CDNA4.
//
// C[m, n] = sum_b 2^(eA[m,b] + eB[n,b]) * sum_{k in b} qA[m,k] qB[n,k], fp32
// accumulation: the same block-scaled dot product as the FP4 GEMM ("NVFP4
// Architecture", section "2. Hardware-Managed Tensor Core Dot-Products"),
// with the element formats of the MX family ("MXFP4" card, section "Core
// Facts": MXFP8/MXFP4 scaled GEMM).  v_mfma_scale_f32_32x32x64_f8f6f4 takes
// the two operands' formats as immediates, so one template serves all pairs.
//
// Operand registers of one 32x32x64 step (lane l: row l % 32, half h = l / 32;
// eight dwords per lane):
//   FP4 / FP6  K = 32h .. 32h + 31, packed contiguously (16 / 24 bytes),
//   FP8        K = 16h .. 16h + 15 in dwords 0-3, 32 + 16h .. 32 + 16h + 15 in
//              dwords 4-7;
// the scale operand of lane l is the E8M0 byte of row l % 32's 32-K block h,
// which the hardware applies to the products of K = 32h .. 32h + 31 whichever
// lane holds them.  (These placements were established on the hardware with
// exact small-integer test products.)
//
// Tiling: a 256 x 256 tile per workgroup of 4 waves (128 x 128 per wave).  K
// advances 128 per stage: the stage's row slice of each operand (128 / 96 / 64
// bytes) lands in LDS by direct-to-LDS buffer loads, rows 128 bytes apart for
// FP8 and FP6 (FP6 leaves two 16-byte slots of each row empty) and 64 apart for
// FP4, 16-byte chunks XOR-swizzled by row so that the 16-byte fragment reads
// of 8 consecutive rows hit distinct banks.  Two LDS slots: while the two
// 32x32x64 segments of stage s run, stage s + 1 lands, and the refill for
// stage s + 2 is issued as soon as every wave holds stage s's fragments.
//
// Grouped form: rows [off[g], off[g+1]) of A and C use the g-th stacked
// [N, K] matrix of B (tiles as in gemm_tiles.h), as for MXFP4.
#include "mx_device.h"
#include "gemm_tiles.h"
#include "mx_expand.h"
#include "mx_kernels.h"

namespace mxk {

template <int F>
struct MxwOp {
  static constexpr int BITS = F <= 1 ? 8 : (F <= 3 ? 6 : 4);
  static constexpr int SB = 16 * BITS;              // bytes of a row per 128-K stage
  static constexpr int CPR = SB / 16;               // 16-byte chunks per row per stage (8 / 6 / 4)
  static constexpr int PCH = BITS == 4 ? 4 : 8;     // LDS chunk slots per row
  static constexpr int PITCH = 16 * PCH;            // LDS bytes per row
  static constexpr int SLOTB = 256 * PITCH;         // LDS bytes per stage (256 rows)
  static constexpr int DMA = SLOTB / 4096;          // 1 KiB direct-to-LDS loads per wave per stage
  // slot of logical chunk c in row r is c ^ swz(r)
  static __device__ __forceinline__ int swz(int r) { return PCH == 8 ? swz8r(r) : ((r >> 1) & 3); }
  // LDS byte offset (within the operand's region) of part 0 / 1 of the
  // fragment of row `row`, 32x32x64 segment kk, lane half h
  static __device__ __forceinline__ int frag_off(int row, int kk, int part, int h) {
    int c;
    if constexpr (BITS == 8) c = 4 * kk + 2 * part + h;                        // two 16-byte chunks
    else if constexpr (BITS == 6) c = part == 0 ? 3 * kk + 2 * h : 3 * kk + 1;  // 16 + 8 bytes
    else c = 2 * kk + h;
    int off = row * PITCH + 16 * (c ^ swz(row));
    if constexpr (BITS == 6) off += part == 1 ? 8 * h : 0;
    return off;
  }
  static __device__ __forceinline__ i32x8 load_frag(const uint8_t* base, int o0, int o1, int h) {
    if constexpr (BITS == 8) {
      const i32x4 x = *reinterpret_cast<const i32x4*>(base + o0), y = *reinterpret_cast<const i32x4*>(base + o1);
      return i32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    } else if constexpr (BITS == 6) {
      typedef int i32x2 __attribute__((ext_vector_type(2)));
      const i32x4 x = *reinterpret_cast<const i32x4*>(base + o0);
      const i32x2 y = *reinterpret_cast<const i32x2*>(base + o1);
      // half 0: bytes 0-15 then 16-23; half 1: bytes 24-31 then 32-47
      return h ? i32x8{y[0], y[1], x[0], x[1], x[2], x[3], 0, 0} : i32x8{x[0], x[1], x[2], x[3], y[0], y[1], 0, 0};
    } else {
      (void)o1;
      (void)h;
      const i32x4 x = *reinterpret_cast<const i32x4*>(base + o0);
      return i32x8{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
    }
  }
};

struct MxwParams {
  const uint8_t* a_codes;   // [M, K * bitsA / 8]
  const uint8_t* a_scales;  // [M, K / 32]
  const uint8_t* b_codes;   // [G * N, K * bitsB / 8] (G = 1 dense)
  const uint8_t* b_scales;  // [G * N, K / 32]
  void* c;
  int64_t ldc;
  int M, N, K;
  int c_bf16;
  int groups;               // 0 = dense
  const int32_t* offsets;   // [groups + 1]
};

constexpr int MXW_GROUP_M = 4;

template <int FA, int FB>
__global__ __launch_bounds__(256) void k_gemm_mxw(MxwParams p) {
  using OA = MxwOp<FA>;
  using OB = MxwOp<FB>;
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128, TI = WM / 32, TJ = WN / 32;
  constexpr int SLOT = OA::SLOTB + OB::SLOTB + 4 * BM + 4 * BN;
  constexpr int EP_PITCH = WN + 8;
  constexpr int EP_BYTES = 4 * (WM / 2) * EP_PITCH * 4;
  constexpr int SMEM = 2 * SLOT > EP_BYTES ? 2 * SLOT : EP_BYTES;
  constexpr int LOADS = OA::DMA + OB::DMA + 2;       // per wave per stage
  // LDS read instructions per MFMA slot: fragments of one segment (two per
  // fragment for FP8 and FP6), plus the scale dwords with segment 0
  constexpr int RPF_A = OA::BITS == 4 ? 1 : 2, RPF_B = OB::BITS == 4 ? 1 : 2;
  constexpr int RD1 = ((TI * RPF_A + TJ * RPF_B) + TI * TJ - 1) / (TI * TJ);
  constexpr int RD0 = ((TI * RPF_A + TJ * RPF_B + (TI + TJ) / 2) + TI * TJ - 1) / (TI * TJ);
  constexpr int VM1 = (LOADS + TI * TJ - 1) / (TI * TJ);
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  static_assert(OA::DMA <= 8 && OB::DMA <= 8, "offset arrays");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets stay scalar
  const int wy = wave >> 1, wx = wave & 1;

  // ---- tile (XCD-aware, MXW_GROUP_M tile rows at a time; grouped rows)
  GemmTile tile;
  if (!gemm_tile<BM, BN, MXW_GROUP_M>(blockIdx.x, p.M, p.N, p.groups, p.offsets, tile)) return;
  const int m0 = tile.m0, n0 = tile.n0, m_end = tile.m_end;
  const int KBA = p.K / 8 * OA::BITS, KBB = p.K / 8 * OB::BITS, KS = p.K / 32;
  const int a_rows = min(BM, m_end - m0), b_rows = min(BN, p.N - n0);
  const size_t b_row0 = (size_t)tile.g * p.N + n0;

  // buffer descriptors over the tile's valid rows: reads beyond return zero
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.a_codes + (size_t)m0 * KBA), 0, a_rows * KBA, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.b_codes + b_row0 * KBB), 0, b_rows * KBB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.a_scales + (size_t)m0 * KS), 0, a_rows * KS, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.b_scales + b_row0 * KS), 0, b_rows * KS, 0x00020000);

  // Per-lane source offsets of the direct-to-LDS loads (stage 0).  LDS 16-byte
  // unit q = (wave * DMA + j) * 64 + lane of an operand holds row q / PCH,
  // slot q % PCH, i.e. logical chunk slot ^ swz(row); a chunk beyond the row's
  // slice (FP6's two spare slots) reads from past the descriptor: zeros.
  constexpr int OOB = 0x7ffffff0;   // beyond every range (K is kept so that ranges stay below 2^30)
  constexpr int DEAD = 0x40000000;  // spare slot: beyond the range at every stage offset too
  // (The lambdas below name no template-dependent member or array bound:
  // with such a capture the host-side launch stub is silently not emitted.)
  constexpr int DMA_A = OA::DMA, DMA_B = OB::DMA, SB_A = OA::SB, SB_B = OB::SB;
  constexpr int REG_B = OA::SLOTB, REG_S = OA::SLOTB + OB::SLOTB;   // B and scale regions of a slot
  int va[8], vb[8];   // the first DMA_A / DMA_B entries are used
#pragma unroll
  for (int j = 0; j < DMA_A; ++j) {
    const int q = (wave * DMA_A + j) * 64 + lane, row = q / OA::PCH, c = (q % OA::PCH) ^ OA::swz(row);
    va[j] = c < OA::CPR ? row * KBA + 16 * c : DEAD;
  }
#pragma unroll
  for (int j = 0; j < DMA_B; ++j) {
    const int q = (wave * DMA_B + j) * 64 + lane, row = q / OB::PCH, c = (q % OB::PCH) ^ OB::swz(row);
    vb[j] = c < OB::CPR ? row * KBB + 16 * c : DEAD;
  }
  const int vs = (wave * 64 + lane) * KS;    // scale dword of row wave * 64 + lane
  const int nst = p.K / 128;
  auto issue = [&](int st) {
    uint8_t* slot = smem + (st & 1) * SLOT;
    const bool in = st < nst;
#pragma unroll
    for (int j = 0; j < DMA_A; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(slot + (wave * DMA_A + j) * 1024), 16,
                                               in ? va[j] + st * SB_A : OOB, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < DMA_B; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(slot + REG_B + (wave * DMA_B + j) * 1024), 16,
                                               in ? vb[j] + st * SB_B : OOB, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(slot + REG_S + wave * 256), 4,
                                             in ? vs + st * 4 : OOB, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(slot + REG_S + 4 * BM + wave * 256), 4,
                                             in ? vs + st * 4 : OOB, 0, 0, 0);
  };

  // ---- fragment reads
  const int lrow = lane & 31, h = lane >> 5;
  const int rowa = wy * WM + lrow, rowb = wx * WN + lrow;   // + 32 i / 32 j (same swizzle)
  int oa[2][2], ob[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      oa[kk][part] = OA::frag_off(rowa, kk, part, h);
      ob[kk][part] = OA::SLOTB + OB::frag_off(rowb, kk, part, h);
    }
  const int osa = REG_S + rowa * 4, osb = REG_S + 4 * BM + rowb * 4;
  constexpr int PITCH_A = OA::PITCH, PITCH_B = OB::PITCH;
  i32x8 fa[2][TI], fb[2][TJ];
  uint32_t sa[TI], sb[TJ];
  auto read_seg = [&](const uint8_t* slot, int kk) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
      fa[kk][i] = OA::load_frag(slot + i * 32 * PITCH_A, oa[kk][0], oa[kk][1], h);
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      fb[kk][j] = OB::load_frag(slot + j * 32 * PITCH_B, ob[kk][0], ob[kk][1], h);
    if (kk == 0) {
#pragma unroll
      for (int i = 0; i < TI; ++i) sa[i] = *reinterpret_cast<const uint32_t*>(slot + osa + i * 128);
#pragma unroll
      for (int j = 0; j < TJ; ++j) sb[j] = *reinterpret_cast<const uint32_t*>(slot + osb + j * 128);
    }
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  issue(0);
  issue(1);
  wait_vmcnt<LOADS>();     // this wave's loads of stage 0 are in LDS
  block_barrier();         // ... and every other wave's
  read_seg(smem, 0);
  const int sshift = 8 * h;
  for (int s = 0; s < nst; ++s) {
    const uint8_t* slot = smem + (s & 1) * SLOT;
    uint32_t sas[TI], sbs[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) sas[i] = sa[i] >> sshift;
#pragma unroll
    for (int j = 0; j < TJ; ++j) sbs[j] = sb[j] >> sshift;
    // segment 0 (K 0..63 of stage s); read segment 1's fragments meanwhile
    read_seg(slot, 1);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[0][i], fb[0][j], acc[i][j], FA, FB, 0, sas[i], 0,
                                                                   sbs[j]);
    // one fragment read between consecutive MFMAs
#pragma unroll
    for (int q = 0; q < TI * TJ; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, RD1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // every wave holds stage s's fragments and stage s + 1 has landed: refill
    // this slot with stage s + 2
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    block_barrier();
    issue(s + 2);
    // segment 1 (K 64..127); read stage s + 1's segment-0 fragments meanwhile
    read_seg(smem + ((s + 1) & 1) * SLOT, 0);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[1][i], fb[1][j], acc[i][j], FA, FB, 2, sas[i], 2,
                                                                   sbs[j]);
    // the refill loads and the next fragment reads spread between the MFMAs
#pragma unroll
    for (int q = 0; q < TI * TJ; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, VM1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, RD0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<0>();

  // ---- epilogue through LDS: each wave stages half of its 128 x 128 fp32
  // tile at a time (row pitch 136 floats), then writes whole row segments.
  block_barrier();
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
          const int lr = ii * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          ep[lr * EP_PITCH + j * 32 + lrow] = acc[half * (TI / 2) + ii][j][r];
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    const int cl = lrow * 4;
    const int col = n0 + wx * WN + cl;
#pragma unroll 4
    for (int t2 = 0; t2 < WM / 4; ++t2) {
      const int lr = 2 * t2 + h;
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
// Exact route for MX pairs with an FP8 or FP6 operand.  The block-scaled MFMA
// above truncates each product of a group of eight K values to 13 bits below
// the group's largest product (measured), which FP4 x FP4 never reaches but
// FP8 and FP6 operands can.  Here every code is expanded, once per workgroup
// while staging into LDS, to the exact bf16 value q * 2^(E-127): the scaled
// conversions v_cvt_scalef32_pk_bf16_fp8 / _bf8 / _fp4 and
// v_cvt_scalef32_pk32_bf16_fp6 / _bf6 apply the block's power of two.  Such a
// value has at most 4 significant bits, so it is exact in bf16 wherever it
// lies in bf16's normal range [2^-126, 2^128); every tensor the quantizer
// writes from inputs below 2^127 in magnitude stays there (its smallest
// nonzero element value is 2^-58, an E5M2 subnormal at the floor scale).  The
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16) form exact products and add
// them in fp32, so the result is the fp32-accumulated block-scaled sum.  4 waves, 256 x 256 tile,
// 128 x 128 per wave, K = 64 per stage (two MX blocks per row), LDS rows of
// 64 bf16 with XOR-swizzled 16-byte chunks, double buffered.
// ---------------------------------------------------------------------------
constexpr int MXX_BK = 64;        // K per stage
constexpr int MXX_ROWB = 128;     // LDS bytes per bf16 row per stage

__device__ __forceinline__ int mxx_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// E8M0 byte -> the fp32 power of two the conversions scale by (bytes 0 and
// 255, which the quantizer never writes, are taken as 1 and 254).
__device__ __forceinline__ float mxx_scale(uint32_t e) { return ffrom(min(max(e, 1u), 254u) << 23); }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <int FA, int FB>
__global__ __launch_bounds__(256) void k_gemm_mxx(MxwParams p) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128, TI = WM / 32, TJ = WN / 32;
  constexpr int NT = 256;
  constexpr int WA = MxwOp<FA>::BITS, WB = MxwOp<FB>::BITS;   // dwords per 32-code block = bits
  constexpr int SEG = BM * 2 / NT;                            // block segments per thread per operand
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * MXX_ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * MXX_ROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wy = wave >> 1, wx = wave & 1;
  GemmTile tile;
  if (!gemm_tile<BM, BN, MXW_GROUP_M>(blockIdx.x, p.M, p.N, p.groups, p.offsets, tile)) return;
  const int m0 = tile.m0, n0 = tile.n0, m_end = tile.m_end;
  const uint8_t* b_codes = p.b_codes + (size_t)tile.g * p.N * (p.K / 8 * WB);
  const uint8_t* b_scales = p.b_scales + (size_t)tile.g * p.N * (p.K / 32);
  const int KBA = p.K / 8 * WA, KBB = p.K / 8 * WB, KS = p.K / 32;   // code bytes per row = K * bits / 8

  // segment q = tid + i*NT of a stage: row q >> 1, MX block q & 1 of the stage
  uint32_t ca[SEG][WA], cb[SEG][WB], sa[SEG], sb[SEG];
  auto load_stage = [&](int s) {
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int q = tid + i * NT, row = q >> 1, blk = s * 2 + (q & 1);
      const bool oka = m0 + row < m_end && blk < KS, okb = n0 + row < p.N && blk < KS;
      const uint32_t* pa = reinterpret_cast<const uint32_t*>(p.a_codes + (size_t)(m0 + row) * KBA + (size_t)blk * WA * 4);
      const uint32_t* pb = reinterpret_cast<const uint32_t*>(b_codes + (size_t)(n0 + row) * KBB + (size_t)blk * WB * 4);
#pragma unroll
      for (int d = 0; d < WA; ++d) ca[i][d] = oka ? pa[d] : 0u;
#pragma unroll
      for (int d = 0; d < WB; ++d) cb[i][d] = okb ? pb[d] : 0u;
      sa[i] = oka ? p.a_scales[(size_t)(m0 + row) * KS + blk] : 127u;
      sb[i] = okb ? b_scales[(size_t)(n0 + row) * KS + blk] : 127u;
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int q = tid + i * NT, row = q >> 1, h = q & 1;
      uint32_t o[16];
      expand_block_bf16<FA>(ca[i], mxx_scale(sa[i]), o);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<u32x4*>(&sA[buf][row * MXX_ROWB + (((4 * h + c) ^ mxx_swz(row)) << 4)]) =
            u32x4{o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]};
      expand_block_bf16<FB>(cb[i], mxx_scale(sb[i]), o);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<u32x4*>(&sB[buf][row * MXX_ROWB + (((4 * h + c) ^ mxx_swz(row)) << 4)]) =
            u32x4{o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]};
    }
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nstages = (p.K + MXX_BK - 1) / MXX_BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  const int lrow = lane & 31, khalf = lane >> 5;
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstages) load_stage(s + 1);
#pragma unroll
    for (int kk = 0; kk < MXX_BK / 16; ++kk) {
      const int c = kk * 2 + khalf;  // lane holds K = 16 kk + 8 khalf + (0..7)
      bf16x8_t fa[TI], fb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int row = wy * WM + i * 32 + lrow;
        fa[i] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][row * MXX_ROWB + ((c ^ mxx_swz(row)) << 4)]);
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int row = wx * WN + j * 32 + lrow;
        fb[j] = *reinterpret_cast<const bf16x8_t*>(&sB[buf][row * MXX_ROWB + ((c ^ mxx_swz(row)) << 4)]);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nstages) store_stage(buf ^ 1);
    __syncthreads();
  }

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

hipError_t launch_gemm_mxw(int fa, int fb, const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                           const uint8_t* b_scales, void* c, int c_bf16, int64_t ldc, int64_t M, int64_t N, int64_t K,
                           int groups, const int32_t* offsets, hipStream_t st, bool exact) {
  MxwParams p;
  p.a_codes = a_codes; p.a_scales = a_scales; p.b_codes = b_codes; p.b_scales = b_scales;
  p.c = c; p.ldc = ldc; p.M = (int)M; p.N = (int)N; p.K = (int)K; p.c_bf16 = c_bf16;
  p.groups = groups; p.offsets = offsets;
  const int64_t tiles = gemm_tile_bound(M, N, 256, 256, groups);
  const int64_t grid = (tiles + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  if (fa < 0 || fa > 4 || fb < 0 || fb > 4) return hipErrorInvalidValue;
#define MXW_L(A, B)                                                                     \
  if (exact) hipLaunchKernelGGL((k_gemm_mxx<A, B>), dim3((unsigned)grid), dim3(256), 0, st, p); \
  else hipLaunchKernelGGL((k_gemm_mxw<A, B>), dim3((unsigned)grid), dim3(256), 0, st, p)
#define MXW_ROW(A)                \
  switch (fb) {                   \
    case 0: MXW_L(A, 0); break;   \
    case 1: MXW_L(A, 1); break;   \
    case 2: MXW_L(A, 2); break;   \
    case 3: MXW_L(A, 3); break;   \
    default: MXW_L(A, 4); break;  \
  }
  switch (fa) {
    case 0: MXW_ROW(0); break;
    case 1: MXW_ROW(1); break;
    case 2: MXW_ROW(2); break;
    case 3: MXW_ROW(3); break;
    default: MXW_ROW(4); break;
  }
#undef MXW_ROW
#undef MXW_L
  return hipGetLastError();
}

}  // namespace mxk
