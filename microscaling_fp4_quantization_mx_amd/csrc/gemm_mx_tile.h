// One 256 x 256 MXFP4 output tile on the block-scaled matrix cores of gfx950
// (v_mfma_scale_f32_32x32x64_f8f6f4): the K loop over a range of K = 256
// stages and the store of the fp32 accumulators to C.  Shared by the
// one-tile-per-workgroup GEMM and the persistent fused quantize + GEMM kernel.
//
// Stages of K = 256 (128 bytes of codes per row), two LDS slots of 64 KiB.
// Whole 128-byte row slices per direct-to-LDS load keep every request a full
// cache line, which roughly doubles the per-CU L2 -> LDS rate over 64-byte
// slices.  A stage is four K = 64 MFMA segments; each segment reads the next
// segment's fragments while its 16 MFMAs run, and the refill of the slot just
// consumed is spread over the last two segments (one load per MFMA), so it
// has about a stage of MFMA time to land.
//
// SP (K % 512 == 0): the scale bytes of two stages (16 per row) travel
// together, one lane per row, into a three-entry ring of their own.  Loading a
// stage's 8 bytes per row touches one cache line per row for 8 bytes; pairing
// stages halves the line touches and spreading the pair's A and B halves over
// two stages leaves one scale load per wave per stage (instead of four).
#pragma once
#include "mx_device.h"

namespace mxk {

constexpr int BK2 = 256, BKB2 = 128;

template <bool SP>
struct MxTile {
  static constexpr int BM = 256, BN = 256, WM = 128, WN = 128;
  static constexpr int NWX = BN / WN;
  static constexpr int NT = (BM / WM) * NWX * 64;   // 256 threads, 4 waves
  static constexpr int TI = WM / 32, TJ = WN / 32;
  static constexpr int SLOT_A = BM * BKB2;          // 32 KiB
  static constexpr int SLOT_B = BN * BKB2;
  static constexpr int OFF_SA = SLOT_A + SLOT_B;    // 2 x [BM] dwords, then 2 x [BN]
  static constexpr int OFF_SB = OFF_SA + 8 * BM;
  static constexpr int SLOT = SP ? SLOT_A + SLOT_B : OFF_SB + 8 * BN;   // 65536 / 69632
  static constexpr int SCL_OFF = 2 * SLOT;          // SP: ring of 3 x ([BM] + [BN]) x 16 bytes
  static constexpr int SCL_BUF = (BM + BN) * 16;
  static constexpr int SMEM = SP ? SCL_OFF + 3 * SCL_BUF : 2 * SLOT;   // 155648 / 139264
  static constexpr int LPS = SP ? 17 : 20;          // loads per wave per stage
  static constexpr int LA = LPS - 8;                // of which A codes and scale bytes
};

// The four operand streams of one tile: codes and scale bytes of its A rows
// [m0, m0 + a_rows) and B rows [n0, n0 + b_rows) (of group matrix g).
struct MxTileSrc {
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
  int KB, KS;   // bytes of codes / scales per row
};

__device__ __forceinline__ MxTileSrc mx_tile_src(const uint8_t* a_codes, const uint8_t* a_scales,
                                                 const uint8_t* b_codes, const uint8_t* b_scales, int K,
                                                 size_t a_row0, int a_rows, size_t b_row0, int b_rows) {
  MxTileSrc t;
  t.KB = K / 2;
  t.KS = K / 32;
  t.ra = __builtin_amdgcn_make_buffer_rsrc((void*)(a_codes + a_row0 * t.KB), 0, a_rows * t.KB, 0x00020000);
  t.rb = __builtin_amdgcn_make_buffer_rsrc((void*)(b_codes + b_row0 * t.KB), 0, b_rows * t.KB, 0x00020000);
  t.rsa = __builtin_amdgcn_make_buffer_rsrc((void*)(a_scales + a_row0 * t.KS), 0, a_rows * t.KS, 0x00020000);
  t.rsb = __builtin_amdgcn_make_buffer_rsrc((void*)(b_scales + b_row0 * t.KS), 0, b_rows * t.KS, 0x00020000);
  return t;
}

// acc += the tile's products over stages [s0, s1) (SP: s0 and s1 even).
// Ends with every load of the range complete; LDS is free on return once the
// caller has passed a barrier.
template <bool SP>
__device__ __forceinline__ void mx_tile_mainloop(uint8_t* smem, const MxTileSrc& t, int s0, int s1,
                                                 f32x16 (&acc)[MxTile<SP>::TI][MxTile<SP>::TJ]) {
  using C = MxTile<SP>;
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, NWX = C::NWX, TI = C::TI, TJ = C::TJ;
  constexpr int SLOT_A = C::SLOT_A, OFF_SA = C::OFF_SA, OFF_SB = C::OFF_SB, SLOT = C::SLOT;
  constexpr int SCL_OFF = C::SCL_OFF, SCL_BUF = C::SCL_BUF, LPS = C::LPS, LA = C::LA;
  // opaque to the optimizer, so that in a persistent caller the per-thread
  // offsets below are formed per tile instead of held in registers across
  // the caller's whole job loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wy = wave / NWX, wx = wave % NWX;
  const int KB = t.KB;

  // LDS 16-byte position q = (wave*8 + j)*64 + lane of a panel holds row q/8,
  // swizzled chunk q%8, i.e. global chunk (q%8) ^ swz8r(row).
  int voff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = (wave * 8 + j) * 64 + lane;
    const int row = q >> 3, cs = q & 7;
    voff[j] = row * KB + ((cs ^ swz8r(row)) << 4);
  }
  const int srow = (wave * 64 + lane) * t.KS;
  // SP: the 16 scale bytes of stages 2P, 2P+1 of row wave*64 + lane -> ring
  // entry P % 3 (one 16-byte load per lane; half 0 = A rows, half 1 = B rows)
  auto issue_scales = [&](int P, int half) {
    uint8_t* dst = smem + SCL_OFF + (P % 3) * SCL_BUF + half * (BM * 16) + wave * 1024;
    const bool in = 2 * P < s1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(half ? t.rsb : t.rsa, (lds_ptr_t)dst, 16,
                                             in ? srow + P * 16 : 0x7ffffff0, 0, 0, 0);
  };
  // All offsets in voffset (range checked); stages past the range load zeros.
  // A stage's loads go out in two parts: the A codes with the scale bytes
  // (LA loads per wave), then the B codes (8).
  auto issue_b = [&](int st) {
    uint8_t* slot = smem + (st & 1) * SLOT;
    const bool in = st < s1;
    const int kb0 = st * BKB2;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t.rb, (lds_ptr_t)(slot + SLOT_A + (wave * 8 + j) * 1024), 16,
                                               in ? voff[j] + kb0 : 0x7ffffff0, 0, 0, 0);
  };
  auto issue_a = [&](int st) {
    uint8_t* slot = smem + (st & 1) * SLOT;
    const bool in = st < s1;
    const int kb0 = st * BKB2;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t.ra, (lds_ptr_t)(slot + (wave * 8 + j) * 1024), 16,
                                               in ? voff[j] + kb0 : 0x7ffffff0, 0, 0, 0);
    if (SP) {
      // scale pair (st + 1) / 2, half (st + 1) % 2 (A rows, then B rows)
      issue_scales((st + 1) >> 1, (st + 1) & 1);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(t.rsa, (lds_ptr_t)(slot + OFF_SA + h * 4 * BM + wave * 256), 4,
                                                 in ? srow + st * 8 + h * 4 : 0x7ffffff0, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(t.rsb, (lds_ptr_t)(slot + OFF_SB + h * 4 * BN + wave * 256), 4,
                                                 in ? srow + st * 8 + h * 4 : 0x7ffffff0, 0, 0, 0);
      }
    }
  };
  auto issue = [&](int st) {
    issue_a(st);
    issue_b(st);
  };

  const int lrow = lane & 31;
  const int khalf = lane >> 5;
  int offa[4][TI], offb[4][TJ];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = wy * WM + i * 32 + lrow;
      offa[kk][i] = row * BKB2 + (((kk * 2 + khalf) ^ swz8r(row)) << 4);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int row = wx * WN + j * 32 + lrow;
      offb[kk][j] = SLOT_A + row * BKB2 + (((kk * 2 + khalf) ^ swz8r(row)) << 4);
    }
  }
  const int offsa = OFF_SA + (wy * WM + lrow) * 4;
  const int offsb = OFF_SB + (wx * WN + lrow) * 4;
  const int sshift = 8 * khalf;

  // All four K = 64 fragment sets of a stage live in registers (F[kk]), so a
  // slot is fully read two segments into the stage.  Two barriers per stage:
  // B1 after segment 2 (slot consumed -> refill it with stage s+2) and B2
  // before segment 4 (stage s+1 landed -> start reading it), which gives the
  // refill a stage and a half of lead time with two slots.
  i32x4 fa[4][TI], fb[4][TJ];
  uint32_t sa[2][TI], sb[2][TJ];   // raw scale dwords (blocks 0-3 / 4-7 of the stage)
  auto read_frag = [&](int kk, const uint8_t* slot) {
#pragma unroll
    for (int i = 0; i < TI; ++i) fa[kk][i] = *reinterpret_cast<const i32x4*>(slot + offa[kk][i]);
#pragma unroll
    for (int j = 0; j < TJ; ++j) fb[kk][j] = *reinterpret_cast<const i32x4*>(slot + offb[kk][j]);
  };
  // scale dword h (blocks 4h..4h+3) of stage st, read from `slot` (or, SP,
  // from ring entry (st / 2) % 3 at dword 2 * (st % 2) + h of the row)
  const int ringa = SCL_OFF + (wy * WM + lrow) * 16, ringb = SCL_OFF + BM * 16 + (wx * WN + lrow) * 16;
  auto read_scales = [&](int h, const uint8_t* slot, int st) {
    if (SP) {
      const int o = ((st >> 1) % 3) * SCL_BUF + (2 * (st & 1) + h) * 4;
#pragma unroll
      for (int i = 0; i < TI; ++i) sa[h][i] = *reinterpret_cast<const uint32_t*>(smem + ringa + o + i * 512);
#pragma unroll
      for (int j = 0; j < TJ; ++j) sb[h][j] = *reinterpret_cast<const uint32_t*>(smem + ringb + o + j * 512);
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i) sa[h][i] = *reinterpret_cast<const uint32_t*>(slot + offsa + h * 4 * BM + i * 128);
#pragma unroll
      for (int j = 0; j < TJ; ++j) sb[h][j] = *reinterpret_cast<const uint32_t*>(slot + offsb + h * 4 * BN + j * 128);
    }
  };
  // 16 MFMAs of segment KK: the lane's block is 2*KK + khalf, i.e. byte
  // 2*(KK%2) + khalf of scale dword KK/2; shifting by 8*khalf leaves it at
  // byte 0 (opsel 0) or byte 2 (opsel 2).
#define MX_SEG(KK, OPS)                                                                                 \
  _Pragma("unroll") for (int i = 0; i < TI; ++i)                                                        \
  _Pragma("unroll") for (int j = 0; j < TJ; ++j) {                                                      \
    const i32x8 a8 = {fa[KK][i][0], fa[KK][i][1], fa[KK][i][2], fa[KK][i][3], 0, 0, 0, 0};              \
    const i32x8 b8 = {fb[KK][j][0], fb[KK][j][1], fb[KK][j][2], fb[KK][j][3], 0, 0, 0, 0};              \
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                                        \
        a8, b8, acc[i][j], 4, 4, OPS, sa[(KK) / 2][i] >> sshift, OPS, sb[(KK) / 2][j] >> sshift);       \
  }
  // Reads for later segments go out two per MFMA at the front of a segment,
  // so each has most of the segment (16 x 32 cycles) to land.
#define MX_INTERLEAVE(NDS)                                              \
  _Pragma("unroll") for (int q = 0; q < (NDS) / 2; ++q) {               \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  \
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                  \
  }                                                                     \
  __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ - (NDS) / 2, 0);  \
  __builtin_amdgcn_sched_barrier(0);

  if (SP) {
    issue_scales(s0 >> 1, 0);
    issue_scales(s0 >> 1, 1);
  }
  issue(s0);
  issue(s0 + 1);
  wait_vmcnt<LPS>();
  block_barrier();
  read_frag(0, smem + (s0 & 1) * SLOT);
  read_scales(0, smem + (s0 & 1) * SLOT, s0);
  for (int s = s0; s < s1; ++s) {
    const uint8_t* cur = smem + (s & 1) * SLOT;
    const uint8_t* nxt = smem + ((s + 1) & 1) * SLOT;
    read_frag(1, cur);
    read_scales(1, cur, s);
    read_frag(2, cur);
    MX_SEG(0, 0)
    MX_INTERLEAVE(2 * (TI + TJ) + 4)
    read_frag(3, cur);
    MX_SEG(1, 2)
    MX_INTERLEAVE(TI + TJ)
    // B1: every wave has read all of `cur`; refill it with stage s+2, one
    // load after each MFMA of segments 2 and 3 (A part, then B part): the
    // direct-to-LDS loads of the four waves take the texture unit about
    // 16 cycles each, so issued in a burst they fill its queue and block the
    // wave, and with it the MFMA stream, until the queue drains.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    block_barrier();
    issue_a(s + 2);
    MX_SEG(2, 0)
#pragma unroll
    for (int q = 0; q < LA; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ - LA, 0);
    __builtin_amdgcn_sched_barrier(0);
    // B2: this wave's loads of stage s+1 have landed (only the LA loads of
    // stage s+2 issued above may still be in flight); after the barrier
    // every wave's have.
    wait_vmcnt<LA>();
    block_barrier();
    read_scales(0, nxt, s + 1);
    read_frag(0, nxt);
    issue_b(s + 2);
    MX_SEG(3, 2)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#undef MX_SEG
#undef MX_INTERLEAVE
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// C[m0 + r, n0 + c] = acc for rows below m_end and columns below N, through
// LDS: each wave stages half of its 128 x 128 fp32 tile (64 rows, row pitch
// 136 floats so the two half-waves' writes fall in different banks), then
// writes whole rows with 8- or 16-byte stores.  Starts with a barrier (every
// wave is done with the LDS of the K loop).
template <bool SP>
__device__ __forceinline__ void mx_tile_store(uint8_t* smem, void* c, int64_t ldc, int c_bf16, int N, int m0,
                                              int m_end, int n0,
                                              const f32x16 (&acc)[MxTile<SP>::TI][MxTile<SP>::TJ]) {
  using C = MxTile<SP>;
  constexpr int WM = C::WM, WN = C::WN, NWX = C::NWX, TI = C::TI, TJ = C::TJ;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));   // formed per tile (see mx_tile_mainloop)
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wy = wave / NWX, wx = wave % NWX;
  const int lrow = lane & 31;
  const int khalf = lane >> 5;
  block_barrier();
  constexpr int EP_PITCH = WN + 8;
  float* ep = reinterpret_cast<float*>(smem) + wave * (WM / 2) * EP_PITCH;
  const bool vec_ok = (ldc % 4) == 0;
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
        if (c_bf16) {
          uint16_t* dst = reinterpret_cast<uint16_t*>(c) + (size_t)row * ldc + col;
          if (vec_ok && col + 3 < N) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            // non-temporal: C is not read again here, and the L2 keeps the A/B panels
            __builtin_nontemporal_store(u32x2{pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3])},
                                        reinterpret_cast<u32x2*>(dst));
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (col + q < N) dst[q] = (uint16_t)f32_to_bf16_rne(v[q]);
          }
        } else {
          float* dst = reinterpret_cast<float*>(c) + (size_t)row * ldc + col;
          if (vec_ok && col + 3 < N) {
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (col + q < N) dst[q] = v[q];
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
  }
}

}  // namespace mxk
