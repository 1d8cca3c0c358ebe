// W4A16 decode GEMV / skinny GEMM for gfx950: y[m, n] = sum_k x[m, k] W_hat[n, k]
// with bf16 activations and MXFP4 weights (weights compressed, arithmetic in
// 16-bit: "Extreme Quantization and Precision Engineering", section "Key
// points"; decode is bound by streaming weight bytes: "NVFP4 Architecture",
// section "The Problem").
//
// The weights are streamed once from HBM and dequantized on chip: 16 code
// bytes (one 32-element MX block) expand with v_cvt_scalef32_pk_bf16_fp4 into
// 32 bf16 weights equal to q * 2^e exactly (at most 2 significant bits), so
// every product with a bf16 activation is exact in fp32 and only the fp32
// summation order differs from the plain definition.
//
// Three kernels:
//  * M = 1 is bound by HBM: many small workgroups, split-K across waves,
//    v_dot2_f32_bf16 on the VALU, the lane's partial sums reduced at the end.
//  * M = 2, 3 (and any M when K is not a multiple of 256): dot2 again, each
//    weight pair converted once and used for all M rows, activations staged
//    in LDS once per workgroup and window.
//  * M = 4 .. 16: one dot2 per weight pair and activation row would make the
//    VALU the bound, so the matrix cores take the products (bf16 MFMA).
// Weights in the wider MX elements (MXFP8 E4M3 / E5M2, MXFP6 E2M3 / E3M2:
// W8A16 / W6A16) take the second kernel for M <= 3 (and any M when K is not a
// multiple of 256) and a matrix-core kernel of the third kind otherwise, with
// the block's 32 / 24 code bytes expanded by the matching scaled conversion
// (mx_expand.h).
#include "mx_device.h"
#include "mx_expand.h"
#include "mx_kernels.h"

namespace mxk {

// Weight codes and scales are read once per call: non-temporal loads (cache
// policy bit NT) keep the weight stream from displacing the activations.
constexpr int GV_NT = 2;

constexpr int GV_T = 256;              // 4 waves
constexpr int GV_WIN = 64 * 32;        // K elements per window (64 lanes x 1 block)
constexpr int GV_SK_RB = 16;           // weight rows per workgroup of the small-M kernel

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
// weight rows (16: every workgroup reads the whole activation row, so fewer,
// larger workgroups read it fewer times); its four waves take the
// 2048-element windows of K in turn (wave w: windows w, w+4, ...), so each
// wave streams RB x 1 KiB of codes per window while reading only its own
// 4 KiB slice of each activation row.  The
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

// Moderate M (VALU-bound), and every M for the wider elements.  A workgroup
// of 8 waves owns 8 x RB weight rows (RB per wave) and walks the windows of K
// together.  Per window:
//  * the activations of all M rows (M x 4 KiB) are copied into LDS by the
//    LDS-DMA path (buffer_load ... lds), one buffer ahead, in a layout where
//    chunk q (16 bytes) of lane l's block sits at (q * 64 + l) * 16, so the
//    ds_read_b128 of a given q across the wave is conflict-free;
//  * each wave loads its RB blocks' codes (16 / 24 / 32 bytes for E2M1 /
//    FP6 / FP8 elements) and scale bytes one window ahead;
//  * each lane converts its RB blocks once (RB x 16 bf16 pairs in registers)
//    and then, per activation row m, reads its 64 activation bytes from LDS
//    and issues RB x 16 dot2.
// Two barriers per window: after the counted wait that covers this window's
// copy, and after the arithmetic (before the buffer is refilled).
constexpr int GL_T = 512;              // 8 waves
constexpr int GV_LG_RB = 4;            // weight rows per wave of the large-M kernel
constexpr int GV_LG_MIN_M = 2;         // smallest M that takes the large-M kernel



// F: element format (E4M3 0, E5M2 1, E2M3 2, E3M2 3, E2M1 4).  MT: activation
// rows the kernel is built for; E2M1 instantiates every M exactly (M = MT),
// the wider formats round M up to MT in {1, 2, 4, 8, 16} and take the rows
// count at run time (m_rows; rows m >= m_rows are staged as zeros and skipped).
template <int F, int MT, int RB>
__global__ __launch_bounds__(GL_T) void k_gemv_lg(const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wc,
                                                  const uint8_t* __restrict__ ws, int N, int K,
                                                  uint16_t* __restrict__ y, int64_t ldy, int m_rows) {
  constexpr int MP = (MT + 1) & ~1;                // staged rows, even: every wave issues MP / 2 copies
  constexpr int XCH = MP * 4;                      // 1 KiB copies per window (4 per activation row)
  constexpr int XPW = XCH / 8;                     // copies per wave
  constexpr int DW = MxElem<F>::DW;                // code dwords of one 32-element block
  constexpr int CB = DW * 4;                       // ... bytes
  const int M = F == 4 ? MT : m_rows;
  __shared__ __attribute__((aligned(16))) uint8_t sx[2][MP * 4096];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * (8 * RB) + wave * RB;
  const int KB = K / 32 * CB, KS = K / 32;
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
          (void*)(x + (size_t)(m < M ? m : 0) * ldx), 0, __builtin_amdgcn_readfirstlane(m < M ? K * 2 : 0), 0x00020000);
      // LDS chunk q * 64 + lane holds window chunk 4 * lane + q
      const int k = w * GV_WIN + (4 * lane + q) * 8;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(&sx[b][(m * 256 + q * 64) * 16]), 16,
                                               k < K ? k * 2 : oob, 0, 0, 0);
    }
  };
  uint32_t sc[2][RB];
  uint32_t cw[2][RB][DW];
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  auto issue = [&](int b, int w) {
    const int kb = w * 64 + lane;
    const bool kok = kb < KS;
#pragma unroll
    for (int r = 0; r < RB; ++r) sc[b][r] = __builtin_amdgcn_raw_buffer_load_b8(rws, kok ? r * KS + kb : oob, 0, GV_NT);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int o0 = kok ? r * KB + kb * CB : oob, o1 = kok ? r * KB + kb * CB + 16 : oob;
      const u32x4 v0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwc, o0, 0, GV_NT));
#pragma unroll
      for (int d = 0; d < 4; ++d) cw[b][r][d] = v0[d];
      if constexpr (DW == 8) {
        const u32x4 v1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwc, o1, 0, GV_NT));
#pragma unroll
        for (int d = 0; d < 4; ++d) cw[b][r][4 + d] = v1[d];
      } else if constexpr (DW == 6) {
        const u32x2 v1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rwc, o1, 0, GV_NT));
        cw[b][r][4] = v1[0];
        cw[b][r][5] = v1[1];
      }
    }
  };
  constexpr int LOADS = XPW + (DW == 4 ? 2 : 3) * RB;   // vector-memory ops per window and wave

  float acc[RB][MT];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  auto compute = [&](int b) {
    bf16x2 wv[RB][16];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const float s = pow2f((int)sc[b][r] - 127);   // byte 0 (zero block) gives +0.0
      uint32_t o[16];
      expand_block_bf16<F>(cw[b][r], s, o);
#pragma unroll
      for (int i = 0; i < 16; ++i) __builtin_memcpy(&wv[r][i], &o[i], 4);
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
    for (int m = 0; m < MT; ++m) {
      if (m >= M) break;                           // uniform (wider formats: rows counted at run time)
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

  // reduce the RB x MT sums over the wave; lane l ends up owning one of them
  constexpr int V = (RB * MT <= 8) ? 8 : (RB * MT <= 16) ? 16 : (RB * MT <= 32) ? 32 : 64;
  static_assert(RB * MT <= 64, "at most 64 sums per wave");
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = i < RB * MT ? acc[i / MT][i % MT] : 0.0f;
  int id;
  const float tot = wave_transpose_sum<V>(v, lane, &id);
  const int r = id / MT, m = id - r * MT;
  if ((lane & (64 / V - 1)) == 0 && id < RB * MT && m < M && n0 + r < N)
    y[(size_t)m * ldy + n0 + r] = (uint16_t)f32_to_bf16_rne(tot);
}

// Skinny M (4..16 rows) on the matrix cores.  With one dot2 per weight pair
// and activation row the VALU caps the large-M kernel far below the weight
// stream; v_mfma_f32_16x16x32_bf16 takes the arithmetic instead (activation
// rows padded to 16; bf16 x bf16 products are exact and the instruction
// accumulates them without truncation).
//
// A workgroup of 8 waves owns 32 weight rows (two 16-row column groups) and
// walks K in 512-element chunks through a ring of four LDS slots, three
// chunks in flight, starting at a chunk that depends on the workgroup (so
// that concurrent workgroups spread over the weight columns).  A chunk's weight codes (32 rows x 256
// bytes) and activations (8 or 16 rows x 1 KiB) arrive by LDS-DMA copies of
// whole cache lines,
// each byte once per workgroup; wave w then covers column group w & 1 and MX
// blocks 4 (w >> 1) .. + 3 of the chunk, one MFMA per block.  In MFMA block
// b, lane l (row or column l % 16, lane group g = l / 16) takes K elements
// 32b + 8g .. + 7: 16 activation bytes (one LDS read) and one code dword,
// expanded with the block's scale into 8 bf16 weights (exactly q * 2^e) by
// v_cvt_scalef32_pk_bf16_fp4.  LDS rows are XOR-swizzled in 16-byte units so
// that these reads are free of bank conflicts.  One barrier per chunk; the
// four quarter-K partial tiles of each column group meet in LDS at the end.
constexpr int GM_T = 512;              // 8 waves
constexpr int GV_MF_MIN_M = 4;         // smallest M that takes the matrix-core kernel
constexpr int GM_CK = 512;             // K elements per chunk

template <int M>
__global__ __launch_bounds__(GM_T) void k_gemv_mf(const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wc,
                                                  const uint8_t* __restrict__ ws, int N, int K,
                                                  uint16_t* __restrict__ y, int64_t ldy) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  constexpr int MA = M <= 8 ? 8 : 16;              // activation rows staged
  constexpr int R = 4;                             // ring slots; chunks in flight: R - 1
  constexpr int WOFF = MA * 1024;                  // weight codes after the activations
  constexpr int SLOT = WOFF + 32 * 256;
  // the ring, and after the loop the partial tiles (float [8][16][16])
  __shared__ __attribute__((aligned(1024))) uint8_t smem[R * SLOT];
  auto ring = [&](int p) -> uint8_t* { return smem + p * SLOT; };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int cg = wave & 1, qd = wave >> 1;         // column group, quarter of the chunk's blocks
  const int n0 = blockIdx.x * 32;
  const int KB = K / 2, KS = K / 32;
  const int rows_ok = __builtin_amdgcn_readfirstlane(max(0, min(32, N - n0)));
  const __amdgpu_buffer_rsrc_t rwc = __builtin_amdgcn_make_buffer_rsrc((void*)(wc + (size_t)n0 * KB), 0, rows_ok * KB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc((void*)(ws + (size_t)n0 * KS), 0, rows_ok * KS, 0x00020000);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, 0, __builtin_amdgcn_readfirstlane((int)(((M - 1) * ldx + K) * 2)), 0x00020000);
  const int nck = (K + GM_CK - 1) / GM_CK;
  const int np = (nck + R - 1) / R * R;            // chunk slots the loop runs through (uniform)
  const int rot = blockIdx.x % np;                 // position v holds chunk (v + rot) mod np
  // Out-of-range parts add 2^30 to an offset, which puts the load past its
  // buffer (every range is below 2^30 bytes) so that it returns zeros.
  constexpr uint32_t FAR = 0x40000000u;

  // Copies of chunk v into slot p.  Weights: copy `wave`, lane l -> row
  // 4 wave + l / 16, position l % 16, holding block (l % 16) ^ (row & 15).
  // Activations: copy m < MA (wave m & 7), lane l -> row m, position l,
  // holding 16-byte piece l ^ m (zeros for rows m >= M).  Scale bytes of this wave's four
  // blocks go to registers.
  const int wrow = 4 * wave + (lane >> 4), wpos = lane & 15;
  uint32_t sc[R];
  auto issue = [&](int p, int v) {
    // chunk at position v (positions past the loop's end copy zeros)
    const int c = v >= np ? nck : (v + rot < np ? v + rot : v + rot - np);
    const int b0 = c * (GM_CK / 32);               // first block of the chunk
    uint8_t* slot = ring(p);
    {
      const int blk = b0 + (wpos ^ (wrow & 15));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rwc, (lds_ptr_t)(slot + WOFF + wave * 1024), 16,
                                               blk < KS ? (uint32_t)(wrow * KB + blk * 16) : FAR, 0, 0, GV_NT);
    }
#pragma unroll
    for (int e = 0; e < MA / 8; ++e) {             // rows m >= M copy zeros (no memory traffic)
      const int m = wave + 8 * e;
      const int k = c * GM_CK + 8 * (lane ^ m);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(slot + m * 1024), 16,
                                               (m < M && k < K) ? (uint32_t)(m * ldx + k) * 2 : FAR, 0, 0, 0);
    }
    const int sb = b0 + 4 * qd;
    sc[p] = __builtin_amdgcn_raw_buffer_load_b32(rws, sb < KS ? (uint32_t)((16 * cg + j) * KS + sb) : FAR, 0, GV_NT);
  };
  constexpr int LPC = 2 + MA / 8;                  // vector-memory ops per chunk and wave

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](int p) {
    const uint8_t* slot = ring(p);
    const int r = 16 * cg + j;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int b = 4 * qd + s;                    // block within the chunk
      // (rows j >= MA repeat rows j - 8; their outputs are never stored)
      const int ja = j & (MA - 1);
      const u32x4 av = *reinterpret_cast<const u32x4*>(slot + ja * 1024 + (((4 * b + g) ^ ja) << 4));
      const uint32_t w = *reinterpret_cast<const uint32_t*>(slot + WOFF + r * 256 + ((b ^ (r & 15)) << 4) + 4 * g);
      const float sf = pow2f((int)((sc[p] >> (8 * s)) & 0xff) - 127);   // byte 0 gives +0.0
      bf16x2 w2[4];
      w2[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 0);
      w2[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 1);
      w2[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 2);
      w2[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 3);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, w2), acc,
                                                    0, 0, 0);
    }
  };

  // Position v sits in slot v % R.  After the barrier of position v every
  // wave is done with position v - 1, whose slot then takes position v + R - 1.
  // Chunks past the end copy zeros; the trip count is uniform.
#pragma unroll
  for (int p = 0; p < R - 1; ++p) issue(p, p);
  for (int v0 = 0; v0 < nck; v0 += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      // this wave's copies of position v0 + u have landed and its reads of
      // the previous one are done; after the barrier the same holds for all waves
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      wait_vmcnt<(R - 2) * LPC>();
      block_barrier();
      issue((u + R - 1) % R, v0 + u + R - 1);
      compute(u);
    }
  }
  wait_vmcnt<0>();

  // lane l holds rows 4g .. 4g + 3 of column j of the wave's 16 x 16 tile
  block_barrier();                                 // every wave is done with the ring
  float(*red)[16][16] = reinterpret_cast<float(*)[16][16]>(smem);
#pragma unroll
  for (int q = 0; q < 4; ++q) red[wave][4 * g + q][j] = acc[q];
  __syncthreads();
  const int t = threadIdx.x;
  const int c = t >> 8, i = (t >> 4) & 15, jj = t & 15;
  float sum = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) sum += red[c + 2 * q][i][jj];
  const int n = n0 + 16 * c + jj;
  if (i < M && n < N) y[(size_t)i * ldy + n] = (uint16_t)f32_to_bf16_rne(sum);
}

// The same matrix-core route for MXFP8 / MXFP6 weights (W8A16 / W6A16,
// 4 <= M <= 16, K % 256 == 0).  A block's codes are 32 (FP8) or 24 (FP6)
// bytes, and the whole block goes to one lane: in chunk position s of its
// wave, lane l (row or column l % 16, lane group g = l / 16) holds block
// 4 qd + g of its row, expands its 32 codes at once (mx_expand.h; for FP6 one
// 32-wide conversion), and the four MFMAs of the step take its elements
// 8 i .. 8 i + 7, i = 0 .. 3 -- the matrix core sums over the lane groups,
// so MFMA i adds piece i of four different blocks, and over i every element
// of the four blocks once.  The activations are staged as in k_gemv_mf and
// read to match (piece 4 b + i of row m).  A row's 16 blocks of a chunk sit
// in LDS at positions XOR-swizzled by the row (block p ^ (row & 15) at
// position p), filled by LDS-DMA copies of 16 (FP8: two per wave and chunk)
// or 4 (FP6: six per wave and chunk) bytes per lane.  MA: activation rows
// staged (8 or 16); the rows count M is taken at run time.
template <int F, int MA>
__global__ __launch_bounds__(GM_T) void k_gemv_mfw(const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wc,
                                                   const uint8_t* __restrict__ ws, int N, int K,
                                                   uint16_t* __restrict__ y, int64_t ldy, int M) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  static_assert(F >= 0 && F <= 3 && (MA == 8 || MA == 16), "wide formats, 8 or 16 staged rows");
  constexpr int R = 4;                             // ring slots; chunks in flight: R - 1
  constexpr int CB = MxElem<F>::DW * 4;            // code bytes per block: 32 or 24
  constexpr int PB = CB == 32 ? 16 : 4;            // bytes per lane of a weight copy
  constexpr int WROW = 16 * CB;                    // a row's bytes in one chunk
  constexpr int WOFF = MA * 1024;                  // weight codes after the activations
  constexpr int SLOT = WOFF + 32 * WROW;
  constexpr int WPW = 32 * WROW / (64 * PB) / 8;   // weight copies per wave and chunk (2 or 6)
  static_assert(WPW * 8 * 64 * PB == 32 * WROW && CB % PB == 0, "whole copies of whole blocks");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[R * SLOT];
  auto ring = [&](int p) -> uint8_t* { return smem + p * SLOT; };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int cg = wave & 1, qd = wave >> 1;         // column group, quarter of the chunk's blocks
  const int n0 = blockIdx.x * 32;
  const int KB = K / 32 * CB, KS = K / 32;
  const int rows_ok = __builtin_amdgcn_readfirstlane(max(0, min(32, N - n0)));
  const __amdgpu_buffer_rsrc_t rwc = __builtin_amdgcn_make_buffer_rsrc((void*)(wc + (size_t)n0 * KB), 0, rows_ok * KB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc((void*)(ws + (size_t)n0 * KS), 0, rows_ok * KS, 0x00020000);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, 0, __builtin_amdgcn_readfirstlane((int)(((M - 1) * ldx + K) * 2)), 0x00020000);
  const int nck = (K + GM_CK - 1) / GM_CK;
  const int np = (nck + R - 1) / R * R;            // chunk slots the loop runs through (uniform)
  const int rot = blockIdx.x % np;                 // position v holds chunk (v + rot) mod np
  constexpr uint32_t FAR = 0x40000000u;            // past every buffer: the load returns zeros

  uint32_t sc[R];
  auto issue = [&](int p, int v) {
    const int c = v >= np ? nck : (v + rot < np ? v + rot : v + rot - np);
    const int b0 = c * (GM_CK / 32);               // first block of the chunk
    uint8_t* slot = ring(p);
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
      const int ci = wave * WPW + i;               // copy ci: pieces 64 ci .. 64 ci + 63 of the slot
      const int pc = ci * 64 + lane;
      const int row = pc / (WROW / PB), pr = pc % (WROW / PB);
      const int pos = pr / (CB / PB), part = pr % (CB / PB);
      const int blk = b0 + (pos ^ (row & 15));
      const uint32_t off = blk < KS ? (uint32_t)(row * KB + blk * CB + part * PB) : FAR;
      if constexpr (PB == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rwc, (lds_ptr_t)(slot + WOFF + ci * 64 * PB), 16, off, 0, 0, GV_NT);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rwc, (lds_ptr_t)(slot + WOFF + ci * 64 * PB), 4, off, 0, 0, GV_NT);
    }
#pragma unroll
    for (int e = 0; e < MA / 8; ++e) {             // rows m >= M copy zeros (no memory traffic)
      const int m = wave + 8 * e;
      const int k = c * GM_CK + 8 * (lane ^ m);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(slot + m * 1024), 16,
                                               (m < M && k < K) ? (uint32_t)(m * ldx + k) * 2 : FAR, 0, 0, 0);
    }
    const int sb = b0 + 4 * qd;
    sc[p] = __builtin_amdgcn_raw_buffer_load_b32(rws, sb < KS ? (uint32_t)((16 * cg + j) * KS + sb) : FAR, 0, GV_NT);
  };
  constexpr int LPC = WPW + MA / 8 + 1;            // vector-memory ops per chunk and wave

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](int p) {
    const uint8_t* slot = ring(p);
    const int r = 16 * cg + j, b = 4 * qd + g;     // the lane's row and block
    const uint8_t* wp = slot + WOFF + r * WROW + (b ^ (r & 15)) * CB;
    uint32_t w[MxElem<F>::DW];
    if constexpr (CB == 32) {
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(wp), w1 = *reinterpret_cast<const u32x4*>(wp + 16);
#pragma unroll
      for (int d = 0; d < 4; ++d) { w[d] = w0[d]; w[4 + d] = w1[d]; }
    } else {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        const u32x2 t = *reinterpret_cast<const u32x2*>(wp + 8 * d);
        w[2 * d] = t[0];
        w[2 * d + 1] = t[1];
      }
    }
    const float sf = pow2f((int)((sc[p] >> (8 * g)) & 0xff) - 127);   // byte 0 gives +0.0
    uint32_t o[16];
    expand_block_bf16<F>(w, sf, o);
    // (rows j >= MA repeat rows j - 8; their outputs are never stored)
    const int ja = j & (MA - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(slot + ja * 1024 + (((4 * b + i) ^ ja) << 4));
      const u32x4 bw = {o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bw), acc,
                                                    0, 0, 0);
    }
  };

  // the ring walk of k_gemv_mf
#pragma unroll
  for (int p = 0; p < R - 1; ++p) issue(p, p);
  for (int v0 = 0; v0 < nck; v0 += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      wait_vmcnt<(R - 2) * LPC>();
      block_barrier();
      issue((u + R - 1) % R, v0 + u + R - 1);
      compute(u);
    }
  }
  wait_vmcnt<0>();

  block_barrier();                                 // every wave is done with the ring
  float(*red)[16][16] = reinterpret_cast<float(*)[16][16]>(smem);
#pragma unroll
  for (int q = 0; q < 4; ++q) red[wave][4 * g + q][j] = acc[q];
  __syncthreads();
  const int t = threadIdx.x;
  const int c = t >> 8, i = (t >> 4) & 15, jj = t & 15;
  float sum = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) sum += red[c + 2 * q][i][jj];
  const int n = n0 + 16 * c + jj;
  if (i < M && n < N) y[(size_t)i * ldy + n] = (uint16_t)f32_to_bf16_rne(sum);
}

hipError_t launch_gemv(int fmt, const void* x, int64_t ldx, int64_t M, const uint8_t* wc, const uint8_t* ws, int64_t N,
                       int64_t K, void* y, int64_t ldy, hipStream_t st) {
  if (N == 0) return hipSuccess;
  if (fmt < 0 || fmt > 4 || M < 1 || M > 16) return hipErrorInvalidValue;
  if (fmt != 4 && M >= GV_MF_MIN_M && K % 256 == 0 && K < (1 << 25) && ((M - 1) * ldx + K) * 2 < (int64_t)0x3ffffff0) {
    const int grid = (int)((N + 31) / 32);
#define MX_GVMW(FF, MA) \
  hipLaunchKernelGGL((k_gemv_mfw<FF, MA>), dim3(grid), dim3(GM_T), 0, st, (const uint16_t*)x, ldx, wc, ws, (int)N, (int)K, (uint16_t*)y, ldy, (int)M)
#define MX_GVMWF(FF) case FF: if (M <= 8) MX_GVMW(FF, 8); else MX_GVMW(FF, 16); break;
    switch (fmt) { MX_GVMWF(0) MX_GVMWF(1) MX_GVMWF(2) MX_GVMWF(3) }
#undef MX_GVMWF
#undef MX_GVMW
    return hipGetLastError();
  }
  if (fmt != 4) {
    constexpr int RB = GV_LG_RB;
    const int grid = (int)((N + 8 * RB - 1) / (8 * RB));
    const int mt = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
#define MX_GVW(FF, MM) \
  case MM: hipLaunchKernelGGL((k_gemv_lg<FF, MM, RB>), dim3(grid), dim3(GL_T), 0, st, (const uint16_t*)x, ldx, wc, ws, (int)N, (int)K, (uint16_t*)y, ldy, (int)M); break;
#define MX_GVWF(FF)                                                                            \
  case FF:                                                                                     \
    switch (mt) { MX_GVW(FF, 1) MX_GVW(FF, 2) MX_GVW(FF, 4) MX_GVW(FF, 8) MX_GVW(FF, 16) }     \
    break;
    switch (fmt) { MX_GVWF(0) MX_GVWF(1) MX_GVWF(2) MX_GVWF(3) }
#undef MX_GVWF
#undef MX_GVW
    return hipGetLastError();
  }
  if (M < GV_LG_MIN_M) {
    constexpr int RB = GV_SK_RB;
    const int grid = (int)((N + RB - 1) / RB);
#define MX_GVS(MM) case MM: hipLaunchKernelGGL((k_gemv_sk<MM, RB>), dim3(grid), dim3(GV_T), 0, st, (const uint16_t*)x, ldx, wc, ws, (int)N, (int)K, (uint16_t*)y, ldy); break;
    switch ((int)M) {
      MX_GVS(1)
      default: return hipErrorInvalidValue;
    }
#undef MX_GVS
    return hipGetLastError();
  }
  if (M >= GV_MF_MIN_M && K % 256 == 0 && K < (1 << 25) && ((M - 1) * ldx + K) * 2 < (int64_t)0x3ffffff0) {
    const int grid = (int)((N + 31) / 32);
#define MX_GVM(MM) case MM: hipLaunchKernelGGL((k_gemv_mf<MM>), dim3(grid), dim3(GM_T), 0, st, (const uint16_t*)x, ldx, wc, ws, (int)N, (int)K, (uint16_t*)y, ldy); break;
    switch ((int)M) {
      MX_GVM(4) MX_GVM(5) MX_GVM(6) MX_GVM(7) MX_GVM(8) MX_GVM(9) MX_GVM(10) MX_GVM(11) MX_GVM(12)
      MX_GVM(13) MX_GVM(14) MX_GVM(15) MX_GVM(16)
      default: return hipErrorInvalidValue;
    }
#undef MX_GVM
    return hipGetLastError();
  }
  constexpr int RB = GV_LG_RB;
  const int grid = (int)((N + 8 * RB - 1) / (8 * RB));
#define MX_GVL(MM) case MM: hipLaunchKernelGGL((k_gemv_lg<4, MM, RB>), dim3(grid), dim3(GL_T), 0, st, (const uint16_t*)x, ldx, wc, ws, (int)N, (int)K, (uint16_t*)y, ldy, (int)M); break;
  switch ((int)M) {
    MX_GVL(2) MX_GVL(3) MX_GVL(4) MX_GVL(5) MX_GVL(6) MX_GVL(7) MX_GVL(8)
    MX_GVL(9) MX_GVL(10) MX_GVL(11) MX_GVL(12) MX_GVL(13) MX_GVL(14) MX_GVL(15) MX_GVL(16)
    default: return hipErrorInvalidValue;
  }
#undef MX_GVL
  return hipGetLastError();
}

}  // namespace mxk
