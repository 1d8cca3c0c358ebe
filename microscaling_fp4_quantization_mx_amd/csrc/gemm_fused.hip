// Dynamic MXFP4 activation quantization fused with the (grouped) W4A4 GEMM in
// one persistent kernel, for gfx950.
//
// The activations of every layer are quantized on the fly ("How Microscaling
// FP4 (MXFP4) Halves Memory Bandwidth", section "Native Pre-Training vs.
// Post-Training Quantization"), so a separate quantize launch would stream the
// bf16 activations through HBM, write the codes back and only then start the
// product ("NVFP4 Architecture", section "2. The Microarchitectural Limits of
// Software Workarounds": re-quantization on every layer).  Here the same
// workgroups do both, and the two overlap.
//
// Work is split per XCD: the 256 x 256 output tiles (grouped: each expert's
// rows in tiles that never straddle experts) form one list, cut into eight
// contiguous chunks, and the workgroups running on XCD x (read from the
// hardware register XCC_ID) take the jobs of chunk x in ticket order from an
// atomic counter.  A chunk's jobs, in ticket order: the quantization of the
// activation rows its tiles read (32 rows per job, the rows of the next tile
// row ahead of the tiles of the current one), its tiles, and last, when the
// chunk's tile count is not a multiple of the XCD's workers, the remaining
// tiles split along K into S parts (so the last round is 1/S of a tile long).
// A tile waits for the quantize jobs of its rows; those jobs hold smaller
// tickets of the same chunk, so workgroups that are already running own them,
// and they wait for nothing: every wait ends.  Producer and consumer run on
// the same XCD and meet in its L2.  A split tile's parts store fp32 partial
// tiles; the last to arrive adds them in part order (the result does not
// depend on arrival order) and writes C.
//
// Counters (tickets, per tile row the finished quantize jobs, per split tile
// the arrived parts) are zeroed by k_fused_reset, launched just before.
#include "mx_device.h"
#include "gemm_mx_tile.h"
#include "mx_kernels.h"

namespace mxk {

constexpr int FQ_ROWS = 32;          // activation rows per quantize job
constexpr int F_CTR_STRIDE = 256;    // counters per chunk (u32)
constexpr int F_READY0 = 16;         // counter index of the first tile row's quantize count
constexpr int F_SPLIT0 = 128;        // counter index of the first split tile's part count
constexpr int F_PART_FLOATS = 65536; // one fp32 256 x 256 partial tile
constexpr int F_MAX_SPLIT = 32;      // partial tiles per chunk
constexpr int F_MAX_PARTS = 4;       // K parts per split tile
constexpr int F_GR = 4;              // tile rows per raster group
constexpr int F_OFFL_BYTES = 32768;  // group offsets staged in LDS (at most 8191 groups)
constexpr float F_QCOST = 0.42f;     // a 32-row bf16 quantize job in units of one tile (same K; measured)
constexpr int F_MAXR = 112;          // tile rows per chunk
constexpr int F_JMAX = 1024;         // jobs per chunk
static_assert(F_READY0 + F_MAXR <= F_SPLIT0 && F_SPLIT0 + F_MAX_SPLIT <= F_CTR_STRIDE, "counter layout");

enum { FJ_Q = 0, FJ_G = 1, FJ_P = 2 };
__device__ __forceinline__ uint32_t fjob(int type, int a, int b) { return (uint32_t)type << 28 | (uint32_t)a << 14 | b; }

struct FusedParams {
  const void* x;          // activations [M, K] (fp32 or bf16), pitch ldx elements
  int64_t ldx;
  int x_bf16;
  uint8_t* a_codes;       // quantized activations [M, K/2]
  uint8_t* a_scales;      // [M, K/32]
  const uint8_t* b_codes; // [G*N, K/2] (G = 1 dense)
  const uint8_t* b_scales;
  void* c;
  int64_t ldc;
  int c_bf16;
  int M, N, K;
  int groups;             // 0 = dense
  const int32_t* offsets; // [groups + 1]
  uint32_t* ctr;          // [nl * F_CTR_STRIDE] counters, zero at launch
  float* part;            // [nl * F_MAX_SPLIT] partial tiles
  int nl;                 // chunks (one per XCD)
  int wpl;                // workgroups per XCD
};

// Quantize rows [r0, r1) of the activations to MXFP4 (codes and E8M0 bytes
// identical to mx_quantize's): wave w takes rows r0 + w, r0 + w + 4, ...; a
// lane owns one 16-byte vector of a row, 64 consecutive vectors per load
// instruction, and a block's max |x| is reduced over the block's lanes.  Row
// addresses are scalar (buffer offsets), so a vector costs no address math.
// bf16 input is converted pairwise as packed bf16 (v_cvt_scalef32_pk_fp4_bf16,
// the same rounding as converting the fp32 values), its max |x| taken with
// packed 16-bit maxima.  Three batches of 12 loads per lane rotate, two in
// flight while one converts.  Ends with every store complete.
template <typename TIn>
__device__ __forceinline__ void fq_rows(const TIn* __restrict__ x, int64_t ldx, int r0, int r1, int K,
                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int EPL = 16 / (int)sizeof(TIn);
  constexpr int LPB = 32 / EPL;
  constexpr int QB = 12;                      // vectors per lane per batch
  int tix = threadIdx.x;
  asm volatile("" : "+v"(tix));   // formed per job, not held across the caller's loop
  const int lane = tix & 63, wave = tix >> 6;
  const int vpr = K / EPL;                    // vectors per row
  const int cpr = (vpr + 63) / 64;            // 64-vector chunks per row
  const int nrow = r1 - r0 > wave ? (r1 - r0 - wave + 3) / 4 : 0;
  const int items = __builtin_amdgcn_readfirstlane(nrow * cpr);   // (row, chunk) pairs of this wave
  const int wrow0 = __builtin_amdgcn_readfirstlane(r0 + wave);
  // the wave's rows, as 32-bit byte offsets from these bases; the input's
  // extent ends with the wave's last row, so the lanes past a row's end in
  // its last chunk read zeros there rather than beyond the tensor
  const int xbytes = nrow ? (int)((4 * (int64_t)(nrow - 1) * ldx + K) * (int64_t)sizeof(TIn)) : 0;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)wrow0 * ldx), 0, __builtin_amdgcn_readfirstlane(xbytes), 0x00020000);
  const int rspan = nrow ? 4 * (nrow - 1) + 1 : 0;   // rows from the wave's first to its last
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      codes + (size_t)wrow0 * (K / 2), 0, __builtin_amdgcn_readfirstlane(rspan * (K / 2)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      scales + (size_t)wrow0 * (K / 32), 0, __builtin_amdgcn_readfirstlane(rspan * (K / 32)), 0x00020000);
  // Every load and store is issued unconditionally (an offset past the
  // descriptor's extent reads zeros and drops the write), so the number of
  // memory operations in flight is the same on every path and the waits
  // before a batch's use count only what is older than that batch.
  constexpr int FAR = 0x7ffffff0;
  auto load = [&](u32x4 (&d)[QB], int it0) {
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int it = it0 + q;
      const int ri = it / cpr, ch = it - ri * cpr;   // uniform
      const bool in = it < items;
      const int so = in ? (int)((4 * ri) * ldx * (int64_t)sizeof(TIn)) + ch * 1024 : 0;
      d[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? lane * 16 : FAR, so, 0);
    }
  };
  auto convert = [&](const u32x4 (&d)[QB], int it0) {
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int it = it0 + q;
      const int ri = it / cpr, ch = it - ri * cpr;
      const int col = ch * 64 + lane;
      uint32_t am, out = 0;
      int e;
      if constexpr (EPL == 8) {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        u16x2 m = __builtin_elementwise_max(__builtin_bit_cast(u16x2, d[q][0] & 0x7fff7fffu),
                                            __builtin_bit_cast(u16x2, d[q][1] & 0x7fff7fffu));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, d[q][2] & 0x7fff7fffu));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, d[q][3] & 0x7fff7fffu));
        am = (uint32_t)max(m.x, m.y) << 16;
      } else {
        am = max(max(d[q][0] & 0x7fffffffu, d[q][1] & 0x7fffffffu), max(d[q][2] & 0x7fffffffu, d[q][3] & 0x7fffffffu));
      }
      if constexpr (LPB >= 2) am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0xb1, 0xf, 0xf, false));
      if constexpr (LPB >= 4) am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x4e, 0xf, 0xf, false));
      if constexpr (LPB >= 8) am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x141, 0xf, 0xf, false));
      e = mx_block_exp(am);
      const float sc = pow2f(e);
      if constexpr (EPL == 8) {
        // each source word passes through its own register first: without
        // that, this compiler feeds word 0 to all four conversions
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        uint32_t w0 = d[q][0], w1 = d[q][1], w2 = d[q][2], w3 = d[q][3];
        asm volatile("" : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, w0), sc, 0);
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, w1), sc, 1);
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, w2), sc, 2);
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, w3), sc, 3);
      } else {
        out = cvt_fp4x2<0>(out, ffrom(d[q][0]), ffrom(d[q][1]), sc);
        out = cvt_fp4x2<1>(out, ffrom(d[q][2]), ffrom(d[q][3]), sc);
      }
      const bool ok = it < items && col < vpr;
      const int row_off = it < items ? 4 * ri : 0;
      if constexpr (EPL == 8)
        __builtin_amdgcn_raw_buffer_store_b32(out, rc, ok ? lane * 4 : FAR, row_off * (K / 2) + ch * 256, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)out, rc, ok ? lane * 2 : FAR, row_off * (K / 2) + ch * 128, 0);
      __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(e + 127), rs,
                                           ok && (lane & (LPB - 1)) == 0 ? lane / LPB : FAR,
                                           row_off * (K / 32) + ch * (64 / LPB), 0);
    }
  };
  // three register batches in rotation: two are in flight while one converts
  u32x4 da[QB], db[QB], dc[QB];
  if (items > 0) load(da, 0);
  if (QB < items) load(db, QB);
  for (int it = 0; it < items; it += 3 * QB) {
    if (it + 2 * QB < items) load(dc, it + 2 * QB);
    convert(da, it);
    if (it + QB >= items) break;
    if (it + 3 * QB < items) load(da, it + 3 * QB);
    convert(db, it + QB);
    if (it + 2 * QB >= items) break;
    if (it + 4 * QB < items) load(db, it + 4 * QB);
    convert(dc, it + 2 * QB);
  }
  __syncthreads();   // waits for every store of the workgroup (vmcnt(0)) as well
}

__global__ void k_fused_reset(uint32_t* ctr, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) ctr[i] = 0u;
}

__global__ __launch_bounds__(256) void k_gemm_mx_fused(FusedParams p) {
  using T = MxTile<true>;
  constexpr int TI = T::TI, TJ = T::TJ;
  // one LDS object: the tile's buffers, then the job table, the tile-row
  // table and a few broadcast words (with several LDS objects the compiler
  // can no longer tell the direct-to-LDS loads' target from the fragment and
  // scale reads, and waits for every load before each such read)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::SMEM + F_JMAX * 4 + F_MAXR * 12 + 32];
  uint32_t* jt = reinterpret_cast<uint32_t*>(smem + T::SMEM);
  int (*rinfo)[3] = reinterpret_cast<int (*)[3]>(smem + T::SMEM + F_JMAX * 4);   // first row, row end, group
  int* sh = reinterpret_cast<int*>(smem + T::SMEM + F_JMAX * 4 + F_MAXR * 12);

  uint32_t xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  const int list = (int)(xcc & 15u) % p.nl;
  uint32_t* ctr = p.ctr + list * F_CTR_STRIDE;
  const int tid = threadIdx.x;
  const int tn_count = (p.N + T::BN - 1) / T::BN;
  const int nst = p.K / BK2;
  const int ng = p.groups ? p.groups : 1;

  // ---- this chunk's jobs, identical in every workgroup of the XCD, in ticket
  // order: the quantize jobs of the chunk's tile rows (row order), the whole
  // tiles in raster groups of up to F_GR tile rows of one group matrix
  // walking the columns (a column's tiles share the B panel, a row's tiles
  // the A panel), then the split parts.  Thread 0 forms the per-row figures,
  // then every thread places jobs.  Build-time arrays live in the (still free)
  // tile buffers.
  int* offl = reinterpret_cast<int*>(smem);                  // clamped group offsets
  int* rw = reinterpret_cast<int*>(smem + F_OFFL_BYTES);     // per local tile row, F_MAXR + 1 each:
  int* qpre = rw;                                            //   quantize jobs before the row
  int* tpre = rw + (F_MAXR + 1);                             //   whole tiles before the row
  int* tlo = rw + 2 * (F_MAXR + 1);                          //   the row's whole-tile columns [tlo, thi)
  int* thi = rw + 3 * (F_MAXR + 1);
  int* rg0 = rw + 4 * (F_MAXR + 1);                          //   its raster group [rg0, rg1)
  int* rg1 = rw + 5 * (F_MAXR + 1);
  if (p.groups)
    for (int i = tid; i <= p.groups; i += 256) offl[i] = min(max(p.offsets[i], 0), p.M);
  __syncthreads();
  if (tid == 0) {
    int trows = 0, nqall = 0;   // tile rows and quantize jobs over all groups
    for (int g = 0; g < ng; ++g) {
      const int o0 = p.groups ? offl[g] : 0, o1 = p.groups ? offl[g + 1] : p.M;
      trows += o1 > o0 ? (o1 - o0 + T::BM - 1) / T::BM : 0;
      nqall += o1 > o0 ? (o1 - o0 + FQ_ROWS - 1) / FQ_ROWS : 0;
    }
    const int total = trows * tn_count;
    // Chunks of equal work: a tile costs 1, a quantize job F_QCOST (x2 for
    // fp32 input); a chunk that starts inside a tile row quantizes that row
    // again.  Tiles are handed out in order until a chunk reaches its share.
    const float wq = F_QCOST * (p.x_bf16 ? 1.0f : 2.0f);
    // (each of the nl - 1 cuts is taken to re-quantize one tile row)
    const float share = ((float)total + wq * (float)(nqall + (p.nl - 1) * (T::BM / FQ_ROWS))) / (float)p.nl;
    int c0 = total, c1 = total;
    {
      int x = 0, t = 0;
      float acc = 0.0f;
      if (list == 0) c0 = 0;
      for (int g = 0; g < ng && x < p.nl - 1; ++g) {
        const int o0 = p.groups ? offl[g] : 0, o1 = p.groups ? offl[g + 1] : p.M;
        const int n = o1 > o0 ? (o1 - o0 + T::BM - 1) / T::BM : 0;
        for (int tm = 0; tm < n && x < p.nl - 1; ++tm) {
          const float qrow = wq * (float)((min(o1, o0 + (tm + 1) * T::BM) - (o0 + tm * T::BM) + FQ_ROWS - 1) / FQ_ROWS);
          acc += qrow;
          int left = tn_count;
          while (left > 0 && x < p.nl - 1) {
            const int k = max(0, (int)(share - acc + 0.5f));
            if (k >= left) { acc += (float)left; t += left; left = 0; break; }
            acc += (float)k; t += k; left -= k;
            if (x == list) c1 = t;          // chunk x ends, chunk x + 1 starts here
            ++x;
            if (x == list) c0 = t;
            acc = left > 0 ? qrow : 0.0f;   // the next chunk quantizes this row too
          }
        }
      }
      if (list == p.nl - 1 || x == list) c1 = total;
      if (c0 > c1) c0 = c1;
    }
    const int tc = c1 - c0;
    int F = tc, S = 1, LR = 0, R_lo = 0;
    if (tc > 0) {
      R_lo = c0 / tn_count;
      LR = (c1 - 1) / tn_count - R_lo + 1;
      // local tile rows: first row, end row and group of global tile rows R_lo..
      int R = 0;
      for (int g = 0; g < ng && R < R_lo + LR; ++g) {
        const int o0 = p.groups ? offl[g] : 0, o1 = p.groups ? offl[g + 1] : p.M;
        const int n = o1 > o0 ? (o1 - o0 + T::BM - 1) / T::BM : 0;
        for (int tm = 0; tm < n; ++tm, ++R)
          if (R >= R_lo && R < R_lo + LR) {
            rinfo[R - R_lo][0] = o0 + tm * T::BM;
            rinfo[R - R_lo][1] = min(o1, o0 + (tm + 1) * T::BM);
            rinfo[R - R_lo][2] = g;
          }
      }
      // whole tiles in rounds of wpl; the rest split along K (pairs of stages)
      const int rem = tc % p.wpl;
      if (rem) {
        S = min(min(p.wpl / rem, nst / 2), min(F_MAX_PARTS, F_MAX_SPLIT / rem));
        if (S >= 2) F = tc - rem; else S = 1;
      }
      int q = 0, tt = 0, g0 = 0;
      for (int l = 0; l < LR; ++l) {
        qpre[l] = q;
        tpre[l] = tt;
        q += (rinfo[l][1] - rinfo[l][0] + FQ_ROWS - 1) / FQ_ROWS;
        const int rb = (R_lo + l) * tn_count;
        const int lo = max(c0, rb) - rb, hi = min(c0 + F, rb + tn_count) - rb;
        tlo[l] = hi > lo ? lo : 0;
        thi[l] = hi > lo ? hi : 0;
        tt += thi[l] - tlo[l];
        if (l > g0 && (l - g0 == F_GR || rinfo[l][2] != rinfo[g0][2])) g0 = l;   // a new raster group
        rg0[l] = g0;
      }
      qpre[LR] = q;
      tpre[LR] = tt;
      for (int l = LR - 1, e = LR; l >= 0; --l) {
        rg1[l] = e;
        if (rg0[l] == l) e = l;
      }
    }
    sh[2] = c0;
    sh[3] = R_lo;
    sh[4] = F;
    sh[5] = S;
    sh[6] = LR;
    sh[7] = tc;
  }
  __syncthreads();
  {
    const int c0 = sh[2], R_lo = sh[3], F = sh[4], S = sh[5], LR = sh[6], tc = sh[7];
    const int NQ = LR ? qpre[LR] : 0;
    for (int k = tid; k < NQ; k += 256) {      // quantize jobs
      int l = 0;
      while (qpre[l + 1] <= k) ++l;
      jt[k] = fjob(FJ_Q, l, k - qpre[l]);
    }
    for (int idx = tid; idx < F; idx += 256) {   // whole tiles
      const int t = c0 + idx, l = t / tn_count - R_lo, tn = t % tn_count;
      int pos = NQ + tpre[rg0[l]];
      for (int m = rg0[l]; m < rg1[l]; ++m) {
        pos += max(0, min(tn, thi[m]) - tlo[m]);                       // earlier columns of the group
        if (m < l && tlo[m] <= tn && tn < thi[m]) ++pos;               // this column, rows above
      }
      jt[pos] = fjob(FJ_G, 0, idx);
    }
    for (int u = tid; u < (tc - F) * S; u += 256) jt[NQ + F + u] = fjob(FJ_P, 0, u);   // split parts
    if (tid == 0) sh[0] = NQ + F + (tc - F) * S;
  }
  __syncthreads();
  // values read back from LDS are uniform: keep them in scalar registers (the
  // buffer descriptors of the tile loads must be scalar)
  const int njobs = __builtin_amdgcn_readfirstlane(sh[0]), c0 = __builtin_amdgcn_readfirstlane(sh[2]);
  const int R_lo = __builtin_amdgcn_readfirstlane(sh[3]), F = __builtin_amdgcn_readfirstlane(sh[4]);
  const int S = __builtin_amdgcn_readfirstlane(sh[5]);

  for (;;) {
    // The previous job is done with LDS and sh[1].  Bare barriers (LDS
    // operations waited for, not memory ones): the previous tile's C stores
    // keep draining while the next job starts, as they would behind a
    // workgroup that ends.
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    block_barrier();
    if (tid == 0) sh[1] = (int)atomicAdd(&ctr[0], 1u);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    block_barrier();
    const int tk = __builtin_amdgcn_readfirstlane(sh[1]);
    if (tk >= njobs) break;
    const uint32_t job = __builtin_amdgcn_readfirstlane(jt[tk]);
    const int type = (int)(job >> 28), ja = (int)((job >> 14) & 0x3fff), jb = (int)(job & 0x3fff);

    if (type == FJ_Q) {
      const int r0 = __builtin_amdgcn_readfirstlane(rinfo[ja][0]) + jb * FQ_ROWS;
      const int r1 = min(__builtin_amdgcn_readfirstlane(rinfo[ja][1]), r0 + FQ_ROWS);
      if (p.x_bf16)
        fq_rows<uint16_t>(static_cast<const uint16_t*>(p.x), p.ldx, r0, r1, p.K, p.a_codes, p.a_scales);
      else
        fq_rows<float>(static_cast<const float*>(p.x), p.ldx, r0, r1, p.K, p.a_codes, p.a_scales);
      if (tid == 0) __hip_atomic_fetch_add(&ctr[F_READY0 + ja], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }

    // a tile (whole, or one K part of a split tile)
    const int ti = type == FJ_G ? jb : F + jb / S;
    const int t = c0 + ti;
    const int l = __builtin_amdgcn_readfirstlane(t / tn_count - R_lo);
    const int tn = __builtin_amdgcn_readfirstlane(t % tn_count);
    const int m0 = __builtin_amdgcn_readfirstlane(rinfo[l][0]), m_end = __builtin_amdgcn_readfirstlane(rinfo[l][1]);
    const int g = __builtin_amdgcn_readfirstlane(rinfo[l][2]);
    if (tid == 0) {
      const uint32_t need = (uint32_t)((m_end - m0 + FQ_ROWS - 1) / FQ_ROWS);
      // bounded: the producers hold smaller tickets and never wait, so this
      // ends long before the bound (about a second) unless something is broken
      for (int spin = 0; spin < (1 << 22); ++spin) {
        if (__hip_atomic_load(&ctr[F_READY0 + l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) break;
        __builtin_amdgcn_s_sleep(4);
      }
    }
    __syncthreads();
    const int n0 = tn * T::BN;
    const int a_rows = __builtin_amdgcn_readfirstlane(m_end - m0), b_rows = __builtin_amdgcn_readfirstlane(min(T::BN, p.N - n0));
    const MxTileSrc src = mx_tile_src(p.a_codes, p.a_scales, p.b_codes, p.b_scales, p.K, (size_t)m0, a_rows,
                                      (size_t)g * p.N + n0, b_rows);
    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // a split part covers stage pairs [part * np / S, (part + 1) * np / S)
    int tix = threadIdx.x;
    asm volatile("" : "+v"(tix));   // per-lane offsets formed per job, not held across the job loop
    const int part = jb % S, np = nst / 2;
    const int s0 = type == FJ_G ? 0 : 2 * (part * np / S), s1 = type == FJ_G ? nst : 2 * ((part + 1) * np / S);
    mx_tile_mainloop<true>(smem, src, s0, s1, acc);
    if (type == FJ_G) {
      mx_tile_store<true>(smem, p.c, p.ldc, p.c_bf16, p.N, m0, m_end, n0, acc);
      continue;
    }
    const int lane = tix & 63, wave = tix >> 6;
    f32x4* mine = reinterpret_cast<f32x4*>(p.part + (size_t)(list * F_MAX_SPLIT + jb) * F_PART_FLOATS);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          mine[(((wave * TI + i) * TJ + j) * 4 + q) * 64 + lane] =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    __syncthreads();   // every store of this part is complete
    if (tid == 0)
      sh[6] = (int)__hip_atomic_fetch_add(&ctr[F_SPLIT0 + jb / S], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(sh[6]) != S - 1) continue;
    // last part to arrive: C = the S partial tiles added in part order.  A
    // partial vector (i, j, q) of lane L holds rows i*32 + 8q + 4(L/32) + e
    // (e = 0..3) of column j*32 + L%32 of this wave's 128 x 128 quarter.
    const int wy = wave >> 1, wx = wave & 1, lrow = lane & 31, khalf = lane >> 5;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.part + (size_t)(list * F_MAX_SPLIT + (jb / S) * S) * F_PART_FLOATS), 0, S * F_PART_FLOATS * 4,
        0x00020000);
    const int col = n0 + wx * 128 + lrow;
#pragma unroll 1
    for (int i = 0; i < TI; ++i)
#pragma unroll 1
      for (int jh = 0; jh < TJ; jh += 1) {
        // the S (<= 4) partial vectors of 4 slots in flight at once, then
        // added in part order
        f32x4 v[F_MAX_PARTS][1][4];
        const int vo = ((((wave * TI + i) * TJ + jh) * 4) * 64 + lane) * 16;
#pragma unroll
        for (int pp = 0; pp < F_MAX_PARTS; ++pp)
          if (pp < S)
#pragma unroll
            for (int jj = 0; jj < 1; ++jj)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                v[pp][jj][q] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, vo + (jj * 4 + q) * 1024, pp * F_PART_FLOATS * 4, 0));
#pragma unroll
        for (int jj = 0; jj < 1; ++jj) {
          const int cj = col + (jh + jj) * 32;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 sum = v[0][jj][q];
#pragma unroll
            for (int pp = 1; pp < F_MAX_PARTS; ++pp)
              if (pp < S) sum += v[pp][jj][q];
            if (cj < p.N) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int row = m0 + wy * 128 + i * 32 + 8 * q + 4 * khalf + e;
                if (row < m_end) {
                  if (p.c_bf16)
                    reinterpret_cast<uint16_t*>(p.c)[(size_t)row * p.ldc + cj] = (uint16_t)f32_to_bf16_rne(sum[e]);
                  else
                    reinterpret_cast<float*>(p.c)[(size_t)row * p.ldc + cj] = sum[e];
                }
              }
            }
          }
        }
      }
  }
}

int fused_lists() { return 8; }

bool fused_fits(int64_t M, int64_t N, int64_t K, int groups, int wpl) {
  if (K % (2 * BK2) != 0 || K < 2 * BK2 || K > (int64_t(1) << 22)) return false;
  if ((int64_t)(groups + 1) * 4 > F_OFFL_BYTES) return false;   // offsets are staged in LDS
  (void)wpl;
  // bounds of one chunk: its tiles stay below the work share plus one
  const int64_t tn = (N + 255) / 256;
  const int64_t tiles = ((M + 255) / 256 + (groups > 0 ? groups : 0)) * tn;
  const int64_t qjobs = M / FQ_ROWS + (groups > 0 ? groups : 1);
  const int64_t per = (int64_t)((tiles + 2.0 * F_QCOST * qjobs) / fused_lists()) + 2;
  const int64_t lr = per / tn + 2;
  return lr <= F_MAXR && per + lr * (256 / FQ_ROWS) + F_MAX_SPLIT <= F_JMAX && per < (1 << 14);
}

size_t fused_workspace_bytes() {
  return (size_t)fused_lists() * F_CTR_STRIDE * 4 + (size_t)fused_lists() * F_MAX_SPLIT * F_PART_FLOATS * 4;
}

hipError_t launch_gemm_mx_fused(const void* x, int x_bf16, int64_t ldx, uint8_t* a_codes, uint8_t* a_scales,
                                const uint8_t* b_codes, const uint8_t* b_scales, void* c, int c_bf16, int64_t ldc,
                                int64_t M, int64_t N, int64_t K, int groups, const int32_t* offsets, void* ws,
                                int wpl, hipStream_t st) {
  FusedParams p;
  p.x = x; p.ldx = ldx; p.x_bf16 = x_bf16;
  p.a_codes = a_codes; p.a_scales = a_scales; p.b_codes = b_codes; p.b_scales = b_scales;
  p.c = c; p.ldc = ldc; p.c_bf16 = c_bf16;
  p.M = (int)M; p.N = (int)N; p.K = (int)K; p.groups = groups; p.offsets = offsets;
  p.nl = fused_lists();
  p.wpl = wpl;
  p.ctr = static_cast<uint32_t*>(ws);
  p.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + (size_t)p.nl * F_CTR_STRIDE * 4);
  hipLaunchKernelGGL(k_fused_reset, dim3(1), dim3(256), 0, st, p.ctr, p.nl * F_CTR_STRIDE);
  hipLaunchKernelGGL(k_gemm_mx_fused, dim3((unsigned)(p.nl * wpl)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace mxk
