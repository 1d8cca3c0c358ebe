// Block-scaled FP4 quantization and dequantization kernels for gfx950.
//
// MXFP4: "NVFP4 Architecture: Microscaling & 4-Bit LLMs on Blackwell",
// section "1. The Dual-Level Mathematical Formulation" (equations S_block and
// q_i, S_global = 1) with 32-element blocks ("How Microscaling FP4 (MXFP4)
// Halves Memory Bandwidth", section "The Microscaling Breakthrough").
// NVFP4: the same equations with 16-element blocks, an FP8 E4M3 block scale
// and an fp32 per-tensor scale ("NVIDIA NVFP4 quantization", section "The
// Physics of NVFP4").
//
// Streaming design: every lane owns one 16-byte input vector (4 fp32 or 8 bf16
// elements); a wave covers 64 consecutive vectors, so each load instruction is
// one contiguous 1 KiB request.  A block spans 2..8 lanes; its max |x| is an
// integer max over the abs bit patterns reduced with xor shuffles.  Each lane
// then writes its own packed codes (2 or 4 bytes), one lane per block the
// scale byte.  Several vectors per lane are loaded before any is used so that
// enough bytes are in flight to cover HBM latency.
#include <type_traits>

#include "mx_device.h"
#include "nv_codes.h"
#include "mx_kernels.h"

namespace mxk {

constexpr int QT = 256;    // threads per workgroup
constexpr int QU = 4;      // vectors per lane per iteration (loads in flight)

// ---------------------------------------------------------------------------
// MXFP4 quantize
// ---------------------------------------------------------------------------
// Vector v of the tensor: flat index v in [0, rows * cols / EPL).  With a
// contiguous tensor (ld == cols) its elements sit at x + v * EPL; otherwise
// row = v / vpr.
// max over the LPB lanes of a block (aligned groups of 2, 4 or 8 lanes) with
// DPP lane swaps inside each row of 16 lanes: no LDS round trip
template <int LPB>
__device__ __forceinline__ uint32_t block_umax(uint32_t v) {
  if constexpr (LPB >= 2) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));   // lane ^ 1
  if constexpr (LPB >= 4) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));   // lane ^ 2
  if constexpr (LPB >= 8) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // 8-lane mirror
  return v;
}

// MODE 0: contiguous rows; 1: rows ld apart; 2: output row r is input row
// gidx[r] (an index outside [0, x_rows) gives a zero row).  FLOOR: the OCP
// exponent rule e = floor(log2 max|x|) - 2 (= F - 129), elements beyond 6
// saturating (the conversion saturates), same floor of -29.
template <typename TIn, int MODE, bool FLOOR = false>
__global__ __launch_bounds__(QT) void k_quant_mx(const TIn* __restrict__ x, int64_t ldx, uint32_t vpr,
                                                 uint32_t nvec, uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales, const int32_t* __restrict__ gidx,
                                                 int64_t x_rows) {
  constexpr int EPL = 16 / (int)sizeof(TIn);  // elements per vector
  constexpr int LPB = 32 / EPL;               // lanes per 32-element block
  const int lane = threadIdx.x & 63;
  const uint32_t wave_global = (blockIdx.x * QT + threadIdx.x) >> 6;
  const uint32_t nwaves = (gridDim.x * QT) >> 6;
  const uint32_t stride = nwaves * (64 * QU);
  auto load = [&](u32x4 (&d)[QU], uint32_t base) {
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      uint32_t v = base + u * 64 + lane;
      const TIn* p;
      bool ok = v < nvec;
      if (MODE == 0) {
        p = x + (size_t)v * EPL;
      } else {
        uint32_t r = v / vpr, c = v - r * vpr;
        int64_t src = r;
        if (MODE == 2) {
          src = ok ? (int64_t)gidx[r] : 0;
          ok = ok && src >= 0 && src < x_rows;
        }
        p = x + (size_t)(ok ? src : 0) * ldx + (size_t)c * EPL;
      }
      // streaming input: non-temporal loads keep it from displacing the
      // quantized outputs (which the consumer reads next) from the caches
      d[u] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)) : u32x4{0, 0, 0, 0};
    }
  };
  // the next iteration's vectors are in flight while this one is converted
  u32x4 d[QU], dn[QU];
  uint32_t base = wave_global * (64 * QU);
  if (base < nvec) load(d, base);
  for (; base < nvec; base += stride) {
    const uint32_t nb = base + stride;
    if (nb < nvec) load(dn, nb);
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const uint32_t v = base + u * 64 + lane;
      float f[EPL];
      if constexpr (EPL == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = ffrom(d[u][i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] = bf16_lo(d[u][i]);
          f[2 * i + 1] = bf16_hi(d[u][i]);
        }
      }
      uint32_t am = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) am = max(am, fbits(f[i]) & 0x7fffffffu);
      am = block_umax<LPB>(am);
      const int e = FLOOR ? max((int)(am >> 23) - 129, -29) : mx_block_exp(am);
      const float s = pow2f(e);
      uint32_t out = 0;
      out = cvt_fp4x2<0>(out, f[0], f[1], s);
      out = cvt_fp4x2<1>(out, f[2], f[3], s);
      if constexpr (EPL == 8) {
        out = cvt_fp4x2<2>(out, f[4], f[5], s);
        out = cvt_fp4x2<3>(out, f[6], f[7], s);
      }
      if (v < nvec) {
        if constexpr (EPL == 4) {
          reinterpret_cast<uint16_t*>(codes)[v] = (uint16_t)out;
        } else {
          reinterpret_cast<uint32_t*>(codes)[v] = out;
        }
        if ((lane & (LPB - 1)) == 0) scales[v / LPB] = (uint8_t)(e + 127);
      }
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) d[u] = dn[u];
  }
}

// ---------------------------------------------------------------------------
// NVFP4: tensor max |x| (partials per workgroup), then quantize
// ---------------------------------------------------------------------------
// A lane keeps AU 16-byte vectors in flight: each step of the grid-stride
// loop issues all of its loads (every one a contiguous 1 KiB per wave) before
// it reduces any of them.
constexpr int AU = 8;
template <typename TIn, bool CONTIG>
__global__ __launch_bounds__(QT) void k_absmax(const TIn* __restrict__ x, int64_t ldx, uint32_t vpr, uint32_t nvec,
                                               uint32_t* __restrict__ partial) {
  constexpr int EPL = 16 / (int)sizeof(TIn);
  __shared__ uint32_t red[QT / 64];
  uint32_t am = 0;
  for (uint32_t base = blockIdx.x * (QT * AU); base < nvec; base += gridDim.x * (QT * AU)) {
    u32x4 d[AU];
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const uint32_t v = base + u * QT + threadIdx.x;
      const TIn* p;
      if (CONTIG) {
        p = x + (size_t)v * EPL;
      } else {
        const uint32_t r = v / vpr, c = v - r * vpr;
        p = x + (size_t)r * ldx + (size_t)c * EPL;
      }
      d[u] = v < nvec ? *reinterpret_cast<const u32x4*>(p) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      if constexpr (EPL == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) am = max(am, d[u][i] & 0x7fffffffu);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) am = max(am, max(d[u][i] & 0x7fffu, (d[u][i] >> 16) & 0x7fffu) << 16);
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) am = umax_xor(am, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int i = 1; i < QT / 64; ++i) r = max(r, red[i]);
    partial[blockIdx.x] = r;
  }
}

// Per-tensor scale from the partial maxima: g = fp32(amax / 2688), 2688 being
// 6 (largest E2M1 state) x 448 (largest E4M3 value), or 1 for an all-zero
// tensor; the fp32 division is IEEE correctly rounded.  The partials (a
// multiple of 4, at most 4096) are loaded as 16-byte vectors by
// nv_partials_load before the caller issues its data loads, so that using
// them waits only for these (vector loads complete in order); the reduction
// ends with a bare barrier, which leaves the data loads in flight.
constexpr int NV_PV = 4;   // 16-byte partial vectors per thread: 4 x 4 x 256 = 4096
__device__ __forceinline__ void nv_partials_load(const uint32_t* __restrict__ partial, int npart, u32x4 (&pv)[NV_PV]) {
#pragma unroll
  for (int k = 0; k < NV_PV; ++k) {
    const int idx = (k * QT + (int)threadIdx.x) * 4;
    pv[k] = idx < npart ? *reinterpret_cast<const u32x4*>(partial + idx) : u32x4{0, 0, 0, 0};
  }
}
__device__ __forceinline__ float nv_global_from_partials(const u32x4 (&pv)[NV_PV], uint32_t* red) {
  uint32_t am = 0;
#pragma unroll
  for (int k = 0; k < NV_PV; ++k) am = max(max(am, max(pv[k][0], pv[k][1])), max(pv[k][2], pv[k][3]));
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) am = umax_xor(am, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS write is done
  block_barrier();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < QT / 64; ++i) r = max(r, red[i]);
  return r == 0 ? 1.0f : ffrom(r) / 2688.0f;
}

// One lane per 16-element block: the block's scale and its seven decision
// boundaries (fp64 work) are computed once per block rather than once per
// 16-byte vector.  A wave takes 64 consecutive blocks per step.  Its loads
// are coalesced (load q of lane l is vector 64 q + l of the wave's range, so
// each load instruction reads 1 KiB of contiguous memory), and the vectors
// reach their block's lane through a 4 KiB (fp32; 2 KiB bf16) LDS area of the
// wave: piece p of block b sits in 16-byte slot VPB b + (p ^ f(b)), f(b) =
// (b / (16 / VPB)) mod VPB, which keeps both the writes and the block-wise
// reads free of bank conflicts; a wave's LDS operations complete in order,
// so no barrier is needed.  The grid is sized so that every wave walks the
// same number of steps (launch_quant_nv), and each step first issues the
// loads of the wave's next step.  The first step's loads go out before the
// per-tensor scale is reduced from the partial maxima (they do not depend
// on it).
template <typename TIn, bool CONTIG>
__global__ __launch_bounds__(QT) void k_quant_nv(const TIn* __restrict__ x, int64_t ldx, uint32_t bpr,
                                                 uint32_t nblk, uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales, float* __restrict__ gout,
                                                 const uint32_t* __restrict__ partial, int npart) {
  constexpr int EPL = 16 / (int)sizeof(TIn);   // elements per 16-byte vector
  constexpr int VPB = 16 / EPL;                // vectors per block (4 or 2)
  __shared__ uint32_t red[QT / 64];
  __shared__ u32x4 stage[QT / 64][64 * VPB];
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4* ws = stage[wave];
  const uint32_t nvec = nblk * VPB, vpr = bpr * VPB;
  const uint32_t step = gridDim.x * QT;        // blocks per step of the grid
  // loads of the wave's 64 blocks from block wb on; vectors past the end read
  // the last vector again (their blocks are not stored)
  auto load = [&](u32x4 (&d)[VPB], uint32_t wb) {
#pragma unroll
    for (int q = 0; q < VPB; ++q) {
      const uint32_t v = min(wb * VPB + q * 64 + lane, nvec - 1);
      const TIn* p;
      if (CONTIG) {
        p = x + (size_t)v * EPL;
      } else {
        const uint32_t r = v / vpr, c = v - r * vpr;
        p = x + (size_t)r * ldx + (size_t)c * EPL;
      }
      d[q] = *reinterpret_cast<const u32x4*>(p);
    }
  };
  auto slot = [](uint32_t b, uint32_t piece) { return VPB * b + (piece ^ ((b / (16 / VPB)) % VPB)); };
  // ALL: every block of the step exists, so the stores are not tested
  auto code_step = [&](const u32x4 (&d)[VPB], uint32_t wb, double g, auto all) {
#pragma unroll
    for (int q = 0; q < VPB; ++q) {
      const uint32_t lv = q * 64 + lane;       // the vector's place in the step
      ws[slot(lv / VPB, lv % VPB)] = d[q];
    }
    u32x4 e[VPB];
#pragma unroll
    for (int q = 0; q < VPB; ++q) e[q] = ws[slot(lane, q)];
    const uint32_t b = wb + lane;
    uint32_t xb[16];
#pragma unroll
    for (int q = 0; q < VPB; ++q) {
      if constexpr (EPL == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xb[q * 4 + i] = e[q][i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xb[q * 8 + 2 * i] = e[q][i] << 16;
          xb[q * 8 + 2 * i + 1] = e[q][i] & 0xffff0000u;
        }
      }
    }
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = max(am, xb[i] & 0x7fffffffu);
    // s_b = E4M3 nearest to amax / (6 g); unit y = s_b * g is exact in fp64.
    const uint32_t sc = e4m3_rne_sat((double)ffrom(am) / (6.0 * g));
    const double y = (double)e4m3_to_f32(sc) * g;
    const NvFast nf = nv_fast_setup(y, am);
    uint32_t lo, hi;
    const bool fast_lo = nv_fast_codes8(xb, nf, lo), fast_hi = nv_fast_codes8(xb + 8, nf, hi);
    if (!(nf.ok && fast_lo && fast_hi)) {   // an element within 2^-20 of a boundary: exact test
      uint32_t U[7];
      nv_boundaries(y, U);
      lo = hi = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo |= nv_code_sel(xb[i], U) << (4 * i);
        hi |= nv_code_sel(xb[8 + i], U) << (4 * i);
      }
    }
    if (decltype(all)::value || b < nblk) {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      *reinterpret_cast<u32x2_t*>(codes + (size_t)b * 8) = u32x2_t{lo, hi};
      scales[b] = (uint8_t)sc;
    }
  };
  const std::true_type all;
  const std::false_type some;
  u32x4 d[VPB], dn[VPB];
  u32x4 pv[NV_PV];
  if (partial) nv_partials_load(partial, npart, pv);
  uint32_t wb = blockIdx.x * QT + wave * 64;   // first block of the wave's step
  load(d, wb);
  float g;
  if (partial) {
    g = nv_global_from_partials(pv, red);
    if (blockIdx.x == 0 && threadIdx.x == 0) *gout = g;
  } else {
    g = *gout;  // static per-tensor scale supplied by the caller
  }
  // while this and the next step are whole, then the last steps with tested
  // stores; the trip counts are uniform over a wave
  for (; (uint64_t)wb + step + 63 < nblk; wb += step) {
    load(dn, wb + step);
    code_step(d, wb, (double)g, all);
#pragma unroll
    for (int q = 0; q < VPB; ++q) d[q] = dn[q];
  }
  for (; wb < nblk; wb += step) {
    load(dn, wb + step);
    code_step(d, wb, (double)g, some);
#pragma unroll
    for (int q = 0; q < VPB; ++q) d[q] = dn[q];
  }
}

// ---------------------------------------------------------------------------
// Dequantize: each lane expands one 32-bit word of codes (8 elements).
// ---------------------------------------------------------------------------
template <bool NV, bool OUT_BF16, bool CONTIG>
__global__ __launch_bounds__(QT) void k_dequant(const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                const float* __restrict__ gptr, uint32_t wpr, uint32_t nwords,
                                                void* __restrict__ y, int64_t ldy) {
  const float g = NV ? *gptr : 1.0f;
  for (uint32_t w = blockIdx.x * QT + threadIdx.x; w < nwords; w += gridDim.x * QT) {
    const uint32_t c = codes[w];
    float f[8];
    if (!NV) {
      // 8 codes of one 32-element block; E8M0 byte -> power of two.
      const float s = pow2f((int)scales[w >> 2] - 127);
      f32x2 t;
      t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, s, 0); f[0] = t.x; f[1] = t.y;
      t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, s, 1); f[2] = t.x; f[3] = t.y;
      t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, s, 2); f[4] = t.x; f[5] = t.y;
      t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, s, 3); f[6] = t.x; f[7] = t.y;
    } else {
      // 8 codes of one 16-element block; fp32(fp32(q * s) * g).
      const float s = e4m3_to_f32(scales[w >> 1]);
      f32x2 t;
      t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0); f[0] = t.x; f[1] = t.y;
      t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1); f[2] = t.x; f[3] = t.y;
      t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2); f[4] = t.x; f[5] = t.y;
      t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3); f[6] = t.x; f[7] = t.y;
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (f[i] * s) * g;
    }
    size_t off;  // element offset of the first of the 8 outputs
    if (CONTIG) {
      off = (size_t)w * 8;
    } else {
      uint32_t r = w / wpr, cw = w - r * wpr;
      off = (size_t)r * ldy + (size_t)cw * 8;
    }
    if (OUT_BF16) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2_rne(f[2 * i], f[2 * i + 1]);
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(y) + off) = o;
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(y) + off);
      dst[0] = f32x4{f[0], f[1], f[2], f[3]};
      dst[1] = f32x4{f[4], f[5], f[6], f[7]};
    }
  }
}

// ---------------------------------------------------------------------------
// Wider MX elements: MXFP8 (E4M3, E5M2) and MXFP6 (E2M3, E3M2), same 32-element
// blocks and E8M0 scales.  The block exponent is the smallest e with
// max|x| <= Emax * 2^e (max|x| raised to 1e-8 first); for Emax = (1 + fE) 2^p
// and max|x| = (1 + f) 2^(F-127) that is F - 127 - p + [f > fE], floored at
// -27 - p (fp32(1e-8) has biased exponent 100 and a mantissa below every
// fE).  Elements: |x| * 2^-e (exact in fp32) rounded to nearest-even in
// software -- below the smallest normal 2^(1-bias) the subnormal step count
// rint(v * 2^(bias-1+M)), else the fp32 mantissa rounded to M bits with the
// carry running into the exponent field.  The scale rule keeps v <= Emax, so
// nothing saturates and no NaN code (E4M3 0x7F) or infinity (E5M2) arises.
// ---------------------------------------------------------------------------
template <int F>
struct WideFmt;
template <> struct WideFmt<0> { static constexpr int E = 4, M = 3, BIAS = 7, P = 8; static constexpr uint32_t FE = 0x600000u; };
template <> struct WideFmt<1> { static constexpr int E = 5, M = 2, BIAS = 15, P = 15; static constexpr uint32_t FE = 0x600000u; };
template <> struct WideFmt<2> { static constexpr int E = 2, M = 3, BIAS = 1, P = 2; static constexpr uint32_t FE = 0x700000u; };
template <> struct WideFmt<3> { static constexpr int E = 3, M = 2, BIAS = 3, P = 4; static constexpr uint32_t FE = 0x600000u; };

template <int F, bool FLOOR = false>
__device__ __forceinline__ int wide_block_exp(uint32_t amax_bits) {
  using T = WideFmt<F>;
  // FLOOR: the OCP rule floor(log2 max|x|) - P
  const int e = (int)(amax_bits >> 23) - 127 - T::P + ((!FLOOR && (amax_bits & 0x7fffffu) > T::FE) ? 1 : 0);
  return e < -27 - T::P ? -27 - T::P : e;
}
template <int F>
__device__ __forceinline__ float wide_emax() {
  return F == 0 ? 448.0f : (F == 1 ? 57344.0f : (F == 2 ? 7.5f : 28.0f));
}

// Code of x (sign from x's bit pattern) for the block scale factor inv = 2^-e.
template <int F>
__device__ __forceinline__ uint32_t wide_encode(uint32_t xbits, float inv) {
  using T = WideFmt<F>;
  constexpr int BITS = 1 + T::E + T::M;
  // saturation (only reachable under the floor rule): rounding a value in
  // (Emax, Emax + half a step) and then saturating gives Emax too
  const float v = fminf(ffrom(xbits & 0x7fffffffu) * inv, wide_emax<F>());
  const uint32_t u = fbits(v);
  const uint32_t sub = (uint32_t)__builtin_rintf(v * pow2f(T::BIAS - 1 + T::M));
  uint32_t t = u >> (23 - T::M);
  const uint32_t rem = u & ((1u << (23 - T::M)) - 1u), half = 1u << (22 - T::M);
  t += (rem > half || (rem == half && (t & 1u))) ? 1u : 0u;
  const uint32_t nrm = t - ((uint32_t)(127 - T::BIAS) << T::M);
  const uint32_t mag = u < ((uint32_t)(128 - T::BIAS) << 23) ? sub : nrm;
  return mag | ((xbits >> 31) << (BITS - 1));
}

template <typename TIn, int F, bool CONTIG, bool FLOOR = false>
__global__ __launch_bounds__(QT) void k_quant_wide(const TIn* __restrict__ x, int64_t ldx, uint32_t vpr, uint32_t nvec,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int EPL = 16 / (int)sizeof(TIn);
  constexpr int LPB = 32 / EPL;
  constexpr int BITS = 1 + WideFmt<F>::E + WideFmt<F>::M;
  const int lane = threadIdx.x & 63;
  const uint32_t wave_global = (blockIdx.x * QT + threadIdx.x) >> 6;
  const uint32_t nwaves = (gridDim.x * QT) >> 6;
  const uint32_t stride = nwaves * (64 * QU);
  auto load = [&](u32x4 (&d)[QU], uint32_t base) {
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const uint32_t v = base + u * 64 + lane;
      const TIn* p;
      if (CONTIG) {
        p = x + (size_t)v * EPL;
      } else {
        const uint32_t r = v / vpr, c = v - r * vpr;
        p = x + (size_t)r * ldx + (size_t)c * EPL;
      }
      d[u] = v < nvec ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)) : u32x4{0, 0, 0, 0};
    }
  };
  u32x4 d[QU], dn[QU];
  uint32_t base = wave_global * (64 * QU);
  if (base < nvec) load(d, base);
  for (; base < nvec; base += stride) {
    const uint32_t nb = base + stride;
    if (nb < nvec) load(dn, nb);
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const uint32_t v = base + u * 64 + lane;
      uint32_t xb[EPL];
      if constexpr (EPL == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xb[i] = d[u][i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xb[2 * i] = d[u][i] << 16;
          xb[2 * i + 1] = d[u][i] & 0xffff0000u;
        }
      }
      uint32_t am = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) am = max(am, xb[i] & 0x7fffffffu);
      am = block_umax<LPB>(am);
      const int e = wide_block_exp<F, FLOOR>(am);
      const float inv = pow2f(-e);
      uint32_t c[EPL];
      uint32_t hw[EPL / 4];                       // FP8 codes from the hardware conversion
      if constexpr (BITS == 8 && !FLOOR) {
        // The scaled conversion divides by 2^e and rounds to nearest even
        // (subnormal codes included); under this exponent rule no element
        // exceeds the format's largest value, so its overflow handling never
        // applies.  The floor rule saturates and keeps the software encoder.
        const float sc = pow2f(e);
        typedef short s16x2 __attribute__((ext_vector_type(2)));
        // (bf16 inputs go through their exact fp32 values: the bf16-source
        // form of the conversion came out of the compiler with its second
        // and later sources replaced by the first)
#pragma unroll
        for (int h = 0; h < EPL / 4; ++h) {
          s16x2 r = {0, 0};
          const float x0 = ffrom(xb[4 * h]), x1 = ffrom(xb[4 * h + 1]);
          const float x2 = ffrom(xb[4 * h + 2]), x3 = ffrom(xb[4 * h + 3]);
          if constexpr (F == 0) {
            r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, x0, x1, sc, false);
            r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, x2, x3, sc, true);
          } else {
            r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, x0, x1, sc, false);
            r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, x2, x3, sc, true);
          }
          hw[h] = __builtin_bit_cast(uint32_t, r);
        }
      } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) c[i] = wide_encode<F>(xb[i], inv);
      }
      if (v < nvec) {
        if constexpr (BITS == 8 && !FLOOR) {
          if constexpr (EPL == 4) {
            reinterpret_cast<uint32_t*>(codes)[v] = hw[0];
          } else {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            reinterpret_cast<u32x2*>(codes)[v] = u32x2{hw[0], hw[1]};
          }
        } else if constexpr (BITS == 8) {
          uint32_t w0 = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
          if constexpr (EPL == 4) {
            reinterpret_cast<uint32_t*>(codes)[v] = w0;
          } else {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const uint32_t w1 = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
            reinterpret_cast<u32x2*>(codes)[v] = u32x2{w0, w1};
          }
        } else {
          // 6-bit fields, element i at bits [6i, 6i + 6) of the lane's bytes
          const uint32_t lo = c[0] | (c[1] << 6) | (c[2] << 12) | (c[3] << 18);   // 24 bits
          if constexpr (EPL == 4) {
            uint8_t* dst = codes + (size_t)v * 3;       // 3 bytes; 2-byte aligned when v is even
            if ((v & 1u) == 0) {
              *reinterpret_cast<uint16_t*>(dst) = (uint16_t)lo;
              dst[2] = (uint8_t)(lo >> 16);
            } else {
              dst[0] = (uint8_t)lo;
              *reinterpret_cast<uint16_t*>(dst + 1) = (uint16_t)(lo >> 8);
            }
          } else {
            const uint32_t hi = c[4] | (c[5] << 6) | (c[6] << 12) | (c[7] << 18);
            const uint32_t w0 = lo | (hi << 24), w1 = hi >> 8;                     // 48 bits
            uint8_t* dst = codes + (size_t)v * 6;       // 6 bytes; 4-byte aligned when v is even
            if ((v & 1u) == 0) {
              *reinterpret_cast<uint32_t*>(dst) = w0;
              *reinterpret_cast<uint16_t*>(dst + 4) = (uint16_t)w1;
            } else {
              *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w0;
              *reinterpret_cast<uint32_t*>(dst + 2) = (w0 >> 16) | (w1 << 16);
            }
          }
        }
        if ((lane & (LPB - 1)) == 0) scales[v / LPB] = (uint8_t)(e + 127);
      }
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) d[u] = dn[u];
  }
}

// MXFP6 (E2M3 / E3M2) under the pages' exponent rule: the hardware converts
// a whole 32-element block at once (v_cvt_scalef32_2xpk16_fp6_f32 / _bf6_f32:
// divide by 2^e, round to nearest even), so a lane owns a block.  The
// instruction interleaves its two 16-value sources (6-bit field 2i from the
// first source's value i, field 2i + 1 from the second's; probed), so the
// block's even elements go in the first and its odd elements in the second,
// which gives element j at bits 6j .. 6j + 5.  The walk and the coalesced
// loads are those of k_quant_nv: a wave takes 64 consecutive blocks per step,
// load q of lane l is vector 64 q + l of that range, and the vectors reach
// their block's lane through an LDS area of the wave (piece p of block b in
// slot VPB b + (p ^ f(b)), f(b) = (b / (16 / VPB)) mod VPB).  bf16 inputs are
// converted from their exact fp32 values.
template <typename TIn, int F, bool CONTIG>
__global__ __launch_bounds__(QT) void k_quant_fp6(const TIn* __restrict__ x, int64_t ldx, uint32_t bpr, uint32_t nblk,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  static_assert(F == 2 || F == 3, "FP6 element formats");
  constexpr int EPL = 16 / (int)sizeof(TIn);   // elements per 16-byte vector
  constexpr int VPB = 32 / EPL;                // vectors per block (8 or 4)
  __shared__ u32x4 stage[QT / 64][64 * VPB];
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4* ws = stage[wave];
  const uint32_t nvec = nblk * VPB, vpr = bpr * VPB;
  const uint32_t step = gridDim.x * QT;        // blocks per step of the grid
  auto load = [&](u32x4 (&d)[VPB], uint32_t wb) {
#pragma unroll
    for (int q = 0; q < VPB; ++q) {
      const uint32_t v = min(wb * VPB + q * 64 + lane, nvec - 1);   // past the end: the last vector again
      const TIn* p;
      if (CONTIG) {
        p = x + (size_t)v * EPL;
      } else {
        const uint32_t r = v / vpr, c = v - r * vpr;
        p = x + (size_t)r * ldx + (size_t)c * EPL;
      }
      d[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    }
  };
  auto slot = [](uint32_t b, uint32_t piece) { return VPB * b + (piece ^ ((b / (16 / VPB)) % VPB)); };
  auto code_step = [&](const u32x4 (&d)[VPB], uint32_t wb, auto all) {
#pragma unroll
    for (int q = 0; q < VPB; ++q) {
      const uint32_t lv = q * 64 + lane;
      ws[slot(lv / VPB, lv % VPB)] = d[q];
    }
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    f32x16 ev, od;                             // even and odd elements of the block
    uint32_t am = 0;
#pragma unroll
    for (int q = 0; q < VPB; ++q) {
      const u32x4 t = ws[slot(lane, q)];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (EPL == 4) {
          const int k = q * 4 + i;
          am = max(am, t[i] & 0x7fffffffu);
          if (k % 2 == 0) ev[k / 2] = ffrom(t[i]); else od[k / 2] = ffrom(t[i]);
        } else {
          const int k = q * 8 + 2 * i;         // elements k (low half) and k + 1
          const uint32_t a = t[i] << 16, b = t[i] & 0xffff0000u;
          am = max(am, max(a & 0x7fffffffu, b & 0x7fffffffu));
          ev[k / 2] = ffrom(a);
          od[k / 2] = ffrom(b);
        }
      }
    }
    const int e = wide_block_exp<F, false>(am);
    const float sc = pow2f(e);
    typedef uint32_t u32x6_t __attribute__((ext_vector_type(6)));
    u32x6_t r;
    if constexpr (F == 2) r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, sc);
    else r = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(ev, od, sc);
    const uint32_t b = wb + lane;
    if (decltype(all)::value || b < nblk) {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      u32x2_t* dst = reinterpret_cast<u32x2_t*>(codes + (size_t)b * 24);
      dst[0] = u32x2_t{r[0], r[1]};
      dst[1] = u32x2_t{r[2], r[3]};
      dst[2] = u32x2_t{r[4], r[5]};
      scales[b] = (uint8_t)(e + 127);
    }
  };
  const std::true_type all;
  const std::false_type some;
  u32x4 d[VPB], dn[VPB];
  uint32_t wb = blockIdx.x * QT + wave * 64;   // first block of the wave's step
  load(d, wb);
  for (; (uint64_t)wb + step + 63 < nblk; wb += step) {
    load(dn, wb + step);
    code_step(d, wb, all);
#pragma unroll
    for (int q = 0; q < VPB; ++q) d[q] = dn[q];
  }
  for (; wb < nblk; wb += step) {
    load(dn, wb + step);
    code_step(d, wb, some);
#pragma unroll
    for (int q = 0; q < VPB; ++q) d[q] = dn[q];
  }
}

// value(code) * 2^(E-127): each lane expands 16 elements (half a block).
template <int F>
__device__ __forceinline__ float wide_decode(uint32_t code) {
  using T = WideFmt<F>;
  constexpr int BITS = 1 + T::E + T::M;
  const uint32_t mag = code & ((1u << (BITS - 1)) - 1u);
  const uint32_t e = mag >> T::M, m = mag & ((1u << T::M) - 1u);
  const float sub = (float)m * pow2f(1 - T::BIAS - T::M);
  const float nrm = ffrom(((e + 127u - T::BIAS) << 23) | (m << (23 - T::M)));
  const float v = e == 0 ? sub : nrm;
  return (code >> (BITS - 1)) ? -v : v;
}

template <int F, bool OUT_BF16, bool CONTIG>
__global__ __launch_bounds__(QT) void k_dequant_wide(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                     uint32_t hpr, uint32_t nhalf, void* __restrict__ y, int64_t ldy) {
  constexpr int BITS = 1 + WideFmt<F>::E + WideFmt<F>::M;
  for (uint32_t h = blockIdx.x * QT + threadIdx.x; h < nhalf; h += gridDim.x * QT) {
    uint32_t c[16];
    if constexpr (BITS == 8) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(codes + (size_t)h * 16);
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = (w[i >> 2] >> (8 * (i & 3))) & 0xffu;
    } else {
      // 12 bytes = 96 bits: field i at bits [6i, 6i + 6)
      const uint32_t* src = reinterpret_cast<const uint32_t*>(codes + (size_t)h * 12);
      const uint64_t lo = (uint64_t)src[0] | ((uint64_t)src[1] << 32);
      const uint32_t w2 = src[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int b = 6 * i;
        if (b + 6 <= 64) c[i] = (uint32_t)(lo >> b) & 63u;
        else if (b >= 64) c[i] = (w2 >> (b - 64)) & 63u;
        else c[i] = ((uint32_t)(lo >> b) | (w2 << (64 - b))) & 63u;
      }
    }
    const int sexp = (int)scales[h >> 1] - 127;
    float f[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i] = __builtin_ldexpf(wide_decode<F>(c[i]), sexp);
    size_t off;
    if (CONTIG) {
      off = (size_t)h * 16;
    } else {
      const uint32_t r = h / hpr, ch = h - r * hpr;
      off = (size_t)r * ldy + (size_t)ch * 16;
    }
    if (OUT_BF16) {
      u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(y) + off);
#pragma unroll
      for (int q = 0; q < 2; ++q)
        dst[q] = u32x4{pack_bf16x2_rne(f[8 * q + 0], f[8 * q + 1]), pack_bf16x2_rne(f[8 * q + 2], f[8 * q + 3]),
                       pack_bf16x2_rne(f[8 * q + 4], f[8 * q + 5]), pack_bf16x2_rne(f[8 * q + 6], f[8 * q + 7])};
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(y) + off);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = f32x4{f[4 * q], f[4 * q + 1], f[4 * q + 2], f[4 * q + 3]};
    }
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static int grid_for(uint64_t work_items, int per_block) {
  uint64_t g = (work_items + per_block - 1) / per_block;
  const uint64_t cap = 256 * 16;  // 16 workgroups per CU is plenty for a grid-stride loop
  if (g > cap) g = cap;
  return (int)(g ? g : 1);
}

hipError_t launch_quant_mx(const void* x, int xdt_bf16, int64_t ldx, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, hipStream_t st, const int32_t* gidx, int64_t x_rows, bool floor_rule) {
  const int epl = xdt_bf16 ? 8 : 4;
  const uint32_t vpr = (uint32_t)(cols / epl);
  const uint32_t nvec = (uint32_t)(rows * cols / epl);
  const int mode = gidx ? 2 : (ldx == cols ? 0 : 1);
  const int grid = grid_for(nvec, QT * QU);
#define MX_QMX(T, MODE) hipLaunchKernelGGL((k_quant_mx<T, MODE>), dim3(grid), dim3(QT), 0, st, (const T*)x, ldx, vpr, nvec, codes, scales, gidx, x_rows)
#define MX_QMXF(T, MODE) hipLaunchKernelGGL((k_quant_mx<T, MODE, true>), dim3(grid), dim3(QT), 0, st, (const T*)x, ldx, vpr, nvec, codes, scales, gidx, x_rows)
  if (floor_rule) {
    if (mode == 2) return hipErrorInvalidValue;
    if (xdt_bf16) { if (mode == 0) MX_QMXF(uint16_t, 0); else MX_QMXF(uint16_t, 1); }
    else { if (mode == 0) MX_QMXF(float, 0); else MX_QMXF(float, 1); }
#undef MX_QMXF
    return hipGetLastError();
  }
  if (xdt_bf16) {
    if (mode == 0) MX_QMX(uint16_t, 0); else if (mode == 1) MX_QMX(uint16_t, 1); else MX_QMX(uint16_t, 2);
  } else {
    if (mode == 0) MX_QMX(float, 0); else if (mode == 1) MX_QMX(float, 1); else MX_QMX(float, 2);
  }
#undef MX_QMX
  return hipGetLastError();
}

int nv_partials_count(int64_t rows, int64_t cols, int xdt_bf16) {
  const int epl = xdt_bf16 ? 8 : 4;
  // Every quantize workgroup first reduces all partials: for tensors of up to
  // 2^23 16-byte vectors (workgroups live briefly) at most 1024 of them; larger
  // tensors keep the full amax-pass grid.
  const uint64_t nvec = (uint64_t)(rows * cols / epl);
  const int n = grid_for(nvec, QT * 4);
  // a multiple of 4 (the quantize kernel reads them as 16-byte vectors); the
  // extra amax workgroups find no vectors and write 0
  return ((nvec <= (1ull << 23) && n > 1024 ? 1024 : n) + 3) & ~3;
}

// k_quant_nv workgroups per CU: as many as its registers keep resident (5
// waves per SIMD for fp32 input, 6 for bf16)
constexpr int QNV_WG_PER_CU_F32 = 5, QNV_WG_PER_CU_BF16 = 6;

hipError_t launch_quant_nv(const void* x, int xdt_bf16, int64_t ldx, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, float* gscale, bool static_global, uint32_t* partial, hipStream_t st) {
  const int epl = xdt_bf16 ? 8 : 4;
  const uint32_t vpr = (uint32_t)(cols / epl);
  const uint32_t nvec = (uint32_t)(rows * cols / epl);
  const bool contig = (ldx == cols);
  int npart = 0;
  if (!static_global) {
    npart = nv_partials_count(rows, cols, xdt_bf16);
#define MX_ABSMAX(T, C) hipLaunchKernelGGL((k_absmax<T, C>), dim3(npart), dim3(QT), 0, st, (const T*)x, ldx, vpr, nvec, partial)
    if (xdt_bf16) { if (contig) MX_ABSMAX(uint16_t, true); else MX_ABSMAX(uint16_t, false); }
    else { if (contig) MX_ABSMAX(float, true); else MX_ABSMAX(float, false); }
#undef MX_ABSMAX
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const uint32_t bpr = (uint32_t)(cols / 16), nblk = (uint32_t)(rows * cols / 16);
  if (nblk == 0) return hipSuccess;   // (the entry point returns before this for empty tensors)
  // Only resident workgroups, each wave walking the same number of steps:
  // no partly filled last round of waves.
  const uint64_t cap_lanes = (uint64_t)(xdt_bf16 ? QNV_WG_PER_CU_BF16 : QNV_WG_PER_CU_F32) * 256 * QT;
  const uint64_t steps = (nblk + cap_lanes - 1) / cap_lanes;
  const int grid = (int)((nblk + steps * QT - 1) / (steps * QT));
  const uint32_t* pp = static_global ? nullptr : partial;
#define MX_QNV(T, C) hipLaunchKernelGGL((k_quant_nv<T, C>), dim3(grid), dim3(QT), 0, st, (const T*)x, ldx, bpr, nblk, codes, scales, gscale, pp, npart)
  if (xdt_bf16) { if (contig) MX_QNV(uint16_t, true); else MX_QNV(uint16_t, false); }
  else { if (contig) MX_QNV(float, true); else MX_QNV(float, false); }
#undef MX_QNV
  return hipGetLastError();
}

hipError_t launch_dequant(bool nv, const uint8_t* codes, const uint8_t* scales, const float* gscale, int64_t rows,
                          int64_t cols, void* y, bool out_bf16, int64_t ldy, hipStream_t st) {
  const uint32_t wpr = (uint32_t)(cols / 8);
  const uint32_t nwords = (uint32_t)(rows * cols / 8);
  const bool contig = (ldy == cols);
  const int grid = grid_for(nwords, QT * 4);
#define MX_DQ(NVF, B, C) hipLaunchKernelGGL((k_dequant<NVF, B, C>), dim3(grid), dim3(QT), 0, st, (const uint32_t*)codes, scales, gscale, wpr, nwords, y, ldy)
  if (nv) {
    if (out_bf16) { if (contig) MX_DQ(true, true, true); else MX_DQ(true, true, false); }
    else { if (contig) MX_DQ(true, false, true); else MX_DQ(true, false, false); }
  } else {
    if (out_bf16) { if (contig) MX_DQ(false, true, true); else MX_DQ(false, true, false); }
    else { if (contig) MX_DQ(false, false, true); else MX_DQ(false, false, false); }
  }
#undef MX_DQ
  return hipGetLastError();
}

constexpr int QF6_WG_PER_CU_F32 = 4, QF6_WG_PER_CU_BF16 = 5;   // k_quant_fp6: resident workgroups per CU

hipError_t launch_quant_wide(int fmt, const void* x, int xdt_bf16, int64_t ldx, int64_t rows, int64_t cols,
                             uint8_t* codes, uint8_t* scales, hipStream_t st, bool floor_rule) {
  const int epl = xdt_bf16 ? 8 : 4;
  const uint32_t vpr = (uint32_t)(cols / epl);
  const uint32_t nvec = (uint32_t)(rows * cols / epl);
  const bool contig = ldx == cols;
  if ((fmt == 2 || fmt == 3) && !floor_rule) {
    // one lane per block; only resident workgroups, each wave walking the
    // same number of steps
    const uint32_t bpr = (uint32_t)(cols / 32), nblk = (uint32_t)(rows * cols / 32);
    if (nblk == 0) return hipSuccess;
    const uint64_t cap = (uint64_t)(xdt_bf16 ? QF6_WG_PER_CU_BF16 : QF6_WG_PER_CU_F32) * 256 * QT;
    const uint64_t steps = (nblk + cap - 1) / cap;
    const int g6 = (int)((nblk + steps * QT - 1) / (steps * QT));
#define MX_QF6(T, F, C) hipLaunchKernelGGL((k_quant_fp6<T, F, C>), dim3(g6), dim3(QT), 0, st, (const T*)x, ldx, bpr, nblk, codes, scales)
#define MX_QF6C(T, F) if (contig) MX_QF6(T, F, true); else MX_QF6(T, F, false)
    if (xdt_bf16) { if (fmt == 2) { MX_QF6C(uint16_t, 2); } else { MX_QF6C(uint16_t, 3); } }
    else { if (fmt == 2) { MX_QF6C(float, 2); } else { MX_QF6C(float, 3); } }
#undef MX_QF6C
#undef MX_QF6
    return hipGetLastError();
  }
  const int grid = grid_for(nvec, QT * QU);
#define MX_QW4(T, F, C, FL) hipLaunchKernelGGL((k_quant_wide<T, F, C, FL>), dim3(grid), dim3(QT), 0, st, (const T*)x, ldx, vpr, nvec, codes, scales)
#define MX_QW3(T, F, C) if (floor_rule) MX_QW4(T, F, C, true); else MX_QW4(T, F, C, false)
#define MX_QW2(T, F) if (contig) { MX_QW3(T, F, true); } else { MX_QW3(T, F, false); }
#define MX_QW(F) if (xdt_bf16) { MX_QW2(uint16_t, F); } else { MX_QW2(float, F); }
  switch (fmt) {
    case 0: MX_QW(0); break;
    case 1: MX_QW(1); break;
    case 2: MX_QW(2); break;
    case 3: MX_QW(3); break;
    default: return hipErrorInvalidValue;
  }
#undef MX_QW
#undef MX_QW2
#undef MX_QW3
#undef MX_QW4
  return hipGetLastError();
}

hipError_t launch_dequant_wide(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, void* y,
                               bool out_bf16, int64_t ldy, hipStream_t st) {
  const uint32_t hpr = (uint32_t)(cols / 16);
  const uint32_t nhalf = (uint32_t)(rows * cols / 16);
  const bool contig = ldy == cols;
  const int grid = grid_for(nhalf, QT * 4);
#define MX_DW3(F, B, C) hipLaunchKernelGGL((k_dequant_wide<F, B, C>), dim3(grid), dim3(QT), 0, st, codes, scales, hpr, nhalf, y, ldy)
#define MX_DW2(F, B) if (contig) MX_DW3(F, B, true); else MX_DW3(F, B, false)
#define MX_DW(F) if (out_bf16) { MX_DW2(F, true); } else { MX_DW2(F, false); }
  switch (fmt) {
    case 0: MX_DW(0); break;
    case 1: MX_DW(1); break;
    case 2: MX_DW(2); break;
    case 3: MX_DW(3); break;
    default: return hipErrorInvalidValue;
  }
#undef MX_DW
#undef MX_DW2
#undef MX_DW3
  return hipGetLastError();
}

}  // namespace mxk
