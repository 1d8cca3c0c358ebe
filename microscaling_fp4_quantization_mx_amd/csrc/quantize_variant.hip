// Variants of block quantization with E8M0 scales, for gfx950: any block
// length (16 or 32), an optional per-tensor scale g inside the block scale,
// the OCP floor rule as an alternative exponent rule, and rows whose length
// is not a multiple of the block (zero-padded).  These complete the pages'
// emulation surface ("NVFP4 Architecture", section "1. The Dual-Level
// Mathematical Formulation", equation S_block with S_global, and section
// "End-to-End Implementation": block length 16 by default, flattened tensor
// zero-padded to whole blocks); the common cases run in quantize.hip.
//
// One thread per block: the block's elements are loaded with bounds checks
// (padding reads as +0), the exponent is found exactly, and each element's
// code is the nearest one to |x| / (g 2^e), decided by comparing |x| with the
// exact fp64 midpoints between neighbouring codes times the unit g 2^e (the
// products are exact: a midpoint has at most 6 significant bits and g 24).
#include "mx_device.h"
#include "mx_kernels.h"

namespace mxk {

struct VarFmt {
  int ebits, mbits, bias, bits;
  float emax;
  int pexp;   // floor(log2 emax)
};

// element formats by the block-scaled MFMA's code: E4M3, E5M2, E2M3, E3M2, E2M1
__device__ __forceinline__ VarFmt var_fmt(int f) {
  switch (f) {
    case 0: return {4, 3, 7, 8, 448.0f, 8};
    case 1: return {5, 2, 15, 8, 57344.0f, 15};
    case 2: return {2, 3, 1, 6, 7.5f, 2};
    case 3: return {3, 2, 3, 6, 28.0f, 4};
    default: return {2, 1, 1, 4, 6.0f, 2};
  }
}

// value of magnitude code c (no sign bit), exact in fp64
__device__ __forceinline__ double var_value(const VarFmt& F, int c) {
  const int e = c >> F.mbits, m = c & ((1 << F.mbits) - 1);
  const double frac = (double)m / (double)(1 << F.mbits);
  return e == 0 ? ldexp(frac, 1 - F.bias) : ldexp(1.0 + frac, e - F.bias);
}

// largest magnitude code (the one whose value is emax)
__device__ __forceinline__ int var_max_code(const VarFmt& F) {
  int c = (1 << (F.bits - 1)) - 1;
  while (var_value(F, c) > (double)F.emax) --c;
  return c;
}

// nearest magnitude code of a >= 0 for the unit u (exact decision)
__device__ __forceinline__ int var_nearest(const VarFmt& F, int cmax, double a, double u) {
  // estimate from the rounded quotient, then correct against exact midpoints
  const double v = a / u;
  int lo = 0, hi = cmax;
  while (lo < hi) {   // largest code with value <= v (binary search, <= 7 steps)
    const int mid = (lo + hi + 1) >> 1;
    if (var_value(F, mid) <= v) lo = mid; else hi = mid - 1;
  }
  int c = lo;
  for (int it = 0; it < 2; ++it) {
    if (c < cmax) {
      const double t = 0.5 * (var_value(F, c) + var_value(F, c + 1)) * u;
      if (a > t || (a == t && (c & 1))) { ++c; continue; }
    }
    if (c > 0) {
      const double t = 0.5 * (var_value(F, c - 1) + var_value(F, c)) * u;
      if (a < t || (a == t && (c & 1))) { --c; continue; }
    }
    break;
  }
  return c;
}

template <typename TIn>
__device__ __forceinline__ float load_elem(const TIn* p) {
  if constexpr (sizeof(TIn) == 4) return *reinterpret_cast<const float*>(p);
  else return ffrom((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
}

template <typename TIn>
__global__ __launch_bounds__(256) void k_quant_variant(const TIn* __restrict__ x, int64_t ldx, int64_t rows, int64_t cols,
                                                       int fmt, int block, int floor_rule,
                                                       const float* __restrict__ gptr, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const VarFmt F = var_fmt(fmt);
  const int cmax = var_max_code(F);
  const int64_t nb = (cols + block - 1) / block;
  const int64_t row_bytes = nb * block * F.bits / 8;
  const double g = gptr ? (double)*gptr : 1.0;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < rows * nb; t += (int64_t)gridDim.x * 256) {
    const int64_t r = t / nb, b = t - r * nb;
    const int64_t c0 = b * block;
    float v[32];
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = (i < block && c0 + i < cols) ? load_elem(x + r * ldx + c0 + i) : 0.0f;
      if (i < block) am = fmaxf(am, fabsf(v[i]));
    }
    const double m = fmax((double)am, (double)1e-8f);
    int e;
    if (!floor_rule) {
      // smallest e with m <= emax * g * 2^e
      const double lim = (double)F.emax * g;
      e = (int)ceil(log2(m / lim));
      for (int it = 0; it < 2; ++it) {
        if (lim * ldexp(1.0, e) < m) ++e;
        if (lim * ldexp(1.0, e - 1) >= m) --e;
      }
    } else {
      int ex;
      frexp(m, &ex);          // m = f * 2^ex, f in [0.5, 1): floor(log2 m) = ex - 1
      e = ex - 1 - F.pexp;
    }
    const double u = g * ldexp(1.0, e);
    uint8_t* crow = codes + r * row_bytes + (c0 * F.bits) / 8;
    uint64_t acc = 0;
    int nbits = 0, outb = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i >= block) break;
      const uint32_t xb = fbits(v[i]);
      const int cm = var_nearest(F, cmax, (double)fabsf(v[i]), u);
      const uint32_t code = (uint32_t)cm | ((xb >> 31) << (F.bits - 1));
      acc |= (uint64_t)code << nbits;
      nbits += F.bits;
      while (nbits >= 8) {
        crow[outb++] = (uint8_t)acc;
        acc >>= 8;
        nbits -= 8;
      }
    }
    scales[r * nb + b] = (uint8_t)(e + 127);
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_dequant_variant(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ gptr, int64_t rows, int64_t cols,
                                                         int fmt, int block, void* __restrict__ y, int64_t ldy) {
  const VarFmt F = var_fmt(fmt);
  const int64_t nb = (cols + block - 1) / block;
  const int64_t row_bytes = nb * block * F.bits / 8;
  const bool has_g = gptr != nullptr;
  const float g = has_g ? *gptr : 1.0f;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < rows * nb; t += (int64_t)gridDim.x * 256) {
    const int64_t r = t / nb, b = t - r * nb;
    const int64_t c0 = b * block;
    const int sexp = (int)scales[r * nb + b] - 127;
    const uint8_t* crow = codes + r * row_bytes + (c0 * F.bits) / 8;
    uint64_t acc = 0;
    int nbits = 0, inb = 0;
    for (int i = 0; i < block; ++i) {
      while (nbits < F.bits) {
        acc |= (uint64_t)crow[inb++] << nbits;
        nbits += 8;
      }
      const uint32_t code = (uint32_t)(acc & ((1u << F.bits) - 1u));
      acc >>= F.bits;
      nbits -= F.bits;
      if (c0 + i >= cols) continue;
      const int cm = (int)(code & ((1u << (F.bits - 1)) - 1u));
      float q = (float)var_value(F, cm);
      q = (code >> (F.bits - 1)) ? -q : q;
      float val = __builtin_ldexpf(q, sexp);
      if (has_g) val = val * g;
      if (OUT_BF16)
        reinterpret_cast<uint16_t*>(y)[r * ldy + c0 + i] = (uint16_t)f32_to_bf16_rne(val);
      else
        reinterpret_cast<float*>(y)[r * ldy + c0 + i] = val;
    }
  }
}

// ---------------------------------------------------------------------------
// E2M1 elements (the FP4 variants) on a vector path: a thread owns 8
// consecutive elements of a padded row (one 32-bit word of codes), the 2 or 4
// threads of a block combine their maxima by lane exchange, and each element
// is decided by seven integer compares of |x| with per-block thresholds.  The
// thresholds are the exact midpoints between neighbouring E2M1 values times
// the unit u = g 2^e, formed in fp64 (exact) and rounded to fp32 towards the
// side that keeps the decision: a strict "above" test (ties to the lower,
// even code) against the threshold rounded down, an "at or above" test (ties
// to the upper, even code) against it rounded up; for g = 1 they are exact
// fp32 values.  Decisions and exponents are those of the per-block kernel.
// ---------------------------------------------------------------------------
template <int LPB>
__device__ __forceinline__ uint32_t group_umax(uint32_t v) {
  if constexpr (LPB >= 2) v = umax_xor(v, 1);
  if constexpr (LPB >= 4) v = umax_xor(v, 2);
  return v;
}

// fp32 rounding of a positive fp64 value towards -inf (DOWN) or +inf
__device__ __forceinline__ uint32_t f32_dir_bits(double t, bool down) {
  const float r = (float)t;
  uint32_t b = fbits(r);
  if (down && (double)r > t) --b;
  if (!down && (double)r < t) ++b;
  return b;
}

// the fp32 bit patterns of elements c0 .. c0 + 7 of a row (zeros past cols);
// VEC: the row start is 16-byte aligned, so whole groups use 16-byte loads
template <typename TIn, bool VEC>
__device__ __forceinline__ void load8(const TIn* xr, int64_t c0, int64_t cols, uint32_t xb[8]) {
  if (VEC && c0 + 8 <= cols) {
    if constexpr (sizeof(TIn) == 4) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(xr + c0), b = *reinterpret_cast<const u32x4*>(xr + c0 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) { xb[i] = a[i]; xb[4 + i] = b[i]; }
    } else {
      const u32x4 a = *reinterpret_cast<const u32x4*>(xr + c0);
#pragma unroll
      for (int i = 0; i < 4; ++i) { xb[2 * i] = a[i] << 16; xb[2 * i + 1] = a[i] & 0xffff0000u; }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) xb[i] = c0 + i < cols ? fbits(load_elem(xr + c0 + i)) : 0u;
  }
}

template <typename TIn, int B, bool HAS_G, bool FLOOR, bool VEC>
__global__ __launch_bounds__(256) void k_quant_v4(const TIn* __restrict__ x, int64_t ldx, int64_t rows, int64_t cols,
                                                  const float* __restrict__ gptr, uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  constexpr int LPB = B / 8;
  const int64_t nb = (cols + B - 1) / B;
  const int64_t U = nb * LPB;                      // 8-element units per padded row
  const double g = HAS_G ? (double)*gptr : 1.0;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < rows * U; t += (int64_t)gridDim.x * 256) {
    const int64_t r = t / U, u = t - r * U;
    const int64_t c0 = 8 * u;
    uint32_t xb[8];
    load8<TIn, VEC>(x + r * ldx, c0, cols, xb);
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = max(am, xb[i] & 0x7fffffffu);
    am = group_umax<LPB>(am);
    const uint32_t mb = max(am, fbits(1e-8f));     // max(m, 1e-8), fp32
    int e;
    if (FLOOR) {
      e = (int)(mb >> 23) - 127 - 2;               // floor(log2 m) - floor(log2 6)
    } else if (!HAS_G) {
      e = (int)(mb >> 23) - 127 - 2 + ((mb & 0x7fffffu) > 0x400000u ? 1 : 0);   // m <= 6 * 2^e
    } else {
      // smallest e with m <= 6 g 2^e: with m = fm 2^em and 6g = fl 2^el
      // (fm, fl in [0.5, 1)), e = em - el + [fm > fl]
      int em, el;
      const double fm = frexp((double)ffrom(mb), &em), fl = frexp(6.0 * g, &el);
      e = em - el + (fm > fl ? 1 : 0);
    }
    uint32_t T[7];
    if (HAS_G) {
      const double unit = ldexp(g, e);
      const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
      for (int i = 0; i < 7; ++i) T[i] = f32_dir_bits(mids[i] * unit, (i & 1) == 0);
    } else {
      const float unit = pow2f(e);
      const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
#pragma unroll
      for (int i = 0; i < 7; ++i) T[i] = fbits(mids[i] * unit);
    }
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t a = xb[k] & 0x7fffffffu;
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < 7; ++i) c += ((i & 1) ? (a >= T[i]) : (a > T[i])) ? 1u : 0u;
      word |= (c | ((xb[k] >> 31) << 3)) << (4 * k);
    }
    *reinterpret_cast<uint32_t*>(codes + r * (nb * B / 2) + 4 * u) = word;
    if (u % LPB == 0) scales[r * nb + u / LPB] = (uint8_t)(e + 127);
  }
}

template <int B, bool HAS_G, bool OUT_BF16, bool VEC>
__global__ __launch_bounds__(256) void k_dequant_v4(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                    const float* __restrict__ gptr, int64_t rows, int64_t cols,
                                                    void* __restrict__ y, int64_t ldy) {
  constexpr int LPB = B / 8;
  const int64_t nb = (cols + B - 1) / B;
  const int64_t U = nb * LPB;
  const float g = HAS_G ? *gptr : 1.0f;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < rows * U; t += (int64_t)gridDim.x * 256) {
    const int64_t r = t / U, u = t - r * U;
    const int64_t c0 = 8 * u;
    const uint32_t word = *reinterpret_cast<const uint32_t*>(codes + r * (nb * B / 2) + 4 * u);
    const int sexp = (int)scales[r * nb + u / LPB] - 127;
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // q exactly (scale 1), then q * 2^e exactly, then one rounding by g
      const f32x2 q = k == 0   ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0)
                      : k == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1)
                      : k == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2)
                               : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
      v[2 * k] = __builtin_ldexpf(q.x, sexp);
      v[2 * k + 1] = __builtin_ldexpf(q.y, sexp);
      if (HAS_G) { v[2 * k] *= g; v[2 * k + 1] *= g; }
    }
    if (OUT_BF16) {
      uint16_t* yr = reinterpret_cast<uint16_t*>(y) + r * ldy + c0;
      if (VEC && c0 + 8 <= cols) {
        *reinterpret_cast<u32x4*>(yr) = u32x4{pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]),
                                              pack_bf16x2_rne(v[4], v[5]), pack_bf16x2_rne(v[6], v[7])};
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (c0 + k < cols) yr[k] = (uint16_t)f32_to_bf16_rne(v[k]);
      }
    } else {
      float* yr = reinterpret_cast<float*>(y) + r * ldy + c0;
      if (VEC && c0 + 8 <= cols) {
        *reinterpret_cast<f32x4*>(yr) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(yr + 4) = f32x4{v[4], v[5], v[6], v[7]};
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (c0 + k < cols) yr[k] = v[k];
      }
    }
  }
}

static int var_grid(int64_t items) {
  int64_t g = (items + 255) / 256;
  if (g > 256 * 16) g = 256 * 16;
  return (int)(g ? g : 1);
}

template <typename TIn, int B, bool HAS_G, bool FLOOR>
static void launch_quant_v4(const void* x, int64_t ldx, int64_t rows, int64_t cols, const float* g, uint8_t* codes,
                            uint8_t* scales, hipStream_t st) {
  const int64_t units = rows * ((cols + B - 1) / B) * (B / 8);
  const int grid = var_grid(units);
  // 16-byte loads need 16-byte aligned rows
  const bool vec = ((uintptr_t)x % 16 == 0) && (ldx * (int64_t)sizeof(TIn)) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((k_quant_v4<TIn, B, HAS_G, FLOOR, true>), dim3(grid), dim3(256), 0, st, (const TIn*)x, ldx, rows,
                       cols, g, codes, scales);
  else
    hipLaunchKernelGGL((k_quant_v4<TIn, B, HAS_G, FLOOR, false>), dim3(grid), dim3(256), 0, st, (const TIn*)x, ldx,
                       rows, cols, g, codes, scales);
}

template <typename TIn>
static void launch_quant_v4_any(int block, bool floor_rule, const float* g, const void* x, int64_t ldx, int64_t rows,
                                int64_t cols, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  if (block == 16) {
    if (floor_rule) launch_quant_v4<TIn, 16, false, true>(x, ldx, rows, cols, g, codes, scales, st);
    else if (g) launch_quant_v4<TIn, 16, true, false>(x, ldx, rows, cols, g, codes, scales, st);
    else launch_quant_v4<TIn, 16, false, false>(x, ldx, rows, cols, g, codes, scales, st);
  } else {
    if (floor_rule) launch_quant_v4<TIn, 32, false, true>(x, ldx, rows, cols, g, codes, scales, st);
    else if (g) launch_quant_v4<TIn, 32, true, false>(x, ldx, rows, cols, g, codes, scales, st);
    else launch_quant_v4<TIn, 32, false, false>(x, ldx, rows, cols, g, codes, scales, st);
  }
}

hipError_t launch_quant_variant(int fmt, int block, bool floor_rule, const float* g, const void* x, int xdt_bf16,
                                int64_t ldx, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                hipStream_t st) {
  // E2M1 elements with 16- or 32-element blocks (the floor rule never with g)
  if (fmt == 4 && (block == 16 || block == 32) && !(floor_rule && g)) {
    if (xdt_bf16) launch_quant_v4_any<uint16_t>(block, floor_rule, g, x, ldx, rows, cols, codes, scales, st);
    else launch_quant_v4_any<float>(block, floor_rule, g, x, ldx, rows, cols, codes, scales, st);
    return hipGetLastError();
  }
  const int64_t nb = (cols + block - 1) / block;
  const int grid = var_grid(rows * nb);
  if (xdt_bf16)
    hipLaunchKernelGGL(k_quant_variant<uint16_t>, dim3(grid), dim3(256), 0, st, (const uint16_t*)x, ldx, rows, cols,
                       fmt, block, floor_rule ? 1 : 0, g, codes, scales);
  else
    hipLaunchKernelGGL(k_quant_variant<float>, dim3(grid), dim3(256), 0, st, (const float*)x, ldx, rows, cols, fmt,
                       block, floor_rule ? 1 : 0, g, codes, scales);
  return hipGetLastError();
}

template <int B, bool HAS_G>
static void launch_dequant_v4(const float* g, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                              void* y, bool out_bf16, int64_t ldy, hipStream_t st) {
  const int grid = var_grid(rows * ((cols + B - 1) / B) * (B / 8));
  const int64_t esz = out_bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)y % 16 == 0) && (ldy * esz) % 16 == 0;
#define MX_DQ4(BF, V) hipLaunchKernelGGL((k_dequant_v4<B, HAS_G, BF, V>), dim3(grid), dim3(256), 0, st, codes, scales, g, rows, cols, y, ldy)
  if (out_bf16) { if (vec) MX_DQ4(true, true); else MX_DQ4(true, false); }
  else { if (vec) MX_DQ4(false, true); else MX_DQ4(false, false); }
#undef MX_DQ4
}

hipError_t launch_dequant_variant(int fmt, int block, const float* g, const uint8_t* codes, const uint8_t* scales,
                                  int64_t rows, int64_t cols, void* y, bool out_bf16, int64_t ldy, hipStream_t st) {
  if (fmt == 4 && (block == 16 || block == 32)) {
    if (block == 16) { if (g) launch_dequant_v4<16, true>(g, codes, scales, rows, cols, y, out_bf16, ldy, st);
                       else launch_dequant_v4<16, false>(g, codes, scales, rows, cols, y, out_bf16, ldy, st); }
    else { if (g) launch_dequant_v4<32, true>(g, codes, scales, rows, cols, y, out_bf16, ldy, st);
           else launch_dequant_v4<32, false>(g, codes, scales, rows, cols, y, out_bf16, ldy, st); }
    return hipGetLastError();
  }
  const int64_t nb = (cols + block - 1) / block;
  const int grid = var_grid(rows * nb);
  if (out_bf16)
    hipLaunchKernelGGL(k_dequant_variant<true>, dim3(grid), dim3(256), 0, st, codes, scales, g, rows, cols, fmt, block,
                       y, ldy);
  else
    hipLaunchKernelGGL(k_dequant_variant<false>, dim3(grid), dim3(256), 0, st, codes, scales, g, rows, cols, fmt,
                       block, y, ldy);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Naive per-tensor FP4 (the pages' coarse baseline, "End-to-End
// Implementation", function naive_per_tensor_fp4; figure "The Outlier
// Distortion in Coarse-Grained FP4"): one fp32 scale s = max(max|x|, 1e-8) / 6
// for the whole tensor, every element the E2M1 state nearest to x / s.  The
// tensor max comes from per-workgroup partial maxima (k_absmax_any); a thread
// then codes 8 consecutive elements into one 32-bit word.
// ---------------------------------------------------------------------------
template <typename TIn, bool VEC>
__global__ __launch_bounds__(256) void k_absmax_any(const TIn* __restrict__ x, int64_t ldx, int64_t rows, int64_t cols,
                                                    uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[4];
  const int64_t U = (cols + 7) / 8;                // 8-element groups per row
  uint32_t am = 0;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < rows * U; t += (int64_t)gridDim.x * 256) {
    const int64_t r = t / U, c0 = 8 * (t - r * U);
    uint32_t xb[8];
    load8<TIn, VEC>(x + r * ldx, c0, cols, xb);
#pragma unroll
    for (int i = 0; i < 8; ++i) am = max(am, xb[i] & 0x7fffffffu);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) am = umax_xor(am, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

template <typename TIn, bool VEC>
__global__ __launch_bounds__(256) void k_quant_naive(const TIn* __restrict__ x, int64_t ldx, int64_t rows, int64_t cols,
                                                     const uint32_t* __restrict__ partial, int npart,
                                                     uint8_t* __restrict__ codes, float* __restrict__ sout) {
  __shared__ uint32_t red[4];
  uint32_t am = 0;
  for (int i = threadIdx.x; i < npart; i += 256) am = max(am, partial[i]);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) am = umax_xor(am, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  const float amax = ffrom(max(max(red[0], red[1]), max(red[2], red[3])));
  const float s = fmaxf(amax, 1e-8f) / 6.0f;   // IEEE fp32 division
  if (blockIdx.x == 0 && threadIdx.x == 0) *sout = s;
  uint32_t Ub[7];
  nv_boundaries((double)s, Ub);
  const int64_t half = cols / 2;                   // cols is even
  const int64_t U = (cols + 7) / 8;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < rows * U; t += (int64_t)gridDim.x * 256) {
    const int64_t r = t / U, c0 = 8 * (t - r * U);
    uint32_t xb[8];
    load8<TIn, VEC>(x + r * ldx, c0, cols, xb);
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) word |= nv_code(xb[k], Ub) << (4 * k);
    uint8_t* cr = codes + r * half + c0 / 2;
    if (c0 + 8 <= cols && half % 4 == 0) {
      *reinterpret_cast<uint32_t*>(cr) = word;     // 4-byte aligned: codes is 16-byte aligned
    } else {
      for (int k = 0; 2 * k < cols - c0 && k < 4; ++k) cr[k] = (uint8_t)(word >> (8 * k));
    }
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_dequant_naive(const uint8_t* __restrict__ codes, const float* __restrict__ sptr,
                                                       int64_t rows, int64_t cols, void* __restrict__ y, int64_t ldy) {
  const float s = *sptr;
  const int64_t half = cols / 2;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < rows * half; t += (int64_t)gridDim.x * 256) {
    const int64_t r = t / half, c = (t - r * half) * 2;
    const uint32_t byte = codes[r * half + (c >> 1)];
    const f32x2 q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0);
    const float v0 = q.x * s, v1 = q.y * s;
    if (OUT_BF16) {
      reinterpret_cast<uint16_t*>(y)[r * ldy + c] = (uint16_t)f32_to_bf16_rne(v0);
      reinterpret_cast<uint16_t*>(y)[r * ldy + c + 1] = (uint16_t)f32_to_bf16_rne(v1);
    } else {
      reinterpret_cast<float*>(y)[r * ldy + c] = v0;
      reinterpret_cast<float*>(y)[r * ldy + c + 1] = v1;
    }
  }
}

hipError_t launch_quant_naive(const void* x, int xdt_bf16, int64_t ldx, int64_t rows, int64_t cols, uint8_t* codes,
                              float* s, uint32_t* partial, int max_partials, hipStream_t st) {
  const int64_t groups = rows * ((cols + 7) / 8);
  int npart = var_grid(groups);
  // every quantize workgroup first reduces all partials (see nv_partials_count)
  if (groups <= (int64_t)1 << 22 && npart > 1024) npart = 1024;
  if (npart > max_partials) npart = max_partials;
  const int grid = var_grid(groups);
  const int64_t esz = xdt_bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)x % 16 == 0) && (ldx * esz) % 16 == 0;
#define MX_NAIVE(T, V)                                                                                           \
  do {                                                                                                         \
    hipLaunchKernelGGL((k_absmax_any<T, V>), dim3(npart), dim3(256), 0, st, (const T*)x, ldx, rows, cols, partial); \
    hipLaunchKernelGGL((k_quant_naive<T, V>), dim3(grid), dim3(256), 0, st, (const T*)x, ldx, rows, cols, partial, \
                       npart, codes, s);                                                                       \
  } while (0)
  if (xdt_bf16) { if (vec) MX_NAIVE(uint16_t, true); else MX_NAIVE(uint16_t, false); }
  else { if (vec) MX_NAIVE(float, true); else MX_NAIVE(float, false); }
#undef MX_NAIVE
  return hipGetLastError();
}

hipError_t launch_dequant_naive(const uint8_t* codes, const float* s, int64_t rows, int64_t cols, void* y, bool out_bf16,
                                int64_t ldy, hipStream_t st) {
  const int grid = var_grid(rows * cols / 2);
  if (out_bf16)
    hipLaunchKernelGGL(k_dequant_naive<true>, dim3(grid), dim3(256), 0, st, codes, s, rows, cols, y, ldy);
  else
    hipLaunchKernelGGL(k_dequant_naive<false>, dim3(grid), dim3(256), 0, st, codes, s, rows, cols, y, ldy);
  return hipGetLastError();
}

}  // namespace mxk
