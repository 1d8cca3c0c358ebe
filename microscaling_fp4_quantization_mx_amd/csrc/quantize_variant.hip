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

static int var_grid(int64_t items) {
  int64_t g = (items + 255) / 256;
  if (g > 256 * 16) g = 256 * 16;
  return (int)(g ? g : 1);
}

hipError_t launch_quant_variant(int fmt, int block, bool floor_rule, const float* g, const void* x, int xdt_bf16,
                                int64_t ldx, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                hipStream_t st) {
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

hipError_t launch_dequant_variant(int fmt, int block, const float* g, const uint8_t* codes, const uint8_t* scales,
                                  int64_t rows, int64_t cols, void* y, bool out_bf16, int64_t ldy, hipStream_t st) {
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
// tensor max comes from per-workgroup partial maxima (k_absmax_any); one
// thread then packs two elements per byte.
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ __launch_bounds__(256) void k_absmax_any(const TIn* __restrict__ x, int64_t ldx, int64_t rows, int64_t cols,
                                                    uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[4];
  uint32_t am = 0;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < rows * cols; t += (int64_t)gridDim.x * 256) {
    const int64_t r = t / cols, c = t - r * cols;
    am = max(am, fbits(load_elem(x + r * ldx + c)) & 0x7fffffffu);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) am = umax_xor(am, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

template <typename TIn>
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
  uint32_t U[7];
  nv_boundaries((double)s, U);
  const int64_t half = cols / 2;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < rows * half; t += (int64_t)gridDim.x * 256) {
    const int64_t r = t / half, c = (t - r * half) * 2;
    const uint32_t a = fbits(load_elem(x + r * ldx + c)), b = fbits(load_elem(x + r * ldx + c + 1));
    codes[r * half + (c >> 1)] = (uint8_t)(nv_code(a, U) | (nv_code(b, U) << 4));
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
  int npart = var_grid(rows * cols);
  if (npart > max_partials) npart = max_partials;
  const int grid = var_grid(rows * cols / 2);
  if (xdt_bf16) {
    hipLaunchKernelGGL(k_absmax_any<uint16_t>, dim3(npart), dim3(256), 0, st, (const uint16_t*)x, ldx, rows, cols,
                       partial);
    hipLaunchKernelGGL(k_quant_naive<uint16_t>, dim3(grid), dim3(256), 0, st, (const uint16_t*)x, ldx, rows, cols,
                       partial, npart, codes, s);
  } else {
    hipLaunchKernelGGL(k_absmax_any<float>, dim3(npart), dim3(256), 0, st, (const float*)x, ldx, rows, cols, partial);
    hipLaunchKernelGGL(k_quant_naive<float>, dim3(grid), dim3(256), 0, st, (const float*)x, ldx, rows, cols, partial,
                       npart, codes, s);
  }
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
