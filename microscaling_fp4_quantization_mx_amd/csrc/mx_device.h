// Device helpers shared by the gfx950 kernels of libmx: number-format codecs
// and small bit tricks.  Everything here is written for CDNA4 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t fbits(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float ffrom(uint32_t u) { return __uint_as_float(u); }

// bf16 <-> fp32.  bf16 -> fp32 is exact; fp32 -> bf16 rounds to nearest even
// (finite inputs).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return ffrom(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return ffrom(pair & 0xffff0000u); }
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = fbits(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two floats -> packed bf16 pair (lo in bits 0-15), round to nearest even, in
// one v_cvt_pk_bf16_f32.  Identical to f32_to_bf16_rne for every non-NaN
// input (a NaN comes out as a quiet NaN).
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t b = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &b, 4);
  return u;
}

// E8M0 block exponent of an MXFP4 block from the bit pattern of its max |x|:
// the smallest e with max <= 6 * 2^e, floored at -29 (the 1e-8 guard of the
// pages' emulation: ceil(log2(1e-8 / 6)) = -29).  For a normal max with
// biased exponent F and mantissa field f, max / 6 = 2^(F-127-2) * (1+f)/1.5,
// so e = F - 129 + [f > 0x400000] exactly; zero and subnormal maxima give -29.
__device__ __forceinline__ int mx_block_exp(uint32_t amax_bits) {
  int e = (int)(amax_bits >> 23) - 129 + ((amax_bits & 0x7fffffu) > 0x400000u ? 1 : 0);
  return e < -29 ? -29 : e;
}
// fp32 2^e for e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) { return ffrom((uint32_t)(e + 127) << 23); }

// FP8 E4M3 ("fn") round-to-nearest-even of r >= 0 with saturation to 448
// (code 0x7E).  r is an fp64 quotient; an fp64 result cannot land on an E4M3
// half-way point unless the exact quotient is one (the dividend has 24 and the
// divisor 26 significant bits), so rounding the fp64 value is exact RNE.
__device__ __forceinline__ uint32_t e4m3_rne_sat(double r) {
  if (!(r < 448.0)) return 0x7Eu;
  if (r < 0.015625) {                      // below 2^-6: subnormal steps of 2^-9
    return (uint32_t)rint(r * 512.0);      // 0..8 (8 is 2^-6, code 0x08)
  }
  uint64_t b = (uint64_t)__double_as_longlong(r);
  uint64_t t = b >> 49;                    // biased exponent (11) | top 3 mantissa bits
  const uint64_t rem = b & ((1ull << 49) - 1);
  const uint64_t half = 1ull << 48;
  t += (rem > half || (rem == half && (t & 1))) ? 1 : 0;
  uint32_t code = (uint32_t)(t - ((uint64_t)(1023 - 7) << 3));
  return code > 0x7Eu ? 0x7Eu : code;
}
// E4M3 byte (non-negative) -> fp32 value (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;
  return ffrom(((e + 120u) << 23) | (m << 20));
}

// E2M1 boundaries for NVFP4 elements.  For a block whose unit is y = s * g
// (exact in fp64), the magnitude code of |x| is the number of boundaries j
// with |x| beyond y * {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}_j, where boundary
// j is crossed strictly when the lower state's code j is even (half-way
// values stay on the even code) and inclusively when it is odd.  Each
// boundary becomes the smallest fp32 bit pattern that crosses it, so the
// element test is an unsigned compare of |x|'s bits.  y == 0 (scale rounded
// to zero) maps every element to code 0.
__device__ __forceinline__ void nv_boundaries(double y, uint32_t U[7]) {
  const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    double T = mids[j] * y;
    float f = (float)T;
    uint32_t ub = fbits(f);
    double fd = (double)f;
    bool ok = (j & 1) ? (fd >= T) : (fd > T);
    U[j] = (y == 0.0) ? 0xffffffffu : (ok ? ub : ub + 1u);
  }
}
// The boundaries increase with j, so the count is found by bisection: three
// compares instead of seven.
__device__ __forceinline__ uint32_t nv_code(uint32_t xbits, const uint32_t U[7]) {
  const uint32_t a = xbits & 0x7fffffffu;
  uint32_t c = a >= U[3] ? 4u : 0u;
  c += a >= (c ? U[5] : U[1]) ? 2u : 0u;
  c += a >= ((c & 4u) ? ((c & 2u) ? U[6] : U[4]) : ((c & 2u) ? U[2] : U[0])) ? 1u : 0u;
  return c | ((xbits >> 31) << 3);
}

// Hardware E2M1 conversion (v_cvt_scalef32_pk_fp4_f32): two fp32 values
// divided by the power-of-two `scale` and rounded to nearest-even E2M1 with
// saturation at +-6 and the sign kept (also of zero); written into byte SEL
// of `old`.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

// wave64 reductions via cross-lane xor shuffles.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier without the implicit wait for outstanding loads that
// __syncthreads() carries (callers issue the counted s_waitcnt they need).
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XOR swizzle of the eight 16-byte chunks of a 128-byte LDS row: the 32
// lanes that read one chunk column of 32 consecutive rows hit distinct banks.
__device__ __forceinline__ int swz8r(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }

// Wait until at most VM of this wave's vector-memory operations (including
// direct-to-LDS loads) are outstanding.
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  // s_waitcnt encoding for gfx9: vmcnt in [3:0] and [15:14]; expcnt and
  // lgkmcnt at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x70 | 0xf00);
}

__device__ __forceinline__ uint32_t umax_xor(uint32_t v, int mask) {
  return max(v, (uint32_t)__shfl_xor((int)v, mask, 64));
}
__device__ __forceinline__ float fadd_xor(float v, int mask) { return v + __shfl_xor(v, mask, 64); }

}  // namespace mxk
