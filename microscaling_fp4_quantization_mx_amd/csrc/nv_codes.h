// NVFP4 element coding by the hardware E2M1 conversion (gfx950), shared by
// the standalone quantizer and the fused RMSNorm quantizer.
#pragma once
#include "mx_device.h"

namespace mxk {

// NVFP4 element codes by the hardware E2M1 conversion, bracketed.  The code
// of x in a block of unit y is the E2M1 value nearest the real quotient x / y
// (ties to the even code, saturating at 6), which is what the boundary test
// above computes.  With r = fp32(1/y), rlo = fp32(r (1 - 2^-21)) and
// rhi = fp32(r (1 + 2^-21)), the products x * rlo and x * rhi rounded to fp32
// lie strictly below and above |x / y| in magnitude (three roundings move a
// value by less than 3 * 2^-24 relative, inside the 2^-21 margin; products
// that land among fp32 subnormals are far below the first boundary, where
// every candidate's code is 0).  The conversion rounds monotonically, so
// where it gives the two products the same code, that is x's code; where
// they differ, x / y lies within 2^-20 of a boundary and the caller takes the
// boundary test.  Valid for finite x and 2^-125 <= y <= 2^125 with
// max |x| / y < 2^100 (nv_fast_setup checks this per block), and for y == 0
// (rlo = rhi = 0: every code is +-0, as the boundary test gives).
struct NvFast {
  float rlo, rhi;
  bool ok;
};
__device__ __forceinline__ NvFast nv_fast_setup(double y, uint32_t amax_bits) {
  NvFast f;
  if (y == 0.0) {
    f.rlo = f.rhi = 0.0f;
    f.ok = amax_bits < 0x7f800000u;
    return f;
  }
  const float r = (float)(1.0 / y);
  f.rlo = r * (1.0f - 0x1p-21f);
  f.rhi = r * (1.0f + 0x1p-21f);
  f.ok = amax_bits < 0x7f800000u && y >= 0x1p-125 && y <= 0x1p125 && (double)ffrom(amax_bits) < y * 0x1p100;
  return f;
}
// Codes of 8 elements (fp32 bit patterns) into one 32-bit word, element 0 in
// the low nibble; returns false where the bracket straddles a boundary.
__device__ __forceinline__ bool nv_fast_codes8(const uint32_t* xb, const NvFast& f, uint32_t& w) {
  uint32_t lo = 0, hi = 0;
  lo = cvt_fp4x2<0>(lo, ffrom(xb[0]) * f.rlo, ffrom(xb[1]) * f.rlo, 1.0f);
  hi = cvt_fp4x2<0>(hi, ffrom(xb[0]) * f.rhi, ffrom(xb[1]) * f.rhi, 1.0f);
  lo = cvt_fp4x2<1>(lo, ffrom(xb[2]) * f.rlo, ffrom(xb[3]) * f.rlo, 1.0f);
  hi = cvt_fp4x2<1>(hi, ffrom(xb[2]) * f.rhi, ffrom(xb[3]) * f.rhi, 1.0f);
  lo = cvt_fp4x2<2>(lo, ffrom(xb[4]) * f.rlo, ffrom(xb[5]) * f.rlo, 1.0f);
  hi = cvt_fp4x2<2>(hi, ffrom(xb[4]) * f.rhi, ffrom(xb[5]) * f.rhi, 1.0f);
  lo = cvt_fp4x2<3>(lo, ffrom(xb[6]) * f.rlo, ffrom(xb[7]) * f.rlo, 1.0f);
  hi = cvt_fp4x2<3>(hi, ffrom(xb[6]) * f.rhi, ffrom(xb[7]) * f.rhi, 1.0f);
  w = lo;
  return lo == hi;
}

// nv_code (the E2M1 state of |x| against the seven fp32 thresholds U of a
// block, sign kept) with the thresholds picked by value masks rather than by
// index, so that U stays in registers (selects by index have made the compiler
// place U in scratch memory).
__device__ __forceinline__ uint32_t nv_code_sel(uint32_t xbits, const uint32_t U[7]) {
  const uint32_t a = xbits & 0x7fffffffu;
  const uint32_t m4 = a >= U[3] ? ~0u : 0u;
  const uint32_t t2 = (U[1] & ~m4) | (U[5] & m4);
  const uint32_t m2 = a >= t2 ? ~0u : 0u;
  const uint32_t t1 = (((U[0] & ~m2) | (U[2] & m2)) & ~m4) | (((U[4] & ~m2) | (U[6] & m2)) & m4);
  const uint32_t c = (m4 & 4u) | (m2 & 2u) | (a >= t1 ? 1u : 0u);
  return c | ((xbits >> 31) << 3);
}

}  // namespace mxk
