// One 32-element MX block expanded to bf16 values q * 2^(E-127) with the
// gfx950 scaled conversions (v_cvt_scalef32_pk_bf16_fp4 / _fp8 / _bf8,
// v_cvt_scalef32_pk32_bf16_fp6 / _bf6), which multiply by their fp32 scale
// operand.  An element value has at most 4 significant bits, so it is exact in
// bf16 wherever it lies in bf16's normal range; the element formats are the MX
// family's ("MXFP4" card, section "Core Facts").
#pragma once
#include "mx_device.h"

namespace mxk {

// Element format codes of the block-scaled MFMA: E4M3 0, E5M2 1, E2M3 2,
// E3M2 3, E2M1 4.  Dwords of packed codes in one 32-element block.
template <int F>
struct MxElem {
  static constexpr int BITS = F <= 1 ? 8 : (F <= 3 ? 6 : 4);
  static constexpr int DW = BITS;   // 32 codes x BITS bits = BITS dwords
};

typedef __bf16 bf16x32_t __attribute__((ext_vector_type(32)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

// The 32 codes of one block (W dwords) -> 16 dwords of bf16 pairs, element
// order kept (o[i] holds elements 2i, 2i + 1).
template <int F>
__device__ __forceinline__ void expand_block_bf16(const uint32_t* w, float sc, uint32_t (&o)[16]) {
  if constexpr (F == 4) {                 // E2M1: 8 codes per dword
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      bf16x2 v[4];
      v[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], sc, 0);
      v[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], sc, 1);
      v[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], sc, 2);
      v[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], sc, 3);
#pragma unroll
      for (int q = 0; q < 4; ++q) __builtin_memcpy(&o[4 * d + q], &v[q], 4);
    }
  } else if constexpr (F == 0 || F == 1) {   // E4M3 / E5M2: 4 codes per dword
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      bf16x2 lo, hi;
      if constexpr (F == 0) {
        lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], sc, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], sc, true);
      } else {
        lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w[d], sc, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w[d], sc, true);
      }
      __builtin_memcpy(&o[2 * d], &lo, 4);
      __builtin_memcpy(&o[2 * d + 1], &hi, 4);
    }
  } else {                                    // E2M3 / E3M2: 32 codes in 6 dwords
    const u32x6 v = {w[0], w[1], w[2], w[3], w[4], w[5]};
    bf16x32_t r;
    if constexpr (F == 2) r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(v, sc);
    else r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(v, sc);
    __builtin_memcpy(&o[0], &r, 64);
  }
}

}  // namespace mxk
