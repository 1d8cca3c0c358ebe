// libmx C ABI: argument validation, workspace layout and kernel dispatch.
// Every check runs on the host before any HIP call, so an invalid call
// returns a negative status without touching the device.
#include <mutex>
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/mx.h"
#include "mx_kernels.h"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 33;   // rows * cols limit (32-bit vector indices)
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxPairs = (int64_t(1) << 31) - 1;   // routed (token, slot) pairs: int32 row indices
constexpr int32_t kMaxExperts = 1 << 16;
constexpr int64_t kMaxNormCols = 256 * 32 * 4;   // fused RMSNorm: a row stays in one workgroup's registers
constexpr size_t kNvPartialBytes = 4096 * sizeof(uint32_t);

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline int block_of(int32_t fmt) {
  return fmt == MX_FMT_NVFP4 || fmt == MX_FMT_MXFP4_K16 ? 16 : (fmt == MX_FMT_FP4_TENSOR ? 2 : 32);
}
inline bool fmt_known(int32_t fmt) { return fmt >= MX_FMT_MXFP4 && fmt <= MX_FMT_FP4_TENSOR; }
// formats with E8M0 block scales: rows of any length (the last block zero-padded)
inline bool fmt_e8m0(int32_t fmt) { return fmt != MX_FMT_NVFP4 && fmt != MX_FMT_FP4_TENSOR; }
inline int64_t pad_to(int64_t v, int64_t k) { return (v + k - 1) / k * k; }
// MXFP8 / MXFP6 (every MX element format but E2M1)
inline bool fmt_wide(int32_t fmt) { return fmt >= MX_FMT_MXFP8_E4M3 && fmt <= MX_FMT_MXFP6_E3M2; }
// element-format code of the block-scaled MFMA: E4M3 0, E5M2 1, E2M3 2, E3M2 3, E2M1 4
inline int mfma_fmt(int32_t fmt) {
  return (fmt == MX_FMT_MXFP4 || fmt == MX_FMT_MXFP4_K16) ? 4 : fmt - MX_FMT_MXFP8_E4M3;
}

inline size_t round256(size_t v) { return (v + 255) & ~size_t(255); }
inline int esize(int32_t dt) { return dt == MX_DT_F32 ? 4 : 2; }
inline bool dtype_ok(int32_t dt) { return dt == MX_DT_F32 || dt == MX_DT_BF16; }

// Descriptor checks common to every entry point.
int check_tensor(const mx_tensor* t) {
  if (!t) return MX_ERR_NULL;
  if (!fmt_known(t->fmt)) return MX_ERR_FORMAT;
  if (t->reserved != 0) return MX_ERR_SHAPE;
  if (t->rows < 0 || t->cols < 0 || t->rows > kMaxDim || t->cols > kMaxDim) return MX_ERR_SHAPE;
  if (t->rows > 0 && t->cols > 0 && t->rows > kMaxElems / t->cols) return MX_ERR_SHAPE;
  if (!fmt_e8m0(t->fmt) && t->cols % block_of(t->fmt) != 0) return MX_ERR_UNSUPPORTED;
  if (t->rows == 0 || t->cols == 0) return MX_OK;
  if (!t->codes || (!t->scales && t->fmt != MX_FMT_FP4_TENSOR)) return MX_ERR_NULL;
  if ((t->fmt == MX_FMT_NVFP4 || t->fmt == MX_FMT_FP4_TENSOR) && !t->global_scale) return MX_ERR_NULL;
  if (!al16(t->codes) || (t->scales && !al16(t->scales))) return MX_ERR_ALIGN;
  if (t->global_scale && (reinterpret_cast<uintptr_t>(t->global_scale) & 3u)) return MX_ERR_ALIGN;
  return MX_OK;
}

int check_dense_input(const void* x, int32_t dt, int64_t ld, int64_t rows, int64_t cols, bool any_pitch = false) {
  if (!dtype_ok(dt)) return MX_ERR_DTYPE;
  if (ld < cols) return MX_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MX_OK;
  if (!x) return MX_ERR_NULL;
  if (any_pitch) return (reinterpret_cast<uintptr_t>(x) % esize(dt)) ? MX_ERR_ALIGN : MX_OK;   // element loads
  if (!al16(x) || (ld * esize(dt)) % 16 != 0) return MX_ERR_ALIGN;
  return MX_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int hip_status(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

inline int elem_bits(int32_t fmt) {
  return fmt == MX_FMT_MXFP8_E4M3 || fmt == MX_FMT_MXFP8_E5M2 ? 8 : (fmt == MX_FMT_MXFP6_E2M3 || fmt == MX_FMT_MXFP6_E3M2 ? 6 : 4);
}
// Element format of a dynamically quantized A: flags bits 4-7 hold the format
// + 1, or 0 for the format of B.
constexpr int32_t kDynShift = 4;
constexpr int32_t kDynMask = 0xF << kDynShift;
inline int32_t dyn_a_fmt(const mx_gemm_args* a) {
  const int32_t sel = (a->flags & kDynMask) >> kDynShift;
  return sel ? sel - 1 : (a->b ? a->b->fmt : MX_FMT_MXFP4);
}
// MX formats a dynamic A can take: E2M1, E4M3, E5M2, E2M3, E3M2 elements with
// E8M0 scales over 32-element blocks
inline bool dyn_fmt_ok(int32_t fmt) { return fmt == MX_FMT_MXFP4 || fmt_wide(fmt); }
// codes then scale bytes of a dynamic A [M, K] (K % 32 == 0)
size_t dyn_codes_bytes(int32_t fmt, int64_t M, int64_t K) { return (size_t)(M * (K / 8 * elem_bits(fmt))); }
size_t dyn_a_bytes(int32_t fmt, int64_t M, int64_t K) {
  return round256(dyn_codes_bytes(fmt, M, K)) + round256((size_t)(M * K / 32));
}

// The fused quantize + GEMM kernel splits its tiles over the 8 XCDs of a
// 256-CU part (32 workgroups each).
constexpr int kFusedCUs = 256;
int device_cus() {
  static std::mutex mu;
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!cus[dev] && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus[dev] = -1;
  return cus[dev];
}
// Dynamic MXFP4 A with MX_GEMM_FUSED_QUANTIZE, of a shape the fused kernel
// takes (the workspace reserves its counters and partial tiles whenever this
// holds).
bool fused_shape(const mx_gemm_args* a) {
  return !a->a && (a->flags & MX_GEMM_FUSED_QUANTIZE) && a->b && a->b->fmt == MX_FMT_MXFP4 &&
         dyn_a_fmt(a) == MX_FMT_MXFP4 && (a->a_raw_dtype == MX_DT_F32 || a->a_raw_dtype == MX_DT_BF16) &&
         a->M > 0 && a->N > 0 && a->K > 0 && a->lda_raw < (int64_t(1) << 24) &&   // 32-bit offsets over 32 rows
         mxk::fused_fits(a->M, a->N, a->K, a->groups, kFusedCUs / 8);
}

// Scratch for the K parts of a partly filled last round of the MXFP4 x MXFP4
// GEMM (K % 256 == 0 paths; not the fused kernel, which splits on its own).
size_t split_bytes(const mx_gemm_args* a) {
  if (!a->b || fused_shape(a)) return 0;
  if (a->M <= 0 || a->N <= 0 || a->K <= 0 || a->groups < 0) return 0;
  const int32_t af = a->a ? a->a->fmt : dyn_a_fmt(a);
  if (a->b->fmt == MX_FMT_MXFP4 && af == MX_FMT_MXFP4)
    return mxk::gemm_mx_split_bytes(a->M, a->N, pad_to(a->K, 32), a->groups, device_cus());
  if (a->b->fmt == MX_FMT_NVFP4 && af == MX_FMT_NVFP4 && a->a && a->groups == 0)
    return mxk::gemm_nv_split_bytes(a->M, a->N, a->K, device_cus());
  return 0;
}
// Bytes of the workspace that the dynamic path's quantized A takes.
size_t ws_a_bytes(const mx_gemm_args* a) {
  if (!a->a && !(a->a_codes_out && a->a_scales_out) && a->M > 0 && a->K > 0 && dyn_fmt_ok(dyn_a_fmt(a)))
    return dyn_a_bytes(dyn_a_fmt(a), a->M, a->K);
  return 0;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

const char* mx_status_string(int status) {
  switch (status) {
    case MX_OK: return "MX_OK: success";
    case MX_ERR_NULL: return "MX_ERR_NULL: a required pointer is NULL";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE: negative or inconsistent sizes or leading dimensions";
    case MX_ERR_ALIGN: return "MX_ERR_ALIGN: pointer or row not 16-byte aligned";
    case MX_ERR_DTYPE: return "MX_ERR_DTYPE: unknown or unsupported element type";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED: valid but not provided by this library";
    case MX_ERR_HIP: return "MX_ERR_HIP: a HIP launch failed";
    case MX_ERR_WORKSPACE: return "MX_ERR_WORKSPACE: workspace missing or too small";
    case MX_ERR_FORMAT: return "MX_ERR_FORMAT: unknown format or mismatched operand formats";
    default: return "unknown mx_status";
  }
}

int mx_version(void) { return 10000; }

size_t mx_workspace_bytes(int32_t op, const void* desc, int32_t flags) {
  if (!desc) return 0;
  if (op == MX_OP_QUANTIZE) {
    const mx_tensor* t = static_cast<const mx_tensor*>(desc);
    if (t->fmt == MX_FMT_NVFP4 && !(flags & MX_QUANT_STATIC_GLOBAL)) return kNvPartialBytes;
    if (t->fmt == MX_FMT_FP4_TENSOR) return kNvPartialBytes;
    return 0;
  }
  if (op == MX_OP_GEMM) {
    const mx_gemm_args* a = static_cast<const mx_gemm_args*>(desc);
    // layout: [fused kernel's counters and partials][quantized A][split partials]
    const size_t n = ws_a_bytes(a);
    if (fused_shape(a)) return n + round256(mxk::fused_workspace_bytes());
    const size_t sb = split_bytes(a);
    return sb ? round256(n) + sb : n;
  }
  if (op == MX_OP_MOE_ROUTE) {
    const int32_t experts = *static_cast<const int32_t*>(desc);
    return experts > 0 && experts <= kMaxExperts ? round256(mxk::route_workspace_bytes(experts)) : 0;
  }
  return 0;
}

// mx_quantize with the workspace given explicitly (a caller's buffer, or the
// static scratch of mx_quantize_noalloc).  launch == false: validate only.
static int quantize_impl(const void* x, int32_t x_dtype, int64_t ld_x, const mx_tensor* out, int32_t flags,
                         void* workspace, size_t workspace_bytes, void* stream, bool launch = true) {
  int st = check_tensor(out);
  if (st) return st;
  if (flags != MX_QUANT_DEFAULT && flags != MX_QUANT_STATIC_GLOBAL && flags != MX_QUANT_SCALE_FLOOR)
    return MX_ERR_UNSUPPORTED;
  if (flags == MX_QUANT_STATIC_GLOBAL && out->fmt != MX_FMT_NVFP4) return MX_ERR_UNSUPPORTED;
  if (flags == MX_QUANT_SCALE_FLOOR && (!fmt_e8m0(out->fmt) || (out->fmt == MX_FMT_MXFP4_K16 && out->global_scale)))
    return MX_ERR_UNSUPPORTED;
  const bool dyn_nv = out->fmt == MX_FMT_NVFP4 && !(flags & MX_QUANT_STATIC_GLOBAL);
  const bool naive = out->fmt == MX_FMT_FP4_TENSOR;
  // rows of whole 32-element blocks run in the vector kernels (either exponent
  // rule); 16-element E8M0 blocks and ragged rows in the per-block kernel
  const bool variant = fmt_e8m0(out->fmt) && (out->fmt == MX_FMT_MXFP4_K16 || out->cols % 32 != 0);
  const bool floor_rule = flags == MX_QUANT_SCALE_FLOOR;
  st = check_dense_input(x, x_dtype, ld_x, out->rows, out->cols, naive || variant);
  if (st) return st;
  if ((dyn_nv || naive) && (!workspace || workspace_bytes < kNvPartialBytes || !al16(workspace)))
    return MX_ERR_WORKSPACE;
  if (out->rows == 0 || out->cols == 0 || !launch) return MX_OK;
  const int bf = x_dtype == MX_DT_BF16;
  hipError_t e;
  if (naive) {
    e = mxk::launch_quant_naive(x, bf, ld_x, out->rows, out->cols, out->codes, out->global_scale,
                                static_cast<uint32_t*>(workspace), (int)(kNvPartialBytes / 4), as_stream(stream));
  } else if (variant) {
    e = mxk::launch_quant_variant(mfma_fmt(out->fmt), block_of(out->fmt), floor_rule,
                                  out->fmt == MX_FMT_MXFP4_K16 ? out->global_scale : nullptr, x, bf, ld_x, out->rows,
                                  out->cols, out->codes, out->scales, as_stream(stream));
  } else if (out->fmt == MX_FMT_MXFP4) {
    e = mxk::launch_quant_mx(x, bf, ld_x, out->rows, out->cols, out->codes, out->scales, as_stream(stream), nullptr, 0,
                             floor_rule);
  } else if (fmt_wide(out->fmt)) {
    e = mxk::launch_quant_wide(mfma_fmt(out->fmt), x, bf, ld_x, out->rows, out->cols, out->codes, out->scales,
                               as_stream(stream), floor_rule);
  } else {
    e = mxk::launch_quant_nv(x, bf, ld_x, out->rows, out->cols, out->codes, out->scales, out->global_scale, !dyn_nv,
                             static_cast<uint32_t*>(workspace), as_stream(stream));
  }
  return hip_status(e);
}

int mx_quantize(const void* x, int32_t x_dtype, int64_t ld_x, const mx_tensor* out, int32_t flags, void* workspace,
                size_t workspace_bytes, void* stream) {
  return quantize_impl(x, x_dtype, ld_x, out, flags, workspace, workspace_bytes, stream);
}

// The same work with the amax partials in the library's static per-device
// scratch array instead of a caller workspace; calls that overlap on one
// device share that array.
int mx_quantize_noalloc(const void* x, int32_t x_dtype, int64_t ld_x, const mx_tensor* out, int32_t flags,
                        void* stream) {
  int st = check_tensor(out);
  if (st) return st;
  const size_t need = mx_workspace_bytes(MX_OP_QUANTIZE, out, flags);
  if (need == 0) return quantize_impl(x, x_dtype, ld_x, out, flags, nullptr, 0, stream);
  if (need > mxk::kNoallocScratchBytes) return MX_ERR_WORKSPACE;   // beyond the static scratch
  // every argument is checked before the first HIP call (an aligned stand-in
  // for the scratch, never dereferenced while only validating)
  st = quantize_impl(x, x_dtype, ld_x, out, flags, reinterpret_cast<void*>(uintptr_t(256)), mxk::kNoallocScratchBytes,
                     stream, false);
  if (st || out->rows == 0 || out->cols == 0) return st;
  void* scratch = nullptr;
  if (mxk::noalloc_scratch(&scratch) != hipSuccess || !scratch) return MX_ERR_HIP;
  return quantize_impl(x, x_dtype, ld_x, out, flags, scratch, mxk::kNoallocScratchBytes, stream);
}

int mx_dequantize(const mx_tensor* in, void* y, int32_t y_dtype, int64_t ld_y, void* stream) {
  int st = check_tensor(in);
  if (st) return st;
  const bool elementwise = in->fmt == MX_FMT_FP4_TENSOR || in->fmt == MX_FMT_MXFP4_K16 ||
                           (fmt_e8m0(in->fmt) && in->cols % 32 != 0);
  st = check_dense_input(y, y_dtype, ld_y, in->rows, in->cols, elementwise);
  if (st) return st;
  if (in->rows == 0 || in->cols == 0) return MX_OK;
  const bool ybf = y_dtype == MX_DT_BF16;
  if (in->fmt == MX_FMT_FP4_TENSOR)
    return hip_status(mxk::launch_dequant_naive(in->codes, in->global_scale, in->rows, in->cols, y, ybf, ld_y,
                                                as_stream(stream)));
  if (in->fmt == MX_FMT_MXFP4_K16 || (fmt_e8m0(in->fmt) && in->cols % 32 != 0))
    return hip_status(mxk::launch_dequant_variant(mfma_fmt(in->fmt), block_of(in->fmt),
                                                  in->fmt == MX_FMT_MXFP4_K16 ? in->global_scale : nullptr,
                                                  in->codes, in->scales, in->rows, in->cols, y, ybf, ld_y,
                                                  as_stream(stream)));
  if (fmt_wide(in->fmt))
    return hip_status(mxk::launch_dequant_wide(mfma_fmt(in->fmt), in->codes, in->scales, in->rows, in->cols, y,
                                               y_dtype == MX_DT_BF16, ld_y, as_stream(stream)));
  return hip_status(mxk::launch_dequant(in->fmt == MX_FMT_NVFP4, in->codes, in->scales, in->global_scale, in->rows,
                                        in->cols, y, y_dtype == MX_DT_BF16, ld_y, as_stream(stream)));
}

int mx_gemm(const mx_gemm_args* a, void* stream) {
  if (!a) return MX_ERR_NULL;
  if (a->flags & ~(MX_GEMM_F8F6F4_MATRIX_CORES | MX_GEMM_FUSED_QUANTIZE | kDynMask)) return MX_ERR_SHAPE;
  if (a->M < 0 || a->N < 0 || a->K < 0 || a->M > kMaxDim || a->N > kMaxDim || a->K > kMaxDim) return MX_ERR_SHAPE;
  if (a->groups < 0) return MX_ERR_SHAPE;
  int st = check_tensor(a->b);
  if (st) return st;
  const int32_t fmt = a->b->fmt;
  if (a->b->cols != a->K) return MX_ERR_SHAPE;
  if (fmt == MX_FMT_MXFP4_K16 || fmt == MX_FMT_FP4_TENSOR) return MX_ERR_UNSUPPORTED;
  if (a->a && (a->a->fmt == MX_FMT_MXFP4_K16 || a->a->fmt == MX_FMT_FP4_TENSOR)) return MX_ERR_UNSUPPORTED;
  if (a->a && (a->flags & kDynMask)) return MX_ERR_FORMAT;   // a format for a dynamic A, but A is given
  // a row length that is not a multiple of 32 is stored zero-padded: the
  // product over the padded length is the same
  const int64_t Kp = fmt == MX_FMT_NVFP4 ? a->K : pad_to(a->K, 32);
  if (a->groups == 0) {
    if (a->b->rows != a->N) return MX_ERR_SHAPE;
  } else {
    if (a->b->rows != (int64_t)a->groups * a->N) return MX_ERR_SHAPE;
    if (!a->group_offsets) return MX_ERR_NULL;
    if (fmt == MX_FMT_NVFP4) return MX_ERR_UNSUPPORTED;
  }
  if (!dtype_ok(a->c_dtype)) return MX_ERR_DTYPE;
  if (a->ldc < a->N) return MX_ERR_SHAPE;
  if (a->M > 0 && a->N > 0) {
    if (!a->c) return MX_ERR_NULL;
    if (!al16(a->c)) return MX_ERR_ALIGN;
  }
  hipStream_t s = as_stream(stream);
  const int cbf = a->c_dtype == MX_DT_BF16;

  // A: pre-quantized, or quantized here (dynamic) into the side outputs or the
  // workspace (after the fused kernel's counters when that kernel runs)
  const int32_t afmt = a->a ? a->a->fmt : dyn_a_fmt(a);
  const uint8_t* a_codes = nullptr;
  const uint8_t* a_scales = nullptr;
  const float* a_global = nullptr;
  bool dynamic = false;
  size_t fused_ws = 0;
  if (a->a) {
    st = check_tensor(a->a);
    if (st) return st;
    if (a->a->rows != a->M || a->a->cols != a->K) return MX_ERR_SHAPE;
    a_codes = a->a->codes; a_scales = a->a->scales; a_global = a->a->global_scale;
  } else {
    if (fmt == MX_FMT_NVFP4) return MX_ERR_UNSUPPORTED;    // dynamic A takes an MX format
    if (!dyn_fmt_ok(afmt)) return MX_ERR_FORMAT;
    if (a->K % 32 != 0) return MX_ERR_UNSUPPORTED;         // ... with whole blocks only
    st = check_dense_input(a->a_raw, a->a_raw_dtype, a->lda_raw, a->M, a->K);
    if (st) return st;
    if (a->M > kMaxElems / (a->K > 0 ? a->K : 1)) return MX_ERR_SHAPE;
    dynamic = true;
    fused_ws = fused_shape(a) ? round256(mxk::fused_workspace_bytes()) : 0;
    if (a->a_codes_out || a->a_scales_out) {
      if (!a->a_codes_out || !a->a_scales_out) return MX_ERR_NULL;
      if (!al16(a->a_codes_out) || !al16(a->a_scales_out)) return MX_ERR_ALIGN;
      a_codes = a->a_codes_out; a_scales = a->a_scales_out;
      if (fused_ws && (!a->workspace || a->workspace_bytes < fused_ws || !al16(a->workspace))) return MX_ERR_WORKSPACE;
    } else if (a->M > 0 && a->K > 0) {
      const size_t need = fused_ws + dyn_a_bytes(afmt, a->M, a->K);
      if (!a->workspace || a->workspace_bytes < need || !al16(a->workspace)) return MX_ERR_WORKSPACE;
      a_codes = static_cast<const uint8_t*>(a->workspace) + fused_ws;
      a_scales = a_codes + round256(dyn_codes_bytes(afmt, a->M, a->K));
    }
  }

  // MX element pairs other than E2M1 x E2M1 (MXFP8 / MXFP6, mixed pairs)
  if (fmt_wide(fmt) || fmt_wide(afmt)) {
    if (afmt == MX_FMT_NVFP4 || fmt == MX_FMT_NVFP4) return MX_ERR_FORMAT;
    if (Kp % 128 != 0 || Kp > (int64_t(1) << 22)) return MX_ERR_UNSUPPORTED;
    if (a->M == 0 || a->N == 0) return MX_OK;
    if (dynamic) {
      const hipError_t e =
          afmt == MX_FMT_MXFP4
              ? mxk::launch_quant_mx(a->a_raw, a->a_raw_dtype == MX_DT_BF16, a->lda_raw, a->M, a->K,
                                     const_cast<uint8_t*>(a_codes), const_cast<uint8_t*>(a_scales), s)
              : mxk::launch_quant_wide(mfma_fmt(afmt), a->a_raw, a->a_raw_dtype == MX_DT_BF16, a->lda_raw, a->M, a->K,
                                       const_cast<uint8_t*>(a_codes), const_cast<uint8_t*>(a_scales), s);
      if (e != hipSuccess) return MX_ERR_HIP;
    }
    return hip_status(mxk::launch_gemm_mxw(mfma_fmt(afmt), mfma_fmt(fmt), a_codes, a_scales, a->b->codes,
                                           a->b->scales, a->c, cbf, a->ldc, a->M, a->N, Kp, a->groups,
                                           a->group_offsets, s, !(a->flags & MX_GEMM_F8F6F4_MATRIX_CORES)));
  }
  if (afmt != fmt) return MX_ERR_FORMAT;
  if (dynamic && fused_ws && a->M > 0 && a->N > 0 && device_cus() == kFusedCUs) {
    if (a->K > (int64_t(1) << 23)) return MX_ERR_UNSUPPORTED;
    return hip_status(mxk::launch_gemm_mx_fused(a->a_raw, a->a_raw_dtype == MX_DT_BF16, a->lda_raw,
                                                const_cast<uint8_t*>(a_codes), const_cast<uint8_t*>(a_scales),
                                                a->b->codes, a->b->scales, a->c, cbf, a->ldc, a->M, a->N, a->K,
                                                a->groups, a->group_offsets, a->workspace, kFusedCUs / 8, s));
  }
  if (fmt == MX_FMT_NVFP4 && a->K % 32 != 0) return MX_ERR_UNSUPPORTED;
  if (a->K > (int64_t(1) << 23)) return MX_ERR_UNSUPPORTED;   // tile byte offsets stay below 2^30
  if (a->M == 0 || a->N == 0) return MX_OK;
  if (dynamic && a->K > 0) {
    hipError_t e = mxk::launch_quant_mx(a->a_raw, a->a_raw_dtype == MX_DT_BF16, a->lda_raw, a->M, a->K,
                                        const_cast<uint8_t*>(a_codes), const_cast<uint8_t*>(a_scales), s);
    if (e != hipSuccess) return MX_ERR_HIP;
  }
  // split partials after what the workspace already holds (none: no split)
  const size_t off = fused_ws + round256(a->a_codes_out ? 0 : ws_a_bytes(a));
  float* part = nullptr;
  size_t part_bytes = 0;
  if (a->workspace && al16(a->workspace) && a->workspace_bytes > off && split_bytes(a) > 0) {
    part = reinterpret_cast<float*>(static_cast<uint8_t*>(a->workspace) + off);
    part_bytes = a->workspace_bytes - off;
  }
  if (fmt == MX_FMT_MXFP4)
    return hip_status(mxk::launch_gemm_mx(a_codes, a_scales, a->b->codes, a->b->scales, a->c, cbf, a->ldc, a->M, a->N,
                                          Kp, a->groups, a->group_offsets, s, part, part_bytes, device_cus()));
  return hip_status(mxk::launch_gemm_nv(a_codes, a_scales, a_global, a->b->codes, a->b->scales, a->b->global_scale,
                                        a->c, cbf, a->ldc, a->M, a->N, a->K, s, part, part_bytes, device_cus()));
}

int mx_moe_route(const int32_t* topk_ids, int64_t tokens, int32_t topk, int32_t experts, int32_t* offsets,
                 int32_t* dest_row, int32_t* src_token, void* workspace, size_t workspace_bytes, void* stream) {
  if (tokens < 0 || topk < 1 || experts < 1 || experts > kMaxExperts) return MX_ERR_SHAPE;
  if (tokens > kMaxPairs / topk) return MX_ERR_SHAPE;
  const int64_t npairs = tokens * topk;
  if (!offsets) return MX_ERR_NULL;
  if (npairs > 0 && (!topk_ids || !dest_row || !src_token)) return MX_ERR_NULL;
  if (!al4(offsets) || (npairs > 0 && (!al4(topk_ids) || !al4(dest_row) || !al4(src_token)))) return MX_ERR_ALIGN;
  if (!workspace || workspace_bytes < mxk::route_workspace_bytes(experts) || !al4(workspace)) return MX_ERR_WORKSPACE;
  return hip_status(mxk::launch_moe_route(topk_ids, npairs, topk, experts, offsets, dest_row, src_token,
                                          static_cast<int32_t*>(workspace), as_stream(stream)));
}

int mx_quantize_rows(const void* x, int32_t x_dtype, int64_t ld_x, int64_t x_rows, const int32_t* row_index,
                     const mx_tensor* out, void* stream) {
  int st = check_tensor(out);
  if (st) return st;
  if (out->fmt != MX_FMT_MXFP4 || out->cols % 32 != 0) return MX_ERR_UNSUPPORTED;
  if (x_rows < 0) return MX_ERR_SHAPE;
  st = check_dense_input(x, x_dtype, ld_x, x_rows, out->cols);
  if (st) return st;
  if (out->rows == 0 || out->cols == 0) return MX_OK;
  if (!row_index) return MX_ERR_NULL;
  if (!al4(row_index)) return MX_ERR_ALIGN;
  if (x_rows > 0 && !x) return MX_ERR_NULL;
  return hip_status(mxk::launch_quant_mx(x, x_dtype == MX_DT_BF16, ld_x, out->rows, out->cols, out->codes, out->scales,
                                         as_stream(stream), row_index, x_rows));
}

int mx_moe_combine(const void* y, int32_t y_dtype, int64_t ld_y, int64_t y_rows, const int32_t* dest_row,
                   const float* weights, int64_t tokens, int32_t topk, int64_t N, void* out, int32_t out_dtype,
                   int64_t ld_out, void* stream) {
  if (tokens < 0 || topk < 1 || N < 0 || y_rows < 0 || N > kMaxDim) return MX_ERR_SHAPE;
  if (tokens > kMaxPairs / topk) return MX_ERR_SHAPE;
  if (N % 8 != 0) return MX_ERR_UNSUPPORTED;
  int st = check_dense_input(y, y_dtype, ld_y, y_rows, N);
  if (st) return st;
  st = check_dense_input(out, out_dtype, ld_out, tokens, N);
  if (st) return st;
  if (tokens == 0 || N == 0) return MX_OK;
  if (!dest_row || !weights) return MX_ERR_NULL;
  if (!al4(dest_row) || !al4(weights)) return MX_ERR_ALIGN;
  return hip_status(mxk::launch_moe_combine(y, y_dtype == MX_DT_BF16, ld_y, y_rows, dest_row, weights, tokens, topk, N,
                                            out, out_dtype == MX_DT_BF16, ld_out, as_stream(stream)));
}

int mx_rmsnorm_quantize(const void* x, int32_t x_dtype, int64_t ld_x, const void* gamma, int32_t gamma_dtype,
                        float eps, const mx_tensor* out, int32_t flags, void* stream) {
  int st = check_tensor(out);
  if (st) return st;
  if (x_dtype != MX_DT_BF16 || !dtype_ok(gamma_dtype)) return MX_ERR_DTYPE;
  if (!(eps > 0.0f) || eps > 3.0e38f) return MX_ERR_SHAPE;   // eps > 0 keeps an all-zero row finite
  if (out->fmt != MX_FMT_MXFP4 && out->fmt != MX_FMT_NVFP4) return MX_ERR_UNSUPPORTED;
  if (out->fmt == MX_FMT_MXFP4 && flags != MX_QUANT_DEFAULT) return MX_ERR_UNSUPPORTED;
  if (out->fmt == MX_FMT_NVFP4 && flags != MX_QUANT_STATIC_GLOBAL) return MX_ERR_UNSUPPORTED;
  if (out->cols % 32 != 0 || out->cols > kMaxNormCols) return MX_ERR_UNSUPPORTED;
  st = check_dense_input(x, x_dtype, ld_x, out->rows, out->cols);
  if (st) return st;
  if (out->rows == 0 || out->cols == 0) return MX_OK;
  if (!gamma) return MX_ERR_NULL;
  if (!al16(gamma)) return MX_ERR_ALIGN;
  return hip_status(mxk::launch_rmsnorm_quant(x, ld_x, out->rows, out->cols, gamma, gamma_dtype == MX_DT_BF16, eps,
                                              out->fmt == MX_FMT_NVFP4, out->codes, out->scales, out->global_scale,
                                              as_stream(stream)));
}

int mx_gemv(const void* x, int32_t x_dtype, int64_t M, int64_t ld_x, const mx_tensor* w, void* y, int32_t y_dtype,
            int64_t ld_y, void* stream) {
  int st = check_tensor(w);
  if (st) return st;
  if (x_dtype != MX_DT_BF16 || y_dtype != MX_DT_BF16) return MX_ERR_DTYPE;
  if ((w->fmt != MX_FMT_MXFP4 && !fmt_wide(w->fmt)) || w->cols % 32 != 0) return MX_ERR_UNSUPPORTED;
  if (M < 0) return MX_ERR_SHAPE;
  if (M > 16) return MX_ERR_UNSUPPORTED;
  const int64_t N = w->rows, K = w->cols;
  if (ld_y < N) return MX_ERR_SHAPE;
  st = check_dense_input(x, x_dtype, ld_x, M, K);
  if (st) return st;
  if (M == 0 || N == 0) return MX_OK;
  if (!y) return MX_ERR_NULL;
  if (!al16(y)) return MX_ERR_ALIGN;
  return hip_status(mxk::launch_gemv(mfma_fmt(w->fmt), x, ld_x, M, w->codes, w->scales, N, K, y, ld_y, as_stream(stream)));
}

}  // extern "C"
#pragma GCC visibility pop
