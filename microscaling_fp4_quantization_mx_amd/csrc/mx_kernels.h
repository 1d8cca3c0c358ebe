// Host-side launchers of the gfx950 kernels (internal to libmx).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {
// Static per-device scratch of the allocation-free entry points (noalloc.hip):
// *ptr receives the current device's address of the array (looked up once per
// device); it holds kNoallocScratchBytes bytes.
constexpr size_t kNoallocScratchBytes = 16384;
hipError_t noalloc_scratch(void** ptr);
// gidx != nullptr: output row r quantizes input row gidx[r] (zero row if the
// index is outside [0, x_rows)).
hipError_t launch_quant_mx(const void* x, int xdt_bf16, int64_t ldx, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, hipStream_t st, const int32_t* gidx = nullptr, int64_t x_rows = 0,
                           bool floor_rule = false);
int nv_partials_count(int64_t rows, int64_t cols, int xdt_bf16);
hipError_t launch_quant_nv(const void* x, int xdt_bf16, int64_t ldx, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, float* gscale, bool static_global, uint32_t* partial, hipStream_t st);
hipError_t launch_dequant(bool nv, const uint8_t* codes, const uint8_t* scales, const float* gscale, int64_t rows,
                          int64_t cols, void* y, bool out_bf16, int64_t ldy, hipStream_t st);
// part / part_bytes: device scratch for the K parts of a last round that
// would leave CUs idle (at least gemm_mx_split_bytes; else no split); cus:
// the device's CU count.
hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, void* c, int c_bf16, int64_t ldc, int64_t M, int64_t N, int64_t K,
                          int groups, const int32_t* offsets, hipStream_t st, float* part = nullptr,
                          size_t part_bytes = 0, int cus = 0);
size_t gemm_mx_split_bytes(int64_t M, int64_t N, int64_t K, int groups, int cus);
// Dynamic MXFP4 quantization fused with the (grouped) GEMM (gemm_fused.hip):
// one persistent launch (after a one-workgroup counter reset) for K % 512 == 0
// on a 256-CU device; the workspace holds fused_workspace_bytes() of counters
// and split partial tiles.
bool fused_fits(int64_t M, int64_t N, int64_t K, int groups, int wpl);
size_t fused_workspace_bytes();
hipError_t launch_gemm_mx_fused(const void* x, int x_bf16, int64_t ldx, uint8_t* a_codes, uint8_t* a_scales,
                                const uint8_t* b_codes, const uint8_t* b_scales, void* c, int c_bf16, int64_t ldc,
                                int64_t M, int64_t N, int64_t K, int groups, const int32_t* offsets, void* ws,
                                int wpl, hipStream_t st);
// part / part_bytes / cus: as for launch_gemm_mx (K % 256 == 0 only).
hipError_t launch_gemm_nv(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                          const uint8_t* b_codes, const uint8_t* b_scales, const float* b_global, void* c, int c_bf16,
                          int64_t ldc, int64_t M, int64_t N, int64_t K, hipStream_t st, float* part = nullptr,
                          size_t part_bytes = 0, int cus = 0);
size_t gemm_nv_split_bytes(int64_t M, int64_t N, int64_t K, int cus);
// Wider MX elements; fmt is the block-scaled MFMA's element code (E4M3 0,
// E5M2 1, E2M3 2, E3M2 3; the GEMM also takes E2M1 4).
hipError_t launch_quant_wide(int fmt, const void* x, int xdt_bf16, int64_t ldx, int64_t rows, int64_t cols,
                             uint8_t* codes, uint8_t* scales, hipStream_t st, bool floor_rule = false);
hipError_t launch_dequant_wide(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, void* y,
                               bool out_bf16, int64_t ldy, hipStream_t st);
// exact: codes expanded to exact bf16 values for the bf16 matrix cores;
// otherwise the block-scaled FP8/FP6/FP4 matrix cores (faster; they truncate
// products with FP8 or FP6 operands).
// groups / offsets: the grouped form, as for launch_gemm_mx (0: dense).
hipError_t launch_gemm_mxw(int fa, int fb, const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                           const uint8_t* b_scales, void* c, int c_bf16, int64_t ldc, int64_t M, int64_t N, int64_t K,
                           int groups, const int32_t* offsets, hipStream_t st, bool exact);
// Emulation variants (quantize_variant.hip): block 16 or 32, the OCP floor
// rule, a per-tensor scale g (NULL = 1), rows of any length (zero-padded to
// whole blocks); naive per-tensor FP4.
hipError_t launch_quant_variant(int fmt, int block, bool floor_rule, const float* g, const void* x, int xdt_bf16,
                                int64_t ldx, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                hipStream_t st);
hipError_t launch_dequant_variant(int fmt, int block, const float* g, const uint8_t* codes, const uint8_t* scales,
                                  int64_t rows, int64_t cols, void* y, bool out_bf16, int64_t ldy, hipStream_t st);
hipError_t launch_quant_naive(const void* x, int xdt_bf16, int64_t ldx, int64_t rows, int64_t cols, uint8_t* codes,
                              float* s, uint32_t* partial, int max_partials, hipStream_t st);
hipError_t launch_dequant_naive(const uint8_t* codes, const float* s, int64_t rows, int64_t cols, void* y, bool out_bf16,
                                int64_t ldy, hipStream_t st);
// fmt: the weights' element format as the matrix-core code above (E2M1 4).
hipError_t launch_gemv(int fmt, const void* x, int64_t ldx, int64_t M, const uint8_t* wc, const uint8_t* ws, int64_t N,
                       int64_t K, void* y, int64_t ldy, hipStream_t st);
// ws: route_workspace_bytes(experts) bytes (per-chunk counts)
size_t route_workspace_bytes(int experts);
hipError_t launch_moe_route(const int32_t* ids, int64_t npairs, int topk, int experts, int32_t* offsets,
                            int32_t* dest_row, int32_t* src_token, int32_t* ws, hipStream_t st);
hipError_t launch_moe_combine(const void* y, int y_bf16, int64_t ldy, int64_t y_rows, const int32_t* dest_row,
                              const float* w, int64_t tokens, int topk, int64_t N, void* out, int o_bf16, int64_t ldo,
                              hipStream_t st);
hipError_t launch_rmsnorm_quant(const void* x, int64_t ldx, int64_t rows, int64_t K, const void* gamma, int g_bf16,
                                float eps, bool nv, uint8_t* codes, uint8_t* scales, const float* gscale,
                                hipStream_t st);
}  // namespace mxk
