// Practical ceilings for the benchmark (not part of libmx): a plain streaming
// read and a plain copy of a device buffer, each 16 bytes per lane per load
// with several loads in flight, so that the rates the quantize and GEMV
// kernels reach can be set beside what the same number of bytes costs with no
// arithmetic at all; and the two on-chip rates the MXFP4 GEMM's K loop lives
// on: the FP4 matrix-core rate with operands in registers, and the LDS read
// rate of 16-byte fragment reads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int CT = 256;   // threads per workgroup
constexpr int CU_ = 4;    // 16-byte vectors per lane per iteration

// Reads n16 16-byte vectors; every workgroup writes the XOR of what it read
// to sink[blockIdx.x] (so the loads cannot be dropped).
__global__ __launch_bounds__(CT) void k_read(const u32x4* __restrict__ p, uint64_t n16, uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[CT / 64];
  uint32_t acc = 0;
  const uint64_t stride = (uint64_t)gridDim.x * CT * CU_;
  for (uint64_t base = (uint64_t)blockIdx.x * CT * CU_ + threadIdx.x; base < n16; base += stride) {
    u32x4 v[CU_];
#pragma unroll
    for (int u = 0; u < CU_; ++u) {
      const uint64_t i = base + (uint64_t)u * CT;
      v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < CU_; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(CT) void k_copy(const u32x4* __restrict__ s, u32x4* __restrict__ d, uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * CT * CU_;
  for (uint64_t base = (uint64_t)blockIdx.x * CT * CU_ + threadIdx.x; base < n16; base += stride) {
    u32x4 v[CU_];
#pragma unroll
    for (int u = 0; u < CU_; ++u) {
      const uint64_t i = base + (uint64_t)u * CT;
      v[u] = i < n16 ? __builtin_nontemporal_load(s + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < CU_; ++u) {
      const uint64_t i = base + (uint64_t)u * CT;
      if (i < n16) __builtin_nontemporal_store(v[u], d + i);
    }
  }
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int MCH = 4;   // independent accumulators per wave

// Register-only FP4 matrix-core loop: every wave issues iters x MCH
// v_mfma_scale_f32_32x32x64_f8f6f4 on operands that stay in registers (E2M1
// codes of 1.0 and 0.5, block scale 2^-8 so the sums stay small); the sums go
// to sink so nothing is dropped.
__global__ __launch_bounds__(CT) void k_mfma(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = i < 4 ? 0x22222222 ^ (lane & 1) : 0;   // 1.0 (and one 0.5) per byte pair
    b[i] = i < 4 ? 0x11111111 : 0;                // 0.5
  }
  f32x16 acc[MCH];
#pragma unroll
  for (int c = 0; c < MCH; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < MCH; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 4, 4, 0, 119, 0, 127);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < MCH; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * CT + threadIdx.x] = s;
}

// LDS read rate: each wave reads 8 x 1 KiB per iteration with ds_read_b128
// (lane l reads bytes 16 l .. 16 l + 15 of a 1 KiB row: no bank conflicts)
// from a 64 KiB array, one workgroup per CU; the XOR of what was read goes
// to sink.
constexpr int LNR = 8;
__global__ __launch_bounds__(CT) void k_lds(uint32_t* __restrict__ sink, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[16384];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 16384; i += CT) lds[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  u32x4 x = {0, 0, 0, 0};
  const int base = (wave * 16 + lane) * 16;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < LNR; ++r)
      x ^= *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(lds) + ((base + r * 1024 + it * 8192) & 65535));
  }
  sink[blockIdx.x * CT + tid] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

}  // namespace

extern "C" {

// Workgroups of the read kernel for `bytes` with `per_cu` workgroups per CU
// (256 CUs), at least 1; the sink needs that many uint32.
__attribute__((visibility("default"))) int mxc_read_grid(uint64_t bytes, int per_cu) {
  const uint64_t n16 = bytes / 16;
  uint64_t g = (n16 + CT * CU_ - 1) / (CT * CU_);
  const uint64_t cap = 256ull * (per_cu > 0 ? per_cu : 1);
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

// Streaming read of `bytes` (a multiple of 16, 16-byte aligned) at p.
__attribute__((visibility("default"))) int mxc_read(const void* p, uint64_t bytes, uint32_t* sink, int per_cu,
                                                    void* stream) {
  if (!p || !sink || (bytes & 15) || ((uintptr_t)p & 15)) return -1;
  const int grid = mxc_read_grid(bytes, per_cu);
  hipLaunchKernelGGL(k_read, dim3(grid), dim3(CT), 0, (hipStream_t)stream, (const u32x4*)p, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Copy of `bytes` (a multiple of 16, both pointers 16-byte aligned).
__attribute__((visibility("default"))) int mxc_copy(const void* src, void* dst, uint64_t bytes, int per_cu,
                                                    void* stream) {
  if (!src || !dst || (bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return -1;
  const int grid = mxc_read_grid(bytes, per_cu);
  hipLaunchKernelGGL(k_copy, dim3(grid), dim3(CT), 0, (hipStream_t)stream, (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Register-only FP4 MFMA loop: `grid` workgroups of 4 waves (512 = two
// waves per SIMD on 256 CUs), iters x 4 MFMAs of 32x32x64 (131072 flops)
// per wave; sink holds grid x 256 floats.
__attribute__((visibility("default"))) int mxc_mfma(float* sink, int grid, int iters, void* stream) {
  if (!sink || grid < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(k_mfma, dim3(grid), dim3(CT), 0, (hipStream_t)stream, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// LDS reads: `grid` workgroups (one per CU with 64 KiB of LDS each), iters x 8
// KiB per wave; sink holds grid x 256 uint32.
__attribute__((visibility("default"))) int mxc_lds(uint32_t* sink, int grid, int iters, void* stream) {
  if (!sink || grid < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(k_lds, dim3(grid), dim3(CT), 0, (hipStream_t)stream, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
