// Practical memory ceilings for the benchmark (not part of libmx): a plain
// streaming read and a plain copy of a device buffer, each 16 bytes per lane
// per load with several loads in flight, so that the rates the quantize and
// GEMV kernels reach can be set beside what the same number of bytes costs
// with no arithmetic at all.
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

}  // extern "C"
