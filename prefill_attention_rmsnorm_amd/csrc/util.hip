// Small utility kernels: workspace clearing (a fill kernel, so that callers
// capturing HIP graphs get no memset nodes) and a plain copy used to
// calibrate bandwidth and HBM-traffic counters.
#include "qa_device.h"

namespace qa {

__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4* p, size_t n16) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * 256)
    p[i] = z;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst,
                                                   size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * 256)
    dst[i] = __builtin_nontemporal_load(src + i);
}

static unsigned grid_for(size_t n16) {
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  return blocks ? (unsigned)blocks : 1u;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n16)), dim3(256), 0, s,
                     static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n16)), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace qa
