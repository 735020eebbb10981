// Small utility kernels.
#include "launch.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16, uint8_t* tail,
                                                        size_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

// Zero `bytes` bytes at 16-byte aligned `p` with a kernel (no memset node under capture).
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  size_t grid = (n16 + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid == 0) grid = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(p), n16, reinterpret_cast<uint8_t*>(p) + n16 * 16,
                     ntail);
  return hipGetLastError();
}

}  // namespace moe
