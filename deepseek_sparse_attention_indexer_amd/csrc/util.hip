// Small utility kernels of the DSA library.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

// Zero a buffer with plain vector stores (used instead of a memset node so that callers may
// capture the initialisation in a HIP graph).
__global__ __launch_bounds__(256) void k_fill_zero(uint8_t* p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t tid = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  u32x4_t* q = reinterpret_cast<u32x4_t*>(p);
  for (size_t i = tid; i < n16; i += stride) q[i] = u32x4_t{0u, 0u, 0u, 0u};
  for (size_t i = n16 * 16 + tid; i < bytes; i += stride) p[i] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const size_t blocks = (bytes / 16 + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 4096 ? (blocks ? blocks : 1) : 4096);
  launch_kernel(k_fill_zero, dim3(grid), dim3(256), st, static_cast<uint8_t*>(p), bytes);
  return hipGetLastError();
}

}  // namespace dsa
