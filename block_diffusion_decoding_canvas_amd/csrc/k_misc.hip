// Small bandwidth kernels: a plain device copy used to calibrate byte counters.
#include "dg_internal.h"

namespace dg {
namespace {

__global__ __launch_bounds__(256) void k_copy(uint4* __restrict__ dst,
                                              const uint4* __restrict__ src, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += stride)
    dst[i] = src[i];
}

}  // namespace

hipError_t launch_copy(void* dst, const void* src, size_t n, hipStream_t s) {
  const size_t n16 = n / 16;
  if (n16 == 0) return hipSuccess;
  const size_t want = (n16 + 255) / 256;
  const unsigned grid = static_cast<unsigned>(std::min<size_t>(want, 256 * 32));
  hipLaunchKernelGGL(k_copy, dim3(grid), dim3(256), 0, s, static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), n16);
  return hipGetLastError();
}

}  // namespace dg
