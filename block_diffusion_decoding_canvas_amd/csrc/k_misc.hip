// Bandwidth and throughput yardsticks: a plain device copy (the byte-counter calibration, and a
// read + write stream), a read-only stream (the XOR of every 32-bit word, so that the result can
// be checked) and a bf16 MFMA loop (the matrix-core rate the chip sustains).
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kCopyBatch = 8;   // 16-byte loads in flight per thread in the copy

// the copy: block b sweeps its contiguous range of pieces [b * per, (b + 1) * per) with
// consecutive threads on consecutive 16-byte pieces, kCopyBatch loads issued before their
// stores in each round, the tail one piece at a time
__global__ __launch_bounds__(256) void k_copy(u32x4* __restrict__ dst,
                                              const u32x4* __restrict__ src, size_t n16) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = min(n16, static_cast<size_t>(blockIdx.x) * per);
  const size_t end = min(n16, beg + per);
  const size_t step = blockDim.x;
  size_t i = beg + threadIdx.x;
  for (; i + (kCopyBatch - 1) * step < end; i += kCopyBatch * step) {
    u32x4 v[kCopyBatch];
#pragma unroll
    for (int j = 0; j < kCopyBatch; ++j) v[j] = src[i + j * step];
#pragma unroll
    for (int j = 0; j < kCopyBatch; ++j) dst[i + j * step] = v[j];
  }
  for (; i < end; i += step) dst[i] = src[i];
}

// the read stream: grid-stride with one streaming (nontemporal) 16-byte load per thread per
// iteration; measured here, this plain form reads faster than per-wave contiguous sweeps or
// several loads per thread in flight.  Each block leaves the XOR of its words in its own slot of
// g_read_part, and one small block combines the slots: one atomic per block on a single word
// had added ~50 us of serialised atomics to every call, which held the measured rate ~10% under
// the kernels it is meant to bound.
constexpr int kReadBlocks = 256 * 16;
__device__ uint32_t g_read_part[kReadBlocks];

__global__ __launch_bounds__(256) void k_read_stream(const u32x4* __restrict__ src, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  uint32_t x = 0;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[4];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) g_read_part[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// XOR of the first nblk block slots (0 when there are none) into *out
__global__ __launch_bounds__(256) void k_read_combine(int nblk, uint32_t* out) {
  uint32_t x = 0;
  for (int i = threadIdx.x; i < nblk; i += blockDim.x) x ^= g_read_part[i];
  __shared__ uint32_t red[4];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) *out = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// every wave runs `iters` rounds of kChains independent 16x16x32 bf16 MFMAs (operands from the
// lane id, so nothing folds away) and writes one sum per lane.  The MFMAs are written as
// instructions on the accumulators in place: through the builtin the compiler copies the
// accumulators between register files every round, which measures the copies instead.  A
// chain's next MFMA follows kChains - 1 others; after the loop, explicit wait states cover the
// last MFMAs' results before ordinary instructions read them
constexpr int kChains = 8;
__global__ __launch_bounds__(256) void k_mfma_loop(int iters, float* out) {
  const uint32_t l = threadIdx.x & 63;
  const u32x4 a = {0x3f803f80u ^ l, 0x3f003f00u, 0x3e803e80u, 0x3f803f80u};
  const u32x4 b = {0x3f803f80u, 0x3f803f80u ^ (l << 1), 0x3f003f00u, 0x3e803e80u};
  f32x4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[c]) : "v"(a), "v"(b));
  }
  asm volatile("s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7" ::);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_copy(void* dst, const void* src, size_t n, hipStream_t s) {
  const size_t n16 = n / 16;
  if (n16 == 0) return hipSuccess;
  const size_t want = (n16 + 255) / 256;
  const unsigned grid = static_cast<unsigned>(std::min<size_t>(want, 256 * 8));
  hipLaunchKernelGGL(k_copy, dim3(grid), dim3(256), 0, s, static_cast<u32x4*>(dst),
                     static_cast<const u32x4*>(src), n16);
  return hipGetLastError();
}

hipError_t launch_read_stream(const void* src, size_t n, uint32_t* out, hipStream_t s) {
  const size_t n16 = n / 16;
  const size_t want = (n16 + 255) / 256;
  const int grid = static_cast<int>(std::min<size_t>(want, kReadBlocks));
  if (grid > 0)
    hipLaunchKernelGGL(k_read_stream, dim3(grid), dim3(256), 0, s, static_cast<const u32x4*>(src),
                       n16);
  hipLaunchKernelGGL(k_read_combine, dim3(1), dim3(256), 0, s, grid, out);
  return hipGetLastError();
}

int mfma_loop_blocks() { return 512; }   // 2 waves per SIMD on 256 CUs

hipError_t launch_mfma_loop(int iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_loop, dim3(mfma_loop_blocks()), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace dg
