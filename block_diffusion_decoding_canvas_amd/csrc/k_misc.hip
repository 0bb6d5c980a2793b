// Bandwidth and throughput yardsticks: a plain device copy (the byte-counter calibration, and a
// read + write stream), a read-only stream (the XOR of every 32-bit word, so that the result can
// be checked) and a bf16 MFMA loop (the matrix-core rate the chip sustains).
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kStreamBatch = 8;   // 16-byte loads in flight per thread

// wave w of the grid sweeps its own contiguous range of pieces [w * per, (w + 1) * per), its
// lanes on consecutive 16-byte pieces (one load instruction reads 1 KiB contiguous); in each
// round a lane issues kStreamBatch streaming (nontemporal) loads before it uses any of them, and
// the tail runs one piece at a time.  Per-wave streams are the pattern that reaches the highest
// read rate here
struct Sweep {
  size_t beg, end;
  __device__ Sweep(size_t n16) {
    const size_t waves = static_cast<size_t>(gridDim.x) * (blockDim.x >> 6);
    const size_t wv = static_cast<size_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const size_t per = (n16 + waves - 1) / waves;
    beg = min(n16, wv * per);
    end = min(n16, beg + per);
  }
};

__global__ __launch_bounds__(256) void k_copy(u32x4* __restrict__ dst,
                                              const u32x4* __restrict__ src, size_t n16) {
  const Sweep w(n16);
  const size_t step = 64;
  size_t i = w.beg + (threadIdx.x & 63);
  for (; i + (kStreamBatch - 1) * step < w.end; i += kStreamBatch * step) {
    u32x4 v[kStreamBatch];
#pragma unroll
    for (int j = 0; j < kStreamBatch; ++j) v[j] = __builtin_nontemporal_load(src + i + j * step);
#pragma unroll
    for (int j = 0; j < kStreamBatch; ++j) dst[i + j * step] = v[j];
  }
  for (; i < w.end; i += step) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void k_read_stream(const u32x4* __restrict__ src, size_t n16,
                                                     uint32_t* out) {
  const Sweep w(n16);
  const size_t step = 64;
  size_t i = w.beg + (threadIdx.x & 63);
  uint32_t x = 0;
  for (; i + (kStreamBatch - 1) * step < w.end; i += kStreamBatch * step) {
    u32x4 v[kStreamBatch];
#pragma unroll
    for (int j = 0; j < kStreamBatch; ++j) v[j] = __builtin_nontemporal_load(src + i + j * step);
#pragma unroll
    for (int j = 0; j < kStreamBatch; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < w.end; i += step) {
    const u32x4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[4];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  // one atomic per block (XOR is order-independent, so the result is deterministic)
  if (threadIdx.x == 0) atomicXor(out, red[0] ^ red[1] ^ red[2] ^ red[3]);
}

__global__ void k_zero_word(uint32_t* p) { *p = 0u; }

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
  hipLaunchKernelGGL(k_zero_word, dim3(1), dim3(1), 0, s, out);
  const size_t n16 = n / 16;
  if (n16 == 0) return hipGetLastError();
  const size_t want = (n16 + 255) / 256;
  const unsigned grid = static_cast<unsigned>(std::min<size_t>(want, 256 * 8));
  hipLaunchKernelGGL(k_read_stream, dim3(grid), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), n16, out);
  return hipGetLastError();
}

int mfma_loop_blocks() { return 512; }   // 2 waves per SIMD on 256 CUs

hipError_t launch_mfma_loop(int iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_loop, dim3(mfma_loop_blocks()), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace dg
