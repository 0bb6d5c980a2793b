// e4m3 (OCP FP8) quantisation and packing for the fp8 configuration.
//
// The model card quotes its speed on H100 in FP8 and gives no scheme; the reading taken here:
// every row (an output channel of a weight matrix, or one token's activations) gets the scale
// s = amax / 448, and its elements become e4m3(x / s), nearest-even with saturation, both
// decided in binary32; products accumulate in fp32 and are multiplied by both scales.
//   quant_rows  one workgroup per row: amax, scale, codes (row-major, natural layout)
//   pack_fp8    e4m3 codes into the fragment-major layout of the fp8 expert kernels: a 16-row x
//               64-k block is 1 KiB, lane l holds row l%16, k = 16 (l/16) .. 16 (l/16) + 15
#include "dg_internal.h"

namespace dg {
namespace {

template <bool F32>
__device__ __forceinline__ float4 load4(const void* src, long long off) {
  if constexpr (F32) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(src) + off);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + off);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
  }
}

template <bool F32>
__global__ __launch_bounds__(256) void k_quant_rows(const void* src, long long ld_src,
                                                    uint8_t* codes, long long ld_codes,
                                                    float* scales, long long rows_a, int cols_a,
                                                    int cols_b) {
  __shared__ float red[4];
  const long long r = blockIdx.x;
  const int cols = r < rows_a ? cols_a : cols_b;
  const long long base = r * ld_src;
  float amax = 0.f;
  for (int c = threadIdx.x * 4; c < cols; c += 1024) {
    const float4 v = load4<F32>(src, base + c);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  uint8_t* o = codes + r * ld_codes;
  for (int c = threadIdx.x * 4; c < cols; c += 1024) {
    const float4 v = load4<F32>(src, base + c);
    *reinterpret_cast<uint32_t*>(o + c) = f2e4m3(v.x / sc) | (f2e4m3(v.y / sc) << 8) |
                                          (f2e4m3(v.z / sc) << 16) | (f2e4m3(v.w / sc) << 24);
  }
  if (threadIdx.x == 0) scales[r] = sc;
}

// element (n, k) of a [rows][cols] code matrix goes to
// ((n/16 * cols/64 + k/64) * 64 + (k%64)/16 * 16 + n%16) * 16 + k%16
__global__ __launch_bounds__(256) void k_pack_fp8(const uint8_t* src, uint8_t* dst,
                                                  long long rows, long long cols) {
  const long long frags = (rows / 16) * (cols / 64);
  const long long i = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (i >= frags) return;
  const int lane = threadIdx.x & 63;
  const long long rt = i / (cols / 64), s = i % (cols / 64);
  const long long n = rt * 16 + (lane & 15), k = s * 64 + (lane >> 4) * 16;
  st16(dst + i * 1024 + lane * 16, ld16(src + n * cols + k));
}

}  // namespace

hipError_t launch_quant_rows(const void* src, bool src_f32, long long ld_src, uint8_t* codes,
                             long long ld_codes, float* scales, long long rows, long long rows_a,
                             int cols_a, int cols_b, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (src_f32)
    hipLaunchKernelGGL(k_quant_rows<true>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s, src,
                       ld_src, codes, ld_codes, scales, rows_a, cols_a, cols_b);
  else
    hipLaunchKernelGGL(k_quant_rows<false>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s,
                       src, ld_src, codes, ld_codes, scales, rows_a, cols_a, cols_b);
  return hipGetLastError();
}

hipError_t launch_pack_fp8(const void* src, void* dst, long long rows, long long cols,
                           hipStream_t s) {
  const long long frags = (rows / 16) * (cols / 64);
  if (frags == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_fp8, dim3(static_cast<unsigned>((frags + 3) / 4)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), rows, cols);
  return hipGetLastError();
}

}  // namespace dg
