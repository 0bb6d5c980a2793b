// Router projection of the MoE: fp32 k-split partials of r = u W_r^T on MFMA.
//
// The router matrix [E, d] is small (0.72 MB at 128 x 2816), so this product is latency-bound,
// not bandwidth-bound.  Each wave works alone on 16 expert rows: weight and token fragments go
// straight from memory into a P-stage register ring (no LDS, no barrier), chunk c is consumed
// while chunks c+1 .. c+P-1 are in flight, and one v_mfma_f32_16x16x32_bf16 takes 16 experts x
// 32 k (A = weights) against 16 tokens x 32 k (B = tokens).  A tile is NTB*16 token rows by one
// 64-expert block and one k-split; split s writes its fp32 partial plane, and the top-k kernel
// sums the planes in split order, so the logits are deterministic.
//
// k-order inside an MFMA: lane group g (= lane / 16) supplies 8 consecutive k of its slice per
// MFMA; A and B use the same assignment, so every dot product is the exact sum over the chunk
// whatever order the hardware adds in.
#include "dg_internal.h"

namespace dg {
namespace {

// streaming (non-temporal) 16-byte load: the router weights are read once per layer and step
__device__ __forceinline__ u32x4 load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

constexpr int kWaves = 4;
constexpr int kRows = kWaves * 16;   // expert rows per workgroup

// out[ks][r][n] = sum over k in split ks of X[r][k] W[n][k]; NTB*16 token rows per tile
template <int NTB, int P>
__global__ __launch_bounds__(256) void k_sgemm(WGemmArgs a) {
  constexpr int TR = NTB * 16;
  constexpr int KC = 128;
  const int slot = xcd_remap(blockIdx.x, gridDim.x);
  const int nb = slot % a.n_nblk;
  const int tk = slot / a.n_nblk;
  const int ks = tk % a.ksplit;
  const int tile = tk / a.ksplit;
  if (tile >= a.grid_tiles) return;
  const int row0 = tile * TR;
  const int nrows = min(TR, a.ntok - row0);
  const int N = a.N, K = a.K;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = nb * kRows + wave * 16;
  if (n0 >= N) return;  // waves are independent: no barrier follows
  // an empty k-range still writes its (zero) partial plane
  const int k_beg = min(K, ks * a.k_per_split);
  const int k_end = min(K, k_beg + a.k_per_split);

  // weight rows past N repeat the last one (computed, never stored)
  const uint16_t* wrow = a.W + static_cast<long long>(min(n0 + r16, N - 1)) * K + g * 8;
  // token rows of the tile; rows past nrows repeat the last one (computed, never stored)
  const uint16_t* xrow[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int t = min(tb * 16 + r16, nrows - 1);
    xrow[tb] = a.X + static_cast<long long>(row0 + t) * a.ldx + g * 8;
  }

  f32x4 acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int klen = k_end - k_beg;
  const int nfull = klen / KC;
  const int ntail = (klen % KC) / 32;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // P-stage ring: chunk c lives in stage c % P; MFMA step m of a chunk covers k = 32 m + 8 g + e.
  // The loop body is straight-line (every load and MFMA unconditional) so that the waits the
  // compiler inserts before each MFMA leave the younger stages in flight.
  u32x4 wst[P][4];
  u32x4 xst[P][NTB][4];
  auto load_chunk = [&](int c, u32x4 (&w)[4], u32x4 (&x)[NTB][4]) __attribute__((always_inline)) {
    const int k0 = k_beg + c * KC;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      w[m] = load_stream(wrow + k0 + 32 * m);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) x[tb][m] = ld16(xrow[tb] + k0 + 32 * m);
    }
  };
  if (nfull > 0) {
#pragma unroll
    for (int q = 0; q < P; ++q) load_chunk(min(q, nfull - 1), wst[q], xst[q]);
    __builtin_amdgcn_sched_barrier(0);
    const int ngroups = (nfull + P - 1) / P;
    for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int cc = gi * P + q;
        const bool live = cc < nfull;  // a chunk past the end repeats the last one: zero it
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const u32x4 wv = live ? wst[q][m] : zero4;
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb) acc[tb] = mfma16x16x32(wv, xst[q][tb][m], acc[tb]);
        }
        // keep the stage order: this chunk's MFMAs, then the refill of its stage
        __builtin_amdgcn_sched_barrier(0);
        load_chunk(min(cc + P, nfull - 1), wst[q], xst[q]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (ntail > 0) {
    const int kt = k_beg + nfull * KC;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      if (s < ntail) {
        const u32x4 wt = ld16(wrow + kt + 32 * s);
        u32x4 xt[NTB];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) xt[tb] = ld16(xrow[tb] + kt + 32 * s);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) acc[tb] = mfma16x16x32(wt, xt[tb], acc[tb]);
      }
    }
  }

  // epilogue: lane holds out[expert n0 + 4g + j][token tb*16 + r16].  Four consecutive experts
  // go out as one 16-byte store when they are all in range and the row stride keeps it aligned;
  // otherwise element by element (any expert count).
  float* o = static_cast<float*>(a.out) + static_cast<long long>(ks) * a.split_stride;
  const int n = n0 + 4 * g;
  const bool vec = (a.ldo & 3) == 0 && n + 3 < N;
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int t = tb * 16 + r16;
    if (t >= nrows || n >= N) continue;
    float* dst = o + static_cast<long long>(row0 + t) * a.ldo + n;
    if (vec) {
      *reinterpret_cast<float4*>(dst) = make_float4(acc[tb][0], acc[tb][1], acc[tb][2], acc[tb][3]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n + j < N) dst[j] = acc[tb][j];
    }
  }
}

template <int NTB, int P>
hipError_t launch_s(WGemmArgs a, hipStream_t s) {
  constexpr int KC = 128;
  a.n_nblk = (a.N + kRows - 1) / kRows;
  a.grid_tiles = (a.ntok + NTB * 16 - 1) / (NTB * 16);
  if (a.ksplit < 1) a.ksplit = 1;
  const int nchunk = (a.K + KC - 1) / KC;
  a.k_per_split = ((nchunk + a.ksplit - 1) / a.ksplit) * KC;
  int grid = a.grid_tiles * a.ksplit * a.n_nblk;
  grid = (grid + 7) & ~7;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_sgemm<NTB, P>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_dense_f32(const WGemmArgs& a, hipStream_t s) {
  // long prefill chunks: 64-token tiles, so the router weights are re-read 4x less often
  if (a.ntok >= 1024) return launch_s<4, 3>(a, s);
  return launch_s<1, 3>(a, s);
}

}  // namespace dg
