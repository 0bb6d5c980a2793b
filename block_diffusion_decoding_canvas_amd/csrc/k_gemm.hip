// Weight-streaming GEMMs on MFMA for the canvas step: out[r][n] = sum_k X[row(r)][k] W[n][k].
//
// The token count of a step is small (one 256-token canvas per batch entry), so every GEMM of
// the decoder is a "skinny" product whose cost is streaming the weight matrix from HBM.  The
// kernel is organised around that:
//   * weights are the MFMA A operand (16 output features x 32 k per v_mfma_f32_16x16x32_bf16),
//     loaded by each wave straight from HBM into registers, KC/4 contiguous k per lane group,
//     one k-chunk ahead of the MFMAs;
//   * tokens are the B operand (32 k x 16 tokens), staged once per workgroup and k-chunk into LDS
//     (double buffered) and shared by all waves;
//   * a tile is (expert, up to NTB*16 token rows, one block of output features, one k-split);
//     dense products enumerate tiles arithmetically, the MoE products read the tile list the
//     permute kernel writes (one expert per tile, the shared expert last), so each touched
//     expert's weights are streamed once per step;
//   * workgroup ids are remapped so consecutive tiles run on the same XCD and share its L2
//     (the token rows of a tile are re-read from there by its feature blocks);
//   * split-K writes fp32 partials [split][row][n] that the consumer sums in split order, so the
//     result is deterministic.
// Epilogues: bf16 store, fp32 (partial) store, SwiGLU (gate and up rows in one wave), and the LM
// head's bf16 logits plus per-block softmax statistics of the tempered, rounded logits.
//
// k-order inside an MFMA: lane group g (= lane / 16) supplies 8 consecutive k of its slice per
// MFMA; A and B use the same assignment, so every dot product is the exact sum over the chunk
// whatever order the hardware adds in.
#include "dg_internal.h"

namespace dg {
namespace {

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// streaming (non-temporal) 16-byte load: weights are read once per step
__device__ __forceinline__ u32x4 load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------------------------------------
// Streaming variant for the weight-bound products (dense projections and grouped experts):
// every wave works alone on its own feature rows, with no LDS and no barrier.  Weights and the
// tile's token fragments go straight from memory into a P-stage register ring, so chunk c is
// consumed while chunks c+1 .. c+P-1 are still in flight; because vector-memory counters retire
// in order, nothing newer than those has to be waited for.  Token fragments are re-read by the
// waves of a workgroup from L2 (a tile holds at most NTB*16 token rows).

template <int NTB, int NRT, int EPI>
struct SCfg {
  static constexpr bool PAIRED = EPI == EPI_SWIGLU;
  static constexpr int WAVES = 4;
  static constexpr int ROWS = PAIRED ? WAVES * 16 : WAVES * NRT * 16;  // features per workgroup
  static constexpr int TR = NTB * 16;
  static_assert(!PAIRED || NRT == 2, "SwiGLU pairs one gate and one up row tile");
};

template <int NTB, int NRT, int EPI, int P>
__global__ __launch_bounds__(256) void k_sgemm(WGemmArgs a) {
  using C = SCfg<NTB, NRT, EPI>;
  constexpr int KC = 128;
  const int slot = xcd_remap(blockIdx.x, gridDim.x);
  const int nb = slot % a.n_nblk;
  const int tk = slot / a.n_nblk;
  const int ks = tk % a.ksplit;
  const int tile = tk / a.ksplit;
  if (tile >= a.grid_tiles) return;
  int expert = 0, row0, nrows;
  if (a.chunks) {
    if (tile >= *a.n_chunks) return;
    expert = a.chunks[3 * tile];
    row0 = a.chunks[3 * tile + 1];
    nrows = a.chunks[3 * tile + 2];
  } else {
    row0 = tile * C::TR;
    nrows = min(C::TR, a.ntok - row0);
  }
  const bool shared = a.chunks && expert == a.n_experts;
  const uint16_t* W = shared ? a.W_sh : a.W + static_cast<long long>(expert) * a.w_estride;
  const int N = shared ? a.N_sh : a.N;
  const int K = shared ? a.K_sh : a.K;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = nb * C::ROWS + wave * (C::PAIRED ? 16 : NRT * 16);
  if (n0 >= N) return;  // waves are independent: no barrier follows
  // an empty k-range still writes its (zero) partial plane
  const int k_beg = min(K, ks * a.k_per_split);
  const int k_end = min(K, k_beg + a.k_per_split);

  const uint16_t* wrow[NRT];
  int tile_n[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int base = C::PAIRED ? n0 : n0 + rt * 16;
    tile_n[rt] = base;
    const int lim = C::PAIRED ? (rt + 1) * N : N;
    const int row = min((C::PAIRED ? base + rt * N : base) + r16, lim - 1);
    wrow[rt] = W + static_cast<long long>(row) * K + g * 8;
  }
  // token rows of the tile; rows past nrows repeat the last one (computed, never stored)
  const uint16_t* xrow[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int t = min(tb * 16 + r16, nrows - 1);
    const int rr = row0 + t;
    const int xr = a.x_rows ? a.x_rows[rr] : rr;
    xrow[tb] = a.X + static_cast<long long>(xr) * a.ldx + g * 8;
  }

  f32x4 acc[NRT][NTB];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[rt][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int klen = k_end - k_beg;
  const int nfull = klen / KC;
  const int ntail = (klen % KC) / 32;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // P-stage ring: chunk c lives in stage c % P; MFMA step m of a chunk covers k = 32 m + 8 g + e.
  // The loop body is straight-line (every load and MFMA unconditional) so that the waits the
  // compiler inserts before each MFMA leave the younger stages in flight.
  u32x4 wst[P][NRT][4];
  u32x4 xst[P][NTB][4];
  auto load_chunk = [&](int c, u32x4 (&w)[NRT][4], u32x4 (&x)[NTB][4]) __attribute__((always_inline)) {
    const int k0 = k_beg + c * KC;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) w[rt][m] = load_stream(wrow[rt] + k0 + 32 * m);
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
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            const u32x4 wv = live ? wst[q][rt][m] : zero4;
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
              acc[rt][tb] = mfma16x16x32(wv, xst[q][tb][m], acc[rt][tb]);
          }
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
        u32x4 wt[NRT], xt[NTB];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) wt[rt] = ld16(wrow[rt] + kt + 32 * s);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) xt[tb] = ld16(xrow[tb] + kt + 32 * s);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) acc[rt][tb] = mfma16x16x32(wt[rt], xt[tb], acc[rt][tb]);
      }
    }
  }

  // epilogue: lane holds out[feature tile_n[rt] + 4g + j][token tb*16 + r16]
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int t = tb * 16 + r16;
    if (t >= nrows) continue;
    const long long orow = row0 + t;
    if constexpr (EPI == EPI_SWIGLU) {
      const int f = tile_n[0] + 4 * g;
      if (f < N) {
        uint2 pk;
        pk.x = pack_bf2(silu(acc[0][tb][0]) * acc[1][tb][0], silu(acc[0][tb][1]) * acc[1][tb][1]);
        pk.y = pack_bf2(silu(acc[0][tb][2]) * acc[1][tb][2], silu(acc[0][tb][3]) * acc[1][tb][3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow * a.ldo + f) = pk;
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int n = tile_n[rt] + 4 * g;
        if (n >= N) continue;
        if constexpr (EPI == EPI_BF16) {
          uint2 pk;
          pk.x = pack_bf2(acc[rt][tb][0], acc[rt][tb][1]);
          pk.y = pack_bf2(acc[rt][tb][2], acc[rt][tb][3]);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow * a.ldo + n) = pk;
        } else {
          float* o = static_cast<float*>(a.out) + static_cast<long long>(ks) * a.split_stride;
          *reinterpret_cast<float4*>(o + orow * a.ldo + n) =
              make_float4(acc[rt][tb][0], acc[rt][tb][1], acc[rt][tb][2], acc[rt][tb][3]);
        }
      }
    }
  }
}

template <int NTB, int NRT, int EPI, int P>
hipError_t launch_s(WGemmArgs a, hipStream_t s) {
  using C = SCfg<NTB, NRT, EPI>;
  constexpr int KC = 128;
  const int nmax = a.chunks ? max(a.N, a.N_sh) : a.N;
  a.n_nblk = (nmax + C::ROWS - 1) / C::ROWS;
  if (!a.chunks) a.grid_tiles = (a.ntok + C::TR - 1) / C::TR;
  if (a.ksplit < 1) a.ksplit = 1;
  const int kmax = a.chunks ? max(a.K, a.K_sh) : a.K;
  const int nchunk = (kmax + KC - 1) / KC;
  a.k_per_split = ((nchunk + a.ksplit - 1) / a.ksplit) * KC;
  int grid = a.grid_tiles * a.ksplit * a.n_nblk;
  grid = (grid + 7) & ~7;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_sgemm<NTB, NRT, EPI, P>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_dense_bf16(const WGemmArgs& a, hipStream_t s) {
  return launch_s<4, 1, EPI_BF16, 2>(a, s);
}
hipError_t launch_gemm_dense_f32(const WGemmArgs& a, hipStream_t s) {
  // long prefill chunks: 64-token tiles, so the router weights are re-read 4x less often
  if (a.ntok >= 1024) return launch_s<4, 1, EPI_F32, 3>(a, s);
  return launch_s<1, 1, EPI_F32, 3>(a, s);
}

}  // namespace dg
