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

template <int NTB, int NRT, int NW, int EPI, int KC>
struct Cfg {
  static constexpr int TR = NTB * 16;                        // token rows per tile
  static constexpr bool PAIRED = EPI == EPI_SWIGLU;
  static constexpr int ROWS = PAIRED ? NW * 16 : NW * NRT * 16;  // features per workgroup
  static constexpr int THREADS = NW * 64;
  static constexpr int STRIDE = KC + 8;                      // bf16 per staged token row
  static constexpr int SEG = KC / 8;                         // 16-byte segments per staged row
  static constexpr int XLOADS = TR * SEG / THREADS;          // 16-byte token loads per thread
  static constexpr int WV = KC / 32;                         // uint4 per lane per row tile
  static_assert(XLOADS >= 1 && TR * SEG % THREADS == 0, "staging must divide evenly");
  static_assert(!PAIRED || NRT == 2, "SwiGLU pairs one gate and one up row tile");
  static constexpr int LDS_BYTES = 2 * TR * STRIDE * 2;
};

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// streaming (non-temporal) 16-byte load: weights are read once per step
__device__ __forceinline__ u32x4 load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// statistics of 8 scaled logits given in increasing vocabulary order
__device__ __forceinline__ SoftStats stats8(const float* y, int n_a, int n_b) {
  float m = y[0];
  int k_best = 0;
#pragma unroll
  for (int k = 1; k < 8; ++k)
    if (y[k] > m) {
      m = y[k];
      k_best = k;
    }
  float r = 0.f, a = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float d = y[k] - m;
    const float e = (k == k_best) ? 0.f : exp2f(d);
    r += e;
    a += d * e;
  }
  SoftStats s;
  s.m = m;
  s.idx = k_best < 4 ? n_a + k_best : n_b + (k_best - 4);
  s.r = r;
  s.a = a;
  return s;
}

template <int NTB, int NRT, int NW, int EPI, int KC>
__global__ __launch_bounds__(NW * 64) void k_wgemm(WGemmArgs a) {
  using C = Cfg<NTB, NRT, NW, EPI, KC>;
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* buf0 = lds;
  uint16_t* buf1 = lds + C::TR * C::STRIDE;

  // ---- tile decode: slot = ((tile * ksplit + ks) * n_nblk + nb) --------------------------
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
  const int n0 = nb * C::ROWS;
  if (n0 >= N) return;
  // an empty k-range still writes its (zero) partial plane
  const int k_beg = min(K, ks * a.k_per_split);
  const int k_end = min(K, k_beg + a.k_per_split);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;

  // weight rows this lane loads (A operand rows) and the first output feature of each row tile
  const uint16_t* wrow[NRT];
  int tile_n[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    int base;
    if (C::PAIRED) {
      base = n0 + wave * 16;  // feature index inside [0, F)
      tile_n[rt] = base;
      base += rt * N;         // rt 0: gate rows, rt 1: up rows
    } else {
      base = n0 + (wave * NRT + rt) * 16;
      tile_n[rt] = base;
    }
    const int lim = C::PAIRED ? (rt + 1) * N : N;
    const int row = min(base + r16, lim - 1);
    wrow[rt] = W + static_cast<long long>(row) * K;
  }

  // token rows this thread stages
  const uint16_t* xptr[C::XLOADS];
  int xoff[C::XLOADS];
  int xseg[C::XLOADS];
  bool xok[C::XLOADS];
#pragma unroll
  for (int it = 0; it < C::XLOADS; ++it) {
    const int idx = tid + it * C::THREADS;
    const int r = idx / C::SEG, c16 = idx % C::SEG;
    xok[it] = r < nrows;
    const int rr = xok[it] ? row0 + r : row0;
    const int xr = a.x_rows ? a.x_rows[rr] : rr;
    xptr[it] = a.X + static_cast<long long>(xr) * a.ldx + c16 * 8;
    xoff[it] = r * C::STRIDE + c16 * 8;
    xseg[it] = c16;
  }

  f32x4 acc[NRT][NTB];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[rt][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int klen = k_end - k_beg;
  const int nfull = klen / KC;
  const int ntail = (klen % KC) / 32;  // trailing 32-wide steps
  const int ntb_live = (nrows + 15) >> 4;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  u32x4 wcur[NRT][C::WV], wnext[NRT][C::WV];
  u32x4 xs[C::XLOADS];

  // full chunk c covers k in [k_beg + c KC, +KC); lane group g loads KC/4 contiguous k
  auto load_w = [&](int c, u32x4 (&w)[NRT][C::WV]) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const uint16_t* p = wrow[rt] + k_beg + c * KC + g * (KC / 4);
#pragma unroll
      for (int v = 0; v < C::WV; ++v) w[rt][v] = load_stream(p + 8 * v);
    }
  };
  auto load_x = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < C::XLOADS; ++it)
      xs[it] = xok[it] ? ld16(xptr[it] + k_beg + c * KC) : zero4;
  };
  auto store_x = [&](uint16_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < C::XLOADS; ++it) st16(buf + xoff[it], xs[it]);
  };
  auto compute = [&](const uint16_t* buf, const u32x4 (&w)[NRT][C::WV]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < C::WV; ++m) {
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        if (tb < ntb_live) {
          const u32x4 bfrag = ld16(buf + (tb * 16 + r16) * C::STRIDE + g * (KC / 4) + m * 8);
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) acc[rt][tb] = mfma16x16x32(w[rt][m], bfrag, acc[rt][tb]);
        }
      }
    }
  };

  if (nfull > 0) {
    load_x(0);
    load_w(0, wcur);
    store_x(buf0);
    __syncthreads();
    for (int c = 0; c < nfull; ++c) {
      const bool more = c + 1 < nfull;
      if (more) {
        load_x(c + 1);
        load_w(c + 1, wnext);
      }
      compute((c & 1) ? buf1 : buf0, wcur);
      if (more) store_x((c & 1) ? buf0 : buf1);
      __syncthreads();
      if (more) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int v = 0; v < C::WV; ++v) wcur[rt][v] = wnext[rt][v];
      }
    }
  }
  if (ntail > 0) {
    // trailing 32-wide steps: step s, lane group g supplies k = kt + 32 s + 8 g + (0..7)
    const int kt = k_beg + nfull * KC;
    uint16_t* buf = (nfull & 1) ? buf1 : buf0;
#pragma unroll
    for (int it = 0; it < C::XLOADS; ++it) {
      if (xseg[it] < ntail * 4) {
        const u32x4 v = xok[it] ? ld16(xptr[it] + kt) : zero4;
        st16(buf + xoff[it], v);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < C::WV - 1; ++s) {
      if (s >= ntail) break;
      u32x4 wt[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) wt[rt] = ld16(wrow[rt] + kt + s * 32 + g * 8);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        if (tb < ntb_live) {
          const u32x4 bfrag = ld16(buf + (tb * 16 + r16) * C::STRIDE + s * 32 + g * 8);
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) acc[rt][tb] = mfma16x16x32(wt[rt], bfrag, acc[rt][tb]);
        }
      }
    }
  }

  // ---- epilogue: lane holds out[feature tile_n[rt] + 4g + j][token tb*16 + r16] ------------
  if constexpr (EPI == EPI_LMHEAD) {
    // bf16 logits, and statistics of the rounded logits scaled by log2(e)/T
    __syncthreads();  // staging buffers are reused for the cross-wave merge
    SoftStats* red = reinterpret_cast<SoftStats*>(lds);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int t = tb * 16 + r16;
      const bool ok = t < nrows;
      float y[8];
      uint16_t* o = static_cast<uint16_t*>(a.out) + static_cast<long long>(row0 + t) * a.ldo;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int n = tile_n[rt] + 4 * g;
        uint2 pk;
        pk.x = pack_bf2(acc[rt][tb][0], acc[rt][tb][1]);
        pk.y = pack_bf2(acc[rt][tb][2], acc[rt][tb][3]);
        if (ok) *reinterpret_cast<uint2*>(o + n) = pk;
        y[rt * 4 + 0] = __uint_as_float(pk.x << 16) * a.inv_t_log2e;
        y[rt * 4 + 1] = __uint_as_float(pk.x & 0xffff0000u) * a.inv_t_log2e;
        y[rt * 4 + 2] = __uint_as_float(pk.y << 16) * a.inv_t_log2e;
        y[rt * 4 + 3] = __uint_as_float(pk.y & 0xffff0000u) * a.inv_t_log2e;
      }
      SoftStats s = stats8(y, tile_n[0] + 4 * g, tile_n[NRT - 1] + 4 * g);
      bool bad = false;
#pragma unroll
      for (int k = 0; k < 8; ++k) bad |= !(fabsf(y[k]) <= 3.402823466e38f);
      if (bad) s.r = NAN;
#pragma unroll
      for (int o2 = 16; o2 <= 32; o2 <<= 1) {
        const SoftStats u = stats_shfl_xor(s, o2);
        const bool nan = isnan(s.r) || isnan(u.r);
        s = stats_merge(s, u);
        if (nan) s.r = NAN;
      }
      if (g == 0) red[wave * C::TR + t] = s;
    }
    __syncthreads();
    for (int t = tid; t < nrows; t += C::THREADS) {
      SoftStats s = red[t];
      bool nan = isnan(s.r);
      for (int w = 1; w < NW; ++w) {
        const SoftStats u = red[w * C::TR + t];
        nan |= isnan(u.r);
        s = stats_merge(s, u);
      }
      if (nan) s.r = NAN;
      a.part[static_cast<long long>(row0 + t) * a.n_nblk + nb] = s;
    }
    return;
  }

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
        } else {  // EPI_F32: split ks writes its own partial plane
          float* o = static_cast<float*>(a.out) + static_cast<long long>(ks) * a.split_stride;
          *reinterpret_cast<float4*>(o + orow * a.ldo + n) =
              make_float4(acc[rt][tb][0], acc[rt][tb][1], acc[rt][tb][2], acc[rt][tb][3]);
        }
      }
    }
  }
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

template <int NTB, int NRT, int NW, int EPI, int KC>
hipError_t launch_cfg(WGemmArgs a, hipStream_t s) {
  using C = Cfg<NTB, NRT, NW, EPI, KC>;
  const int nmax = a.chunks ? max(a.N, a.N_sh) : a.N;
  a.n_nblk = (nmax + C::ROWS - 1) / C::ROWS;
  if (!a.chunks) a.grid_tiles = (a.ntok + C::TR - 1) / C::TR;
  if (a.ksplit < 1) a.ksplit = 1;
  const int kmax = a.chunks ? max(a.K, a.K_sh) : a.K;
  // k per split: a multiple of KC (except the last split)
  const int nchunk = (kmax + KC - 1) / KC;
  a.k_per_split = ((nchunk + a.ksplit - 1) / a.ksplit) * KC;
  int grid = a.grid_tiles * a.ksplit * a.n_nblk;
  grid = (grid + 7) & ~7;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_wgemm<NTB, NRT, NW, EPI, KC>), dim3(grid), dim3(C::THREADS), C::LDS_BYTES,
                     s, a);
  return hipGetLastError();
}

}  // namespace

int gemm_lmhead_rows_per_block() { return Cfg<16, 2, 8, EPI_LMHEAD, 64>::ROWS; }

hipError_t launch_gemm_dense_bf16(const WGemmArgs& a, hipStream_t s) {
  return launch_s<4, 1, EPI_BF16, 2>(a, s);
}
hipError_t launch_gemm_dense_f32(const WGemmArgs& a, hipStream_t s) {
  return launch_s<4, 1, EPI_F32, 2>(a, s);
}
hipError_t launch_gemm_lmhead(const WGemmArgs& a, hipStream_t s) {
  return launch_cfg<16, 2, 8, EPI_LMHEAD, 64>(a, s);
}

}  // namespace dg
