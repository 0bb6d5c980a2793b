// Expert (routed + shared) SwiGLU FFN products: the HBM-bound core of the step.
//
// The MoE layer (DiffusionGemma model card, dimension table: 8 of 128 experts active plus 1
// shared) touches every expert's weights once per step while each expert sees only ~16 of the
// canvas tokens, so the products stream ~1.5 GB per layer at ~16 flop/byte.  Layout and schedule:
//   * expert weights are stored fragment-major ("tiled"): each 16-row x 32-k MFMA A fragment is a
//     contiguous 1 KiB block with lane i's 8 elements at 16 i bytes, so one wave load instruction
//     reads 1 KiB contiguous (dg_pack_weight makes the layout);
//   * a workgroup (4 waves) takes one token tile (<= 32 rows of one expert, gathered through the
//     permutation) and 4 x 16 output features; each wave streams its 32 weight rows through a
//     register ring PS steps deep (one step = 32 k), pinned with scheduling barriers so that the
//     in-order vector-memory counter only waits for the oldest step;
//   * the token rows are staged in LDS in 512-k segments, double buffered, loaded one segment
//     ahead, so they are read from L2 once per workgroup instead of once per wave and MFMA;
//   * gate/up: the wave holds 16 gate rows and the matching 16 up rows and applies SwiGLU in
//     the epilogue; down: 2 tiles of 16 output rows; outputs are bf16 rows in permuted order.
#include "dg_internal.h"

namespace dg {
namespace {

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }

__device__ __forceinline__ u32x4 ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// statistics of NV scaled logits in increasing vocabulary order, y[k] the logit of vocabulary
// row n0 + (k / 4) * 16 + k % 4 (4 rows of each of NV / 4 16-row tiles): the maximum from a max
// tree, its first position (lowest index on ties) from a reverse scan, 2^(y - m) with the
// hardware exp2 (arguments <= 0).  Non-finite inputs leave r or a NaN (+inf through inf - inf,
// NaN directly, -inf through -inf * 0), which the caller turns into the flag.
template <int NV>
__device__ __forceinline__ SoftStats stats_rows(const float* y, int n0) {
  float mx[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) mx[k] = y[k];
#pragma unroll
  for (int w = NV / 2; w >= 1; w >>= 1)
#pragma unroll
    for (int k = 0; k < w; ++k) mx[k] = fmaxf(mx[k], mx[k + w]);
  const float m = mx[0];
  int k_best = NV - 1;
#pragma unroll
  for (int k = NV - 2; k >= 0; --k) k_best = (y[k] == m) ? k : k_best;
  float r = 0.f, acc = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const float d = y[k] - m;
    const float e = (k == k_best) ? 0.f : __builtin_amdgcn_exp2f(d);
    r += e;
    acc = __builtin_fmaf(d, e, acc);
  }
  SoftStats s;
  s.m = m;
  s.idx = n0 + (k_best >> 2) * 16 + (k_best & 3);
  s.r = (r != r || acc != acc) ? NAN : r;
  s.a = acc;
  return s;
}

// NTB: 16-token blocks per tile; SEG: k per staged token segment; WAVES per workgroup; PS: depth
// of the weight register ring in steps; F8: e4m3 codes for X and W (with per-row scales)
// instead of bf16.  A step is one 16-byte fragment load per lane and weight row tile: 32 k of
// bf16 (one MFMA) or 64 k of e4m3 (two steps make one 16x16x128 MFMA).  EPI_SWIGLU: gate/up pairs, 16 features per
// wave (bf16 output, fp32 with F8); otherwise 32 output rows per wave.  EPI_BF16 stores bf16;
// EPI_F32 stores the fp32 partial of k-split ks in its own plane; EPI_LMHEAD stores bf16
// logits and, per (token, workgroup block of rows), the softmax statistics of the rounded
// logits scaled by log2(e)/T.
template <int EPI, int NTB, int SEG, int WAVES, int PS, bool F8 = false, int RT = 2>
__global__ __launch_bounds__(WAVES * 64) void k_stream(WGemmArgs a) {
  static_assert(RT == 2 || EPI != EPI_SWIGLU, "gate/up pairs take two row tiles per wave");
  constexpr int NTHR = WAVES * 64;
  constexpr int EB = F8 ? 1 : 2;                    // bytes per element
  constexpr int KSTEP = F8 ? 64 : 32;               // k per step
  constexpr int MT = NTB * 16;                      // token rows per tile
  constexpr int SEGB = SEG * EB;                    // bytes of one staged row segment
  constexpr int STRIDE = SEGB + 16;                 // bytes per staged row (conflict-free reads)
  constexpr int XL = MT * (SEGB / 16) / NTHR;       // 16-byte token loads per thread per segment
  constexpr int SSTEPS = SEG / KSTEP;
  static_assert(SSTEPS % PS == 0 && XL >= 1 && MT * (SEGB / 16) % NTHR == 0,
                "segment must hold whole ring groups");
  static_assert(!F8 || PS % 2 == 0, "e4m3 steps go in pairs through the ring");
  __shared__ __align__(16) uint8_t xs_lds[2][MT * STRIDE];

  // logical slot -> (token tile, k split, row block).  Consecutive slots run on one XCD (one L2):
  // grouped products put a tile's row blocks together (its gathered token rows are shared);
  // dense products put the token tiles of one row block together, so every weight band is
  // fetched from HBM into one L2 and reused there by all token tiles
  int slot, n_ch = 0;
  if (a.chunks) {
    // the grid is sized for the most tiles a routing can produce; the active slots (known only
    // on the device) are spread evenly over the 8 XCDs, a contiguous run on each
    n_ch = *a.n_chunks;
    const int n_active = n_ch * a.ksplit * a.n_nblk;
    const int per = (n_active + 7) >> 3;
    const int j = blockIdx.x >> 3;
    slot = (blockIdx.x & 7) * per + j;
    if (j >= per || slot >= n_active) return;
  } else {
    slot = xcd_remap(blockIdx.x, gridDim.x);
  }
  int nb, ks, tile;
  if (a.chunks) {
    const int sh_first = n_ch - a.sh_tiles;   // the shared expert's tiles close the list
    if (a.sh_tiles > 0 && a.ksplit == 1 && slot >= sh_first * a.n_nblk) {
      // the shared expert's tiles of one row block in consecutive slots (one XCD, one L2)
      const int j = slot - sh_first * a.n_nblk;
      nb = j / a.sh_tiles;
      tile = sh_first + j % a.sh_tiles;
      ks = 0;
    } else {
      nb = slot % a.n_nblk;
      const int tk = slot / a.n_nblk;
      ks = tk % a.ksplit;
      tile = tk / a.ksplit;
    }
  } else {
    tile = slot % a.grid_tiles;
    const int rest = slot / a.grid_tiles;
    ks = rest % a.ksplit;
    nb = rest / a.ksplit;
  }
  if (tile >= a.grid_tiles || nb >= a.n_nblk) return;
  int expert = 0, row0, nrows;
  if (a.chunks) {
    if (tile >= *a.n_chunks) return;
    expert = a.chunks[3 * tile];
    row0 = a.chunks[3 * tile + 1];
    nrows = a.chunks[3 * tile + 2];
  } else {
    row0 = tile * MT;
    nrows = min(MT, a.ntok - row0);
  }
  const bool shared = a.chunks && expert == a.n_experts;
  // w_estride counts elements (EB bytes each)
  const uint8_t* W = shared ? reinterpret_cast<const uint8_t*>(a.W_sh)
                            : reinterpret_cast<const uint8_t*>(a.W) +
                                  static_cast<long long>(expert) * a.w_estride * EB;
  const int N = shared ? a.N_sh : a.N;      // gate/up: F; otherwise output rows
  const int K = shared ? a.K_sh : a.K;
  constexpr bool GU = EPI == EPI_SWIGLU;
  const int n0 = nb * (GU ? WAVES * 16 : WAVES * 16 * RT);  // first output feature of the workgroup
  if (n0 >= N) return;                      // uniform across the workgroup
  const int k_beg = min(K, ks * a.k_per_split);   // a multiple of SEG
  const int k_end = min(K, k_beg + a.k_per_split);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int ksteps = K / KSTEP;
  const int s_first = k_beg / KSTEP, s_last = k_end / KSTEP;   // this split's steps

  // the wave's RT row tiles (fragment-major weights: tile rt, step s at (rt * ksteps + s) KiB)
  int feat[RT];
  const uint8_t* wfrag[RT];
  bool wave_live;
  if (GU) {
    const int f = n0 + wave * 16;
    wave_live = f < N;
    const int fc = wave_live ? f : N - 16;
    feat[0] = feat[1] = f;
    wfrag[0] = W + (static_cast<long long>(fc / 16) * ksteps) * 1024 + lane * 16;        // gate
    wfrag[1] = W + (static_cast<long long>((N + fc) / 16) * ksteps) * 1024 + lane * 16;  // up
  } else {
    const int r = n0 + wave * 16 * RT;
    wave_live = r < N;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      feat[rt] = r + 16 * rt;
      const int rc = min(feat[rt], N - 16);     // tiles past the last row read a valid tile
      wfrag[rt] = W + (static_cast<long long>(rc / 16) * ksteps) * 1024 + lane * 16;
    }
  }

  // token staging: piece it of a thread is the 16 bytes at column xc16 of segment row
  // xr0 + it * RS.  Every load is issued unconditionally from an in-range address (rows past the
  // tile read its last row, k past the range reads the range's last piece) and the piece is
  // zeroed at the store: conditional loads would make the compiler wait for every outstanding
  // load (the weight ring included) before the LDS store.  Row addresses are 32-bit byte offsets
  // from a uniform base (the tile's first row, or row 0 of a gathered matrix: fewer than 65,536
  // rows of at most 16 KiB), so that a thread's staging state is one register per piece
  constexpr int PPR = SEGB / 16;                    // 16-byte pieces per staged row
  constexpr int RS = NTHR / PPR;                    // rows between a thread's pieces
  static_assert(NTHR % PPR == 0, "a segment row must split evenly over the threads");
  const int xr0 = tid / PPR, xc16 = tid % PPR;
  const int xcol = xc16 * (16 / EB);                // element column in the segment
  const uint8_t* Xb = reinterpret_cast<const uint8_t*>(a.X) +
                      (a.x_rows ? 0ll : static_cast<long long>(row0) * a.ldx * EB);
  uint32_t xoff[XL];
#pragma unroll
  for (int it = 0; it < XL; ++it) {
    const int r = min(xr0 + it * RS, nrows - 1);   // rows past the tile repeat its last row
    const int xr = a.x_rows ? a.x_rows[row0 + r] : r;
    xoff[it] = static_cast<uint32_t>(xr) * static_cast<uint32_t>(a.ldx * EB);
  }
  const int nseg = (k_end - k_beg + SEG - 1) / SEG;
  u32x4 xr_[XL];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  // piece it of segment sg (segments past the range read an in-range piece, stored as zeros)
  auto load_piece = [&](int it, int sg) __attribute__((always_inline)) {
    const int kc = min(k_beg + sg * SEG + xcol, k_end - 16 / EB);
    xr_[it] = ld16(Xb + (xoff[it] + static_cast<uint32_t>(kc * EB)));
  };
  // piece it, holding segment sg, into buffer sg & 1 (zeros past the tile's rows or the range)
  auto store_piece = [&](int it, int sg) __attribute__((always_inline)) {
    const bool ok = xr0 + it * RS < nrows && k_beg + sg * SEG + xcol < k_end;
    st16(&xs_lds[sg & 1][(xr0 + it * RS) * STRIDE + xc16 * 16], ok ? xr_[it] : zero4);
  };
  auto load_seg = [&](int sg) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < XL; ++it) load_piece(it, sg);
  };
  auto store_seg = [&](int sg) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < XL; ++it) store_piece(it, sg);
  };

  f32x4 acc[RT][NTB];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[rt][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weight ring: local step s (global step s_first + s) lives in stage s % PS.  Steps past the
  // end (the ring's last refills) still issue their loads, so that the loads stay straight-line,
  // but from a 1 KiB block that stays L2-resident instead of re-reading a weight fragment from
  // HBM; their data is replaced by zeros when used
  u32x4 wst[PS][RT];
  const uint8_t* hot = a.hot ? a.hot + lane * 16
                            : wfrag[0] + static_cast<long long>(max(s_last - 1, 0)) * 1024;
  auto load_step = [&](int s, u32x4 (&w)[RT]) __attribute__((always_inline)) {
    const bool in = s_first + s < s_last;
    const long long off = static_cast<long long>(s_first + s) * 1024;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) w[rt] = ld_nt(in ? wfrag[rt] + off : hot);
  };

  if (nseg > 0) {
    // the weight ring first: it depends only on the tile's expert, while the token pieces may
    // wait for the gathered row indices
    if (wave_live) {
#pragma unroll
      for (int q = 0; q < PS; ++q) load_step(q, wst[q]);
    }
    load_seg(0);
    store_seg(0);
    if (nseg > 1) load_seg(1);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }
  const int nsteps = s_last - s_first;
  // e4m3 operands go through the 16x16x128 MFMA, twice the rate of the 16x16x32 e4m3 form:
  // steps s and s + 1 (64 k each) make one MFMA.  A lane's 32 bytes are its 16 bytes of step s
  // then its 16 of step s + 1, for the weights (two ring stages) and the tokens (two LDS reads)
  // alike, so both operands list the same 128 k in the same order.  A pair always starts at an
  // even step from the split's first, so every tile shape sums the same pairs in the same order.
  // step_pair: the MFMAs with ring stages q, q + 1 (zero weights for a step past the end), then
  // both stages refilled with steps s + PS and s + 1 + PS
  auto step_pair = [&](const uint8_t* xb, int s, int s_beg, int q, bool live0, bool live1)
      __attribute__((always_inline)) {
    const int kin0 = (s - s_beg) * 64 + g * 16;
    const int kin1 = live1 ? kin0 + 64 : kin0;   // past the end: any staged bytes (zero weights)
    u32x4 w0[RT], w1[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      w0[rt] = live0 ? wst[q][rt] : zero4;
      w1[rt] = live1 ? wst[q + 1][rt] : zero4;
    }
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const uint8_t* xr = xb + (tb * 16 + r16) * STRIDE;
      const u32x4 b0 = ld16(xr + kin0), b1 = ld16(xr + kin1);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][tb] = mfma_f8_128(w0[rt], w1[rt], b0, b1, acc[rt][tb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_step(s + PS, wst[q]);
    load_step(s + 1 + PS, wst[q + 1]);
    __builtin_amdgcn_sched_barrier(0);
  };
  // one step (bf16): the token fragments of step s from LDS, the MFMAs with ring stage q (zero
  // weights when the step is past the end), then the ring stage refilled with step s + PS
  auto step = [&](const uint8_t* xb, int s, int s_beg, int q, bool live)
      __attribute__((always_inline)) {
    const int kin = (s - s_beg) * 64 + g * 16;   // byte offset in the staged row
    u32x4 wv[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) wv[rt] = live ? wst[q][rt] : zero4;
    auto mma = [&](const u32x4& bt, int tb) __attribute__((always_inline)) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][tb] = mfma16x16x32(wv[rt], bt, acc[rt][tb]);
    };
    if constexpr (NTB <= 4) {
      u32x4 b[NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) b[tb] = ld16(xb + (tb * 16 + r16) * STRIDE + kin);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) mma(b[tb], tb);
    } else {
      // many token blocks: their fragments flow through a 4-deep register ring, each read
      // issued four blocks ahead of its MFMAs (pinned), so LDS latency overlaps the MFMAs
      u32x4 br[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) br[i] = ld16(xb + (i * 16 + r16) * STRIDE + kin);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        mma(br[tb % 4], tb);
        if (tb + 4 < NTB) br[tb % 4] = ld16(xb + ((tb + 4) * 16 + r16) * STRIDE + kin);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_step(s + PS, wst[q]);
    __builtin_amdgcn_sched_barrier(0);
  };
  // the next segment's pieces go to the other LDS buffer, then the one after is loaded
  auto next_seg = [&](int sg) __attribute__((always_inline)) {
    if (sg + 1 < nseg) {
      store_seg(sg + 1);
      if (sg + 2 < nseg) load_seg(sg + 2);
    }
  };
  for (int sg = 0; sg < nseg; ++sg) {
    const uint8_t* xb = xs_lds[sg & 1];
    const int s_beg = sg * SSTEPS;
    if (wave_live && s_beg + SSTEPS <= nsteps) {
      // a full segment as straight-line code: the only loop-carried loads are then the token
      // pieces issued at the end of the previous segment, which are older than this segment's
      // weight loads, so the store below waits for them alone and the ring stays in flight.
      // With 4 or more token blocks (the dense products, run at one or two waves per SIMD) the
      // token fragments of the whole segment (fragment f = step u * NTB + block tb) stream
      // through a D-deep register ring, each LDS read issued D fragments ahead of its MFMAs, so
      // the LDS latency hides under independent MFMAs, and the token staging (the next
      // segment's pieces into the other buffer, free since the last barrier, then the pieces of
      // the one after from L2) is spread over the segment instead of waiting for its end; the
      // grouped expert products (2 token blocks, several waves per SIMD) keep their registers
      // for occupancy instead
      if constexpr (NTB < 4) {
        if constexpr (F8) {
#pragma unroll
          for (int u = 0; u < SSTEPS; u += 2) step_pair(xb, s_beg + u, s_beg, u % PS, true, true);
        } else {
#pragma unroll
          for (int u = 0; u < SSTEPS; ++u) step(xb, s_beg + u, s_beg, u % PS, true);
        }
        next_seg(sg);
      } else if constexpr (F8) {
        // as below, over pairs of steps: pair fragment f = pair p * NTB + block tb, each two LDS
        // reads (steps 2p and 2p + 1) through a D-deep ring (2 deep: a pair fragment feeds RT
        // MFMAs of 4x the work, and a deeper ring spills the 8-wave tiles)
        constexpr int NF = SSTEPS / 2 * NTB;
        constexpr int D = NF < 2 ? NF : 2;
        static_assert(NF % XL == 0, "token pieces must spread evenly over the fragments");
        constexpr int EVERY = NF / XL;
        const uint8_t* xf = xb + r16 * STRIDE + g * 16;
        u32x4 br0[D], br1[D];
        auto read = [&](int f, int slot) __attribute__((always_inline)) {
          const uint8_t* p = xf + (f % NTB) * 16 * STRIDE + (f / NTB) * 128;
          br0[slot] = ld16(p);
          br1[slot] = ld16(p + 64);
        };
#pragma unroll
        for (int i = 0; i < D; ++i) read(i, i);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int u = 2 * (f / NTB), tb = f % NTB;
          const u32x4 b0 = br0[f % D], b1 = br1[f % D];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            acc[rt][tb] = mfma_f8_128(wst[u % PS][rt], wst[(u + 1) % PS][rt], b0, b1, acc[rt][tb]);
          if (f + D < NF) read(f + D, f % D);
          __builtin_amdgcn_sched_barrier(0);
          if (tb == NTB - 1) {
            // the pair's last MFMAs have read its two ring stages: refill them
            load_step(s_beg + u + PS, wst[u % PS]);
            load_step(s_beg + u + 1 + PS, wst[(u + 1) % PS]);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (f % EVERY == EVERY - 1) {
            store_piece(f / EVERY, sg + 1);
            load_piece(f / EVERY, sg + 2);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
        constexpr int NF = SSTEPS * NTB;
        constexpr int D = NF < (NTB == 4 ? 8 : 4) ? NF : (NTB == 4 ? 8 : 4);
        static_assert(NF % XL == 0, "token pieces must spread evenly over the fragments");
        constexpr int EVERY = NF / XL;
        const uint8_t* xf = xb + r16 * STRIDE + g * 16;
        u32x4 br[D];
#pragma unroll
        for (int i = 0; i < D; ++i) br[i] = ld16(xf + (i % NTB) * 16 * STRIDE + (i / NTB) * 64);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int u = f / NTB, tb = f % NTB;
          const u32x4 bt = br[f % D];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            acc[rt][tb] = mfma16x16x32(wst[u % PS][rt], bt, acc[rt][tb]);
          if (f + D < NF)
            br[f % D] = ld16(xf + ((f + D) % NTB) * 16 * STRIDE + ((f + D) / NTB) * 64);
          __builtin_amdgcn_sched_barrier(0);
          if (tb == NTB - 1) {
            // the step's last MFMAs have read its ring stage: refill it with step s + PS
            load_step(s_beg + u + PS, wst[u % PS]);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (f % EVERY == EVERY - 1) {
            // unconditional: past the last segment the store fills the free buffer with
            // zeros and the load reads an in-range piece
            store_piece(f / EVERY, sg + 1);
            load_piece(f / EVERY, sg + 2);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else {
      // the last, partial segment (or a wave past the last output row, which only joins the
      // barriers)
      const int s_end = wave_live ? min(nsteps, s_beg + SSTEPS) : s_beg;
      for (int s0 = s_beg; s0 < s_end; s0 += PS) {
        if constexpr (F8) {
#pragma unroll
          for (int q = 0; q < PS; q += 2)
            step_pair(xb, s0 + q, s_beg, q, s0 + q < s_end, s0 + q + 1 < s_end);
        } else {
#pragma unroll
          for (int q = 0; q < PS; ++q) step(xb, s0 + q, s_beg, q, s0 + q < s_end);
        }
      }
      next_seg(sg);
    }
    if (sg + 1 < nseg) {
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (F8) {
    // dequantise: accumulator * token-row scale * weight-row scale
    const float* wsc = shared ? a.w_scale_sh : a.w_scale + static_cast<long long>(expert) * a.wsc_estride;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float sw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int wrow = (GU && rt == 1 ? N : 0) + feat[rt] + 4 * g + j;
        sw[j] = (wave_live && feat[rt] < N) ? wsc[wrow] : 0.f;
      }
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const int rr = row0 + min(tb * 16 + r16, nrows - 1);
        const float sa = a.x_scale[a.x_rows ? a.x_rows[rr] : rr];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rt][tb][j] = acc[rt][tb][j] * sa * sw[j];
      }
    }
  }
  if constexpr (EPI == EPI_LMHEAD) {
    // bf16 logits; each lane's statistics of the rounded, scaled logits it holds for a token
    // (4 rows of each of its RT tiles) go to LDS as one of the token's WAVES * 4 partials (the staging buffers are free
    // after this barrier), then TPT threads per token merge them in a fixed order
    __syncthreads();
    constexpr int NP = WAVES * 4;          // partials per token: (wave, lane group)
    constexpr int TPT = NTHR / MT;         // merging threads per token
    static_assert(TPT >= 1 && (TPT & (TPT - 1)) == 0 && NP % TPT == 0 && TPT <= 64,
                  "token partials must split evenly over a power-of-two thread group");
    static_assert(sizeof(SoftStats) * NP * MT <= sizeof(xs_lds), "LDS too small for stats");
    SoftStats* red = reinterpret_cast<SoftStats*>(&xs_lds[0][0]);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int t = tb * 16 + r16;
      const bool ok = t < nrows && wave_live;
      const int orow = row0 + min(t, nrows - 1);   // rows past the tile are never stored
      const long long orow_out =
          a.omap_C > 0 ? static_cast<long long>(a.omap[orow / a.omap_C]) * a.omap_C + orow % a.omap_C
                       : orow;
      uint16_t* o = static_cast<uint16_t*>(a.out) + orow_out * a.ldo;
      float y[4 * RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        uint2 pk;
        pk.x = pack_bf2(acc[rt][tb][0], acc[rt][tb][1]);
        pk.y = pack_bf2(acc[rt][tb][2], acc[rt][tb][3]);
        if (ok) *reinterpret_cast<uint2*>(o + feat[rt] + 4 * g) = pk;
        y[rt * 4 + 0] = __uint_as_float(pk.x << 16) * a.inv_t_log2e;
        y[rt * 4 + 1] = __uint_as_float(pk.x & 0xffff0000u) * a.inv_t_log2e;
        y[rt * 4 + 2] = __uint_as_float(pk.y << 16) * a.inv_t_log2e;
        y[rt * 4 + 3] = __uint_as_float(pk.y & 0xffff0000u) * a.inv_t_log2e;
      }
      SoftStats st = stats_rows<4 * RT>(y, feat[0] + 4 * g);
      if (!wave_live) st = SoftStats{-INFINITY, 0x7fffffff, 0.f, 0.f};   // rows past N: neutral
      red[(wave * 4 + g) * MT + t] = st;
    }
    __syncthreads();
    {
      // thread -> (token tid / TPT, partials (tid % TPT) * NP / TPT ...); then the group's
      // threads (consecutive lanes) combine by xor shuffles
      const int t = tid / TPT, part0 = (tid % TPT) * (NP / TPT);
      SoftStats st = red[part0 * MT + t];
      bool nan = isnan(st.r);
#pragma unroll
      for (int p = 1; p < NP / TPT; ++p) {
        const SoftStats u = red[(part0 + p) * MT + t];
        nan |= isnan(u.r);
        st = stats_merge(st, u);
      }
#pragma unroll
      for (int o2 = 1; o2 < TPT; o2 <<= 1) {
        const SoftStats u = stats_shfl_xor(st, o2);
        nan |= isnan(u.r);
        st = stats_merge(st, u);
      }
      if (nan) st.r = NAN;
      if (tid % TPT == 0 && t < nrows) a.part[static_cast<long long>(row0 + t) * a.n_nblk + nb] = st;
    }
    return;
  }
  if (!wave_live) return;

  // epilogue: lane holds out[feature tile + 4g + j][token tb*16 + r16]
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int t = tb * 16 + r16;
    if (t >= nrows) continue;
    const long long orow = row0 + t;
    if constexpr (GU && F8) {
      float* o = static_cast<float*>(a.out) + orow * a.ldo;
      const int f = feat[0] + 4 * g;
      *reinterpret_cast<float4*>(o + f) =
          make_float4(silu_f(acc[0][tb][0]) * acc[1][tb][0], silu_f(acc[0][tb][1]) * acc[1][tb][1],
                      silu_f(acc[0][tb][2]) * acc[1][tb][2], silu_f(acc[0][tb][3]) * acc[1][tb][3]);
    } else if constexpr (GU) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + orow * a.ldo;
      const int f = feat[0] + 4 * g;
      uint2 pk;
      pk.x = pack_bf2(silu_f(acc[0][tb][0]) * acc[1][tb][0], silu_f(acc[0][tb][1]) * acc[1][tb][1]);
      pk.y = pack_bf2(silu_f(acc[0][tb][2]) * acc[1][tb][2], silu_f(acc[0][tb][3]) * acc[1][tb][3]);
      *reinterpret_cast<uint2*>(o + f) = pk;
    } else if constexpr (EPI == EPI_BF16) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + orow * a.ldo;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (feat[rt] >= N) continue;
        uint2 pk;
        pk.x = pack_bf2(acc[rt][tb][0], acc[rt][tb][1]);
        pk.y = pack_bf2(acc[rt][tb][2], acc[rt][tb][3]);
        *reinterpret_cast<uint2*>(o + feat[rt] + 4 * g) = pk;
      }
    } else {
      float* o = static_cast<float*>(a.out) + static_cast<long long>(ks) * a.split_stride +
                 orow * a.ldo;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        if (feat[rt] < N)
          *reinterpret_cast<float4*>(o + feat[rt] + 4 * g) =
            make_float4(acc[rt][tb][0], acc[rt][tb][1], acc[rt][tb][2], acc[rt][tb][3]);
    }
  }
}

// fragment-major packing of a [rows][cols] bf16 matrix (rows % 16 == 0, cols % 32 == 0):
// element (n, k) goes to ((n/16 * cols/32 + k/32) * 64 + (k%32)/8 * 16 + n%16) * 8 + k%8
__global__ __launch_bounds__(256) void k_pack(const uint16_t* src, uint16_t* dst, long long rows,
                                              long long cols) {
  const long long frags = (rows / 16) * (cols / 32);
  const long long i = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (i >= frags) return;
  const int lane = threadIdx.x & 63;
  const long long rt = i / (cols / 32), s = i % (cols / 32);
  const long long n = rt * 16 + (lane & 15), k = s * 32 + (lane >> 4) * 8;
  st16(dst + i * 512 + lane * 8, ld16(src + n * cols + k));
}

template <int EPI, int NTB, int SEG, int WAVES, int PS, bool F8 = false, int RT = 2>
hipError_t launch_stream(WGemmArgs a, hipStream_t s) {
  const int per = EPI == EPI_SWIGLU ? WAVES * 16 : WAVES * 16 * RT;
  a.n_nblk = (std::max(a.N, a.chunks ? a.N_sh : a.N) + per - 1) / per;
  if (!a.chunks) a.grid_tiles = (a.ntok + NTB * 16 - 1) / (NTB * 16);
  if (a.ksplit < 1) a.ksplit = 1;
  const int kmax = a.chunks ? std::max(a.K, a.K_sh) : a.K;
  const int nseg = (kmax + SEG - 1) / SEG;
  a.k_per_split = ((nseg + a.ksplit - 1) / a.ksplit) * SEG;
  int grid = a.grid_tiles * a.ksplit * a.n_nblk;
  grid = (grid + 7) & ~7;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_stream<EPI, NTB, SEG, WAVES, PS, F8, RT>), dim3(grid), dim3(WAVES * 64), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

// A decoder step routes ~16 rows to an expert: 32-row tiles.  A long prefill chunk routes
// ~64 or more (2,048 tokens: ~128): 128-row tiles, so that an expert's weights are streamed
// once per 128 rows instead of once per 32, with 8 waves per workgroup (measured on the
// 8,192-token prefill: 126 ms against 134 ms with 4 waves and 153 ms with 64-row tiles)
constexpr int kMoeWideTokens = 1024;
int moe_tile_rows(int ntok) { return ntok >= kMoeWideTokens ? 128 : 32; }
int moe_tile_rows_min() { return 32; }
int gemm_lmhead_rows_per_block() { return 256; }   // both LM-head shapes below

hipError_t launch_moe_gateup(const WGemmArgs& a, int tile_rows, hipStream_t s) {
  if (tile_rows == 128) return launch_stream<EPI_SWIGLU, 8, 256, 8, 4>(a, s);
  if (tile_rows != 32) return hipErrorInvalidValue;
  return launch_stream<EPI_SWIGLU, 2, 256, 4, 4>(a, s);
}
hipError_t launch_moe_down(const WGemmArgs& a, int tile_rows, hipStream_t s) {
  if (tile_rows == 128) return launch_stream<EPI_BF16, 8, 256, 8, 4>(a, s);
  if (tile_rows != 32) return hipErrorInvalidValue;
  // a 2-step weight ring: 90 VGPRs, 4 waves per SIMD (87 us against 91 us with 4 steps and
  // 3 waves per SIMD on the decoder shape)
  return launch_stream<EPI_BF16, 2, 256, 4, 2, false, 4>(a, s);
}
// Calls of >= 1,024 tokens (long prefill chunks, batches of four canvases): 128-token tiles halve
// the weight re-reads (183 -> ~160 us per layer at 2,048 tokens), on 8 waves of 32 rows, so a
// CU keeps twice the fragments in flight (8,192-token prefill 101.0 -> 94.6 ms, long-context
// bench step 1,234 -> 1,212 ms against 4 waves, A/B on one box)
hipError_t launch_dense_packed_bf16(const WGemmArgs& a, hipStream_t s) {
  if (a.ntok >= kMoeWideTokens) return launch_stream<EPI_BF16, 8, 256, 8, 4>(a, s);
  return launch_stream<EPI_BF16, 4, 256, 4, 8>(a, s);
}
hipError_t launch_dense_packed_f32(const WGemmArgs& a, hipStream_t s) {
  if (a.ntok >= kMoeWideTokens) return launch_stream<EPI_F32, 8, 256, 8, 4>(a, s);
  return launch_stream<EPI_F32, 8, 256, 4, 4>(a, s);
}
hipError_t launch_lmhead_packed(const WGemmArgs& a, hipStream_t s) {
  return launch_stream<EPI_LMHEAD, 16, 128, 8, 4>(a, s);
}

// e4m3 expert products: 32-row tiles for a decoder step; 128-row tiles on 8 waves once a call
// routes >= 1,024 tokens (a batch of 4 canvases: ~64 rows per expert), as for bf16 weights
hipError_t launch_moe_gateup_fp8(const WGemmArgs& a, int tile_rows, hipStream_t s) {
  if (tile_rows == 128) return launch_stream<EPI_SWIGLU, 8, 512, 8, 4, true>(a, s);
  if (tile_rows != 32) return hipErrorInvalidValue;
  return launch_stream<EPI_SWIGLU, 2, 512, 4, 4, true>(a, s);
}
hipError_t launch_moe_down_fp8(const WGemmArgs& a, int tile_rows, hipStream_t s) {
  if (tile_rows == 128) return launch_stream<EPI_BF16, 8, 512, 8, 4, true>(a, s);
  if (tile_rows != 32) return hipErrorInvalidValue;
  return launch_stream<EPI_BF16, 2, 512, 4, 4, true>(a, s);
}
// 256-token tiles, as for bf16 weights: one weight pass per canvas, 4 for a batch of four (the
// 128-token tiles took 8; long-context bench step 1,298.5 -> 1,290.1 ms, A/B on one box)
hipError_t launch_lmhead_packed_fp8(const WGemmArgs& a, hipStream_t s) {
  return launch_stream<EPI_LMHEAD, 16, 256, 8, 4, true>(a, s);
}

hipError_t launch_pack(const void* src, void* dst, long long rows, long long cols, hipStream_t s) {
  const long long frags = (rows / 16) * (cols / 32);
  if (frags == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack, dim3(static_cast<unsigned>((frags + 3) / 4)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), rows, cols);
  return hipGetLastError();
}

}  // namespace dg
