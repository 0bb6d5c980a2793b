// Canvas attention: every canvas query attends, in one softmax, to the visible cached keys and
// to the canvas keys (DiffusionGemma model card, "Model overview": bidirectional attention over
// the canvas plus cross-attention to the cached context; the encoder reads a finished canvas
// causally).  GQA: query head h reads KV head floor(h * Hkv / Hq); scale 1/sqrt(head_dim).
// Sliding-window layers: canvas query i at absolute position len + i sees cache position j
// only if (len + i) - j < window (model card dimension table: 1,024-token window).
//
// Layout of the work: one workgroup = (canvas b, KV head g, 128 query rows, one split of the
// key range).  The query rows of a KV head are its Hq/Hkv query heads
// times the canvas positions, so the K/V tiles staged in LDS serve every query head that reads
// them.  Keys are processed in tiles of 64 (K and V tiles [key][dh] in LDS, double buffered: tile
// t + 1 is staged while tile t is computed, one barrier per tile).
// Up to head_dim 128 there are 4 waves (one per SIMD), each holding 32 query rows as two 16-row
// MFMA tiles, so every K and V^T fragment read from LDS feeds two MFMAs; at head_dim 256 the
// registers hold one 16-row tile per wave and there are 8 waves.  Each wave computes S^T = K Q^T, so the probabilities come out of the MFMA in the
// lane layout that the P V product takes as its B operand (O^T = V^T P^T) with no shuffle.
// Staging loads are coalesced (consecutive lanes on consecutive 16-byte pieces of a key row) and
// both tiles are stored row-major with 16-byte stores; the V^T fragments of the P V product come
// from CDNA4's transposing LDS read, 8 keys of one dh per lane from two 8-byte reads.  LDS rows
// are padded to a stride at which the 16-byte K reads and the transposing V reads run at the
// full LDS rate.  Splits of the key range write unnormalised partial outputs (bf16) with their
// running max and sum (fp32), merged afterwards by log-sum-exp.
#include "dg_internal.h"

#include <type_traits>

namespace dg {
namespace {

constexpr int KT = 64;               // keys per tile
constexpr int QB = 128;              // query rows per workgroup

template <int DH>
struct AttnCfg {
  static constexpr int QT = DH >= 256 ? 1 : 2;  // 16-row query tiles per wave
  static constexpr int NWAVE = QB / (16 * QT);  // waves per workgroup
  static constexpr int NTHR = NWAVE * 64;
  static constexpr int KS_STRIDE = DH + 16;  // bf16 per K or V row in LDS
  static constexpr int NKS = (DH + 31) / 32; // 32-wide dh steps of QK^T
  static constexpr int NDT = DH / 16;        // 16-row dh tiles of O^T
  static constexpr int KBUF = KT * KS_STRIDE;
  static constexpr int KCH = DH / 8;         // 16-byte pieces per key row
  // staging: piece p = t + j * NTHR (j < PIT) of thread t is chunk p % KCH of key p / KCH
  static constexpr int NPC = KT * KCH;       // pieces per tile (K or V)
  static constexpr int PIT = (NPC + NTHR - 1) / NTHR;
  static constexpr int RING = 8 / QT;  // fragment ring depth: 8 MFMAs of cover
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// CDNA4 transposing LDS read of 16-bit data: within each group of 16 lanes, lane 4a + b receives
// element b of the 8-byte pieces addressed by lanes a, a + 4, a + 8 and a + 12 (in that order)
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// the maximum and the sum of x over lanes l, l ^ 16, l ^ 32 and l ^ 48, with the CDNA4 lane
// swaps (each returns x of lane l and of lane l ^ 32, resp. l ^ 16, as a pair), on the VALU
// rather than through the LDS crossbar
__device__ __forceinline__ float lanes_max4(float x) {
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
  x = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
  return fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
}
__device__ __forceinline__ float lanes_sum4(float x) {
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
  x = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
  return __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
}

template <int DH>
__global__ __launch_bounds__(AttnCfg<DH>::NTHR) void k_attn(AttnArgs a) {
  using C = AttnCfg<DH>;
  constexpr int QT = C::QT, NTHR = C::NTHR;
  __shared__ __align__(16) uint16_t ks[2][C::KBUF];
  __shared__ __align__(16) uint16_t vs[2][C::KBUF];

  // logical block -> (canvas, KV head, key split, query block); the query blocks that share a
  // KV head and split are consecutive, so they run on one XCD and share its L2 for K/V tiles
  const int R = (a.Hq / a.Hkv) * a.C;
  const int n_qblk = (R + QB - 1) / QB;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int qblk = L % n_qblk;
  int rest = L / n_qblk;
  const int split = rest % a.n_split;
  rest /= a.n_split;
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;
  if (b >= a.B) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, lg = lane >> 4;
  const int hpg = a.Hq / a.Hkv;
  const int ldqkv = (a.Hq + 2 * a.Hkv) * DH;

  const int len = a.len[b];
  const int c_lo = a.window > 0 ? max(0, len - a.window + 1) : 0;
  const int nc = len - c_lo;           // cache keys in the union of the visible ranges
  const int nk = nc + a.C;             // + canvas keys
  const int ntiles = (nk + KT - 1) / KT;
  const int per = (ntiles + a.n_split - 1) / a.n_split;
  const int t_beg = split * per;
  const int t_end = min(ntiles, t_beg + per);

  // this lane's query rows (B operand columns), one per query tile
  int r[QT], qi[QT], h[QT], win_lo[QT];
  bool r_ok[QT];
  long long qrow[QT];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  u32x4 qf[C::NKS][QT];
#pragma unroll
  for (int q = 0; q < QT; ++q) {
    r[q] = qblk * QB + wave * 16 * QT + q * 16 + r16;
    r_ok[q] = r[q] < R;
    const int rr = r_ok[q] ? r[q] : R - 1;
    const int hl = rr / a.C;
    qi[q] = rr % a.C;
    h[q] = g * hpg + hl;
    qrow[q] = static_cast<long long>(b) * a.C + qi[q];
    win_lo[q] = len + qi[q] - a.window + 1;   // first visible cache position (windowed layers)
    const uint16_t* qp = a.qkv + qrow[q] * ldqkv + h[q] * DH;
#pragma unroll
    for (int ks_ = 0; ks_ < C::NKS; ++ks_) {
      const int d0 = ks_ * 32 + lg * 8;
      qf[ks_][q] = (d0 < DH) ? ld16(qp + d0) : zero4;
    }
  }

  f32x4 o[C::NDT][QT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int q = 0; q < QT; ++q) o[dt][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int q = 0; q < QT; ++q) {
    m_run[q] = -INFINITY;
    l_run[q] = 0.f;
  }

  const uint16_t* kcache = a.kc + (static_cast<long long>(b) * a.Hkv + g) * a.cap * DH;
  const uint16_t* vcache = a.vc + (static_cast<long long>(b) * a.Hkv + g) * a.cap * DH;
  const uint16_t* kcanvas = a.qkv + static_cast<long long>(b) * a.C * ldqkv + (a.Hq + g) * DH;
  const uint16_t* vcanvas = kcanvas + a.Hkv * DH;

  // wave-uniform range of this wave's canvas positions (tiles that no query of the wave sees
  // partially are processed without per-element masks)
  int qi_lo = qi[0], qi_hi = qi[0];
#pragma unroll
  for (int q = 1; q < QT; ++q) {
    qi_lo = min(qi_lo, qi[q]);
    qi_hi = max(qi_hi, qi[q]);
  }
#pragma unroll
  for (int o2 = 1; o2 < 64; o2 <<= 1) {
    qi_lo = min(qi_lo, __shfl_xor(qi_lo, o2, 64));
    qi_hi = max(qi_hi, __shfl_xor(qi_hi, o2, 64));
  }
  qi_lo = __builtin_amdgcn_readfirstlane(qi_lo);
  qi_hi = __builtin_amdgcn_readfirstlane(qi_hi);

  // staging: K of the next tile is fetched before this tile's S^T and stored after it; V of the
  // next tile is fetched then and stored after the P V product.  Every load is unconditional: a
  // key past the range reads the last key of the range (finite data whose scores are masked to
  // -inf, so its probability is 0), and the cache or canvas row is chosen by bit arithmetic on
  // both (clamped) addresses, so no branch makes the compiler wait for loads in flight
  auto kv_row = [&](int kk, const uint16_t* cache, const uint16_t* canvas) -> const uint16_t* {
    const int kc = min(kk, nk - 1);
    const uintptr_t pc = reinterpret_cast<uintptr_t>(
        cache + static_cast<long long>(c_lo + max(min(kc, nc - 1), 0)) * DH);
    const uintptr_t pn = reinterpret_cast<uintptr_t>(
        canvas + static_cast<long long>(max(kc - nc, 0)) * ldqkv);
    const uintptr_t m = -static_cast<uintptr_t>(kc < nc);
    return reinterpret_cast<const uint16_t*>((pc & m) | (pn & ~m));
  };
  constexpr bool PFULL = C::NPC % NTHR == 0;   // every thread has all its pieces
  int p_key[C::PIT], p_off[C::PIT];            // piece -> key in the tile, offset in a row
#pragma unroll
  for (int it = 0; it < C::PIT; ++it) {
    const int pc = min(tid + it * NTHR, C::NPC - 1);
    p_key[it] = pc / C::KCH;
    p_off[it] = (pc % C::KCH) * 8;
  }
  u32x4 pk[C::PIT], pv[C::PIT];
  auto fetch_k = [&](int tt) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < C::PIT; ++it)
      pk[it] = ld16(kv_row(tt * KT + p_key[it], kcache, kcanvas) + p_off[it]);
  };
  auto fetch_v = [&](int tt) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < C::PIT; ++it)
      pv[it] = ld16(kv_row(tt * KT + p_key[it], vcache, vcanvas) + p_off[it]);
  };
  auto stage = [&](uint16_t* dst, const u32x4 (&pr)[C::PIT]) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < C::PIT; ++it) {
      if (!PFULL && tid + it * NTHR >= C::NPC) continue;
      st16(dst + p_key[it] * C::KS_STRIDE + p_off[it], pr[it]);
    }
  };
  auto stage_k = [&](int buf) __attribute__((always_inline)) { stage(ks[buf], pk); };
  auto stage_v = [&](int buf) __attribute__((always_inline)) { stage(vs[buf], pv); };

  const float sc = a.scale_log2e;
  if (t_beg < t_end) {
    fetch_k(t_beg);
    fetch_v(t_beg);
    stage_k(0);
    stage_v(0);
  }
  // the query fragments, opaque to the compiler from here on (after the first tile's loads are
  // issued, so that all of them overlap): they stay in registers for the whole key range instead
  // of being re-loaded in every tile
#pragma unroll
  for (int q = 0; q < QT; ++q)
#pragma unroll
    for (int ks_ = 0; ks_ < C::NKS; ++ks_) asm volatile("" : "+v"(qf[ks_][q]));
  __syncthreads();
  // one key tile; STAGE: also stage tile tt + 1 into the other buffers.  Every tile but the last
  // stages, so the loop body is straight-line code (a branch around the staging would make the
  // compiler wait for the next tile's loads as soon as they are issued)
  auto tile = [&](int tt, auto stage_tag) __attribute__((always_inline)) {
    constexpr bool STAGE = decltype(stage_tag)::value;
    const int kbase = tt * KT;
    const int cur = (tt - t_beg) & 1;
    const uint16_t* ksb = ks[cur];
    const uint16_t* vsb = vs[cur];
    if constexpr (STAGE) fetch_k(tt + 1);

    // S^T[key][q] for 4 sub-tiles of 16 keys and the wave's query tiles (raw dot products).  The
    // K fragments run ks-major through a ring read from LDS RING fragments ahead of use (pinned
    // by scheduling barriers); each fragment feeds the MFMAs of every query tile
    constexpr int NS = 4 * C::NKS;
    auto kfrag = [&](int i) -> u32x4 {
      const int d0 = (i / 4) * 32 + lg * 8;
      return (d0 < DH) ? ld16(ksb + ((i % 4) * 16 + r16) * C::KS_STRIDE + d0) : zero4;
    };
    f32x4 s[QT][4];
#pragma unroll
    for (int q = 0; q < QT; ++q)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) s[q][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int KR = C::RING < NS ? C::RING : NS;
    u32x4 kr[KR];
#pragma unroll
    for (int i = 0; i < KR; ++i) kr[i] = kfrag(i);
    // a wave in an MFMA loop takes issue priority over the wave sharing its SIMD, which is then
    // left to its softmax (measured: 2% faster at head_dim 256)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
#pragma unroll
      for (int q = 0; q < QT; ++q) s[q][i % 4] = mfma16x16x32(kr[i % KR], qf[i / 4][q], s[q][i % 4]);
      if (i + KR < NS) kr[i % KR] = kfrag(i + KR);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (STAGE) {
      stage_k(cur ^ 1);   // the other buffer was last read before the previous barrier
      fetch_v(tt + 1);
    }
    // the first V^T fragments of the P V product, read while the softmax below runs
    // V^T fragment (dh tile i % NDT, key half kp = i / NDT): lane (dh r16, group lg) gets V at
    // keys 32 kp + 4 lg + 0..3 and 32 kp + 16 + 4 lg + 0..3, the keys (in that order) of its P
    // fragment; lane r16 of the group addresses key row 4 lg + r16 / 4 (+ 16), columns
    // 16 (i % NDT) + 4 (r16 % 4) .. + 3
    constexpr int NP = 2 * C::NDT;
    const uint16_t* vlane = vsb + (4 * lg + (r16 >> 2)) * C::KS_STRIDE + 4 * (r16 & 3);
    auto vfrag = [&](int i) -> u32x4 {
      const uint16_t* p = vlane + (i / C::NDT) * 32 * C::KS_STRIDE + (i % C::NDT) * 16;
      const s16x4 lo = lds_read_tr16(p);
      const s16x4 hi = lds_read_tr16(p + 16 * C::KS_STRIDE);
      return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int VR = C::RING < NP ? C::RING : NP;
    u32x4 vr[VR];
#pragma unroll
    for (int i = 0; i < VR; ++i) vr[i] = vfrag(i);
    // visibility: a tile inside the canvas or inside the cache that every query of this wave
    // sees entirely needs no per-element mask (the lane's keys: nt*16 + 4 lg + j)
    const bool in_cache = kbase + KT <= nc;
    const bool full =
        kbase + KT <= nk &&
        (in_cache ? (a.window == 0 || c_lo + kbase >= len + qi_hi - a.window + 1)
                  : (kbase >= nc && (!a.causal || kbase + KT - 1 - nc <= qi_lo)));
    u32x4 pb[QT][2];
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      float tmax = -INFINITY;
      if (full) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          tmax = fmaxf(tmax, fmaxf(fmaxf(s[q][nt][0], s[q][nt][1]), fmaxf(s[q][nt][2], s[q][nt][3])));
      } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kk = kbase + nt * 16 + 4 * lg + j;
            bool vis = kk < nk;
            if (kk < nc) {
              if (a.window > 0) vis = vis && (c_lo + kk >= win_lo[q]);
            } else if (a.causal) {
              vis = vis && (kk - nc <= qi[q]);
            }
            s[q][nt][j] = vis ? s[q][nt][j] : -INFINITY;
            tmax = fmaxf(tmax, s[q][nt][j]);
          }
        }
      }
      tmax = lanes_max4(tmax);
      // running max in scaled (log2) units; the scale is > 0, so it commutes with the max
      const float m_new = fmaxf(m_run[q], tmax * sc);
      const float neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[q] + neg_m);   // m_run = -inf: 0
      m_run[q] = m_new;
      // rescale only when some lane's maximum moved (a wave-uniform branch)
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
        l_run[q] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) o[dt][q] *= alpha;
      }
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        f32x4 lo, hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[q][2 * kp][j], sc, neg_m));
          hi[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[q][2 * kp + 1][j], sc, neg_m));
        }
        l_run[q] += (lo[0] + lo[1]) + (lo[2] + lo[3]) + (hi[0] + hi[1]) + (hi[2] + hi[3]);
        pb[q][kp] = u32x4{cvt_pk_bf16(lo[0], lo[1]), cvt_pk_bf16(lo[2], lo[3]),
                          cvt_pk_bf16(hi[0], hi[1]), cvt_pk_bf16(hi[2], hi[3])};
      }
    }
    // O^T[dh][q] += V^T[dh][keys] P^T[keys][q]; the B operand's 8 keys per lane are
    // {32 kp + 4 lg + 0..3, 32 kp + 16 + 4 lg + 0..3}.  kp-major V^T fragment ring; each
    // fragment feeds every query tile
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
#pragma unroll
      for (int q = 0; q < QT; ++q)
        o[i % C::NDT][q] = mfma16x16x32(vr[i % VR], pb[q][i / C::NDT], o[i % C::NDT][q]);
      if (i + VR < NP) vr[i % VR] = vfrag(i + VR);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (STAGE) stage_v(cur ^ 1);
    __syncthreads();
  };
  for (int tt = t_beg; tt + 1 < t_end; ++tt) tile(tt, std::true_type{});
  if (t_beg < t_end) tile(t_end - 1, std::false_type{});

#pragma unroll
  for (int q = 0; q < QT; ++q) {
    // row sum over the 4 lanes that share this query
    const float l = lanes_sum4(l_run[q]);
    if (!r_ok[q]) continue;
    if (a.n_split == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* op = a.out + qrow[q] * (a.Hq * DH) + h[q] * DH;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        uint2 pk2;
        pk2.x = pack_bf2(o[dt][q][0] * inv, o[dt][q][1] * inv);
        pk2.y = pack_bf2(o[dt][q][2] * inv, o[dt][q][3] * inv);
        *reinterpret_cast<uint2*>(op + dt * 16 + 4 * lg) = pk2;
      }
    } else {
      const long long prow = ((static_cast<long long>(split) * a.B + b) * a.Hkv + g) * R + r[q];
      // unnormalised partial rows in bf16 (one rounding, well inside the output's own)
      uint16_t* op = a.o_part + prow * DH;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        uint2 pk2;
        pk2.x = pack_bf2(o[dt][q][0], o[dt][q][1]);
        pk2.y = pack_bf2(o[dt][q][2], o[dt][q][3]);
        *reinterpret_cast<uint2*>(op + dt * 16 + 4 * lg) = pk2;
      }
      if (lg == 0) {
        a.ml_part[prow * 2] = m_run[q];
        a.ml_part[prow * 2 + 1] = l;
      }
    }
  }
}

// merge of split partials: one thread per (query row, 4 dh values).  Splits are merged in split
// order, 8 at a time: each group's running maxima, sums and partial rows are loaded together
// (clamped split index, zero weight past the last split), so up to 8 splits cost one memory
// round trip; the result so far is rescaled when a later group raises the maximum.
template <int DH>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const int hpg = a.Hq / a.Hkv;
  const int R = hpg * a.C;
  const long long rows = static_cast<long long>(a.B) * a.Hkv * R;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = DH / 4;
  if (idx >= rows * per_row) return;
  const long long row = idx / per_row;  // (b, g, r)
  const int c4 = static_cast<int>(idx % per_row) * 4;
  const long long stride = rows;        // rows per split
  float mmax = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp0 = 0; sp0 < a.n_split; sp0 += 8) {
    float2 ml[8];
    uint2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const long long r2 = static_cast<long long>(min(sp0 + u, a.n_split - 1)) * stride + row;
      ml[u] = *reinterpret_cast<const float2*>(a.ml_part + r2 * 2);
      v[u] = *reinterpret_cast<const uint2*>(a.o_part + r2 * DH + c4);
    }
    float gmax = mmax;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (sp0 + u < a.n_split) gmax = fmaxf(gmax, ml[u].x);
    if (gmax != mmax) {   // a later group raised the maximum: rescale what is merged so far
      const float r = (mmax == -INFINITY) ? 0.f : exp2f(mmax - gmax);
      l *= r;
      acc.x *= r;
      acc.y *= r;
      acc.z *= r;
      acc.w *= r;
      mmax = gmax;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (sp0 + u < a.n_split) {  // uniform; the loads above are already in flight
        const float m = ml[u].x;
        const float w = (m == -INFINITY) ? 0.f : exp2f(m - mmax);
        l += w * ml[u].y;
        acc.x += w * __uint_as_float(v[u].x << 16);
        acc.y += w * __uint_as_float(v[u].x & 0xffff0000u);
        acc.z += w * __uint_as_float(v[u].y << 16);
        acc.w += w * __uint_as_float(v[u].y & 0xffff0000u);
      }
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int r = static_cast<int>(row % R);
  const long long bg = row / R;
  const int g = static_cast<int>(bg % a.Hkv), b = static_cast<int>(bg / a.Hkv);
  const int hl = r / a.C, qi = r % a.C;
  const int h = g * hpg + hl;
  uint16_t* op = a.out + (static_cast<long long>(b) * a.C + qi) * (a.Hq * DH) + h * DH + c4;
  uint2 pk;
  pk.x = pack_bf2(acc.x * inv, acc.y * inv);
  pk.y = pack_bf2(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2*>(op) = pk;
}

template <int DH>
hipError_t launch_dh(const AttnArgs& a, hipStream_t s) {
  const int R = (a.Hq / a.Hkv) * a.C;
  int grid = ((R + QB - 1) / QB) * a.Hkv * a.B * a.n_split;
  grid = (grid + 7) & ~7;
  hipLaunchKernelGGL(k_attn<DH>, dim3(grid), dim3(AttnCfg<DH>::NTHR), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const long long n = static_cast<long long>(a.B) * a.Hkv * R * (DH / 4);
  hipLaunchKernelGGL(k_attn_merge<DH>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace

int attention_pick_split(int B, int C, int Hq, int Hkv, int max_keys) {
  const int R = (Hq / Hkv) * C;
  const int base = B * Hkv * ((R + QB - 1) / QB);
  const int ntiles = (max_keys + KT - 1) / KT;
  int n = (256 + base - 1) / base;
  n = std::min(n, std::max(1, ntiles / 2));
  n = std::min(n, std::max(1, 1024 / base));
  return std::max(1, n);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  switch (a.dh) {
    case 16: return launch_dh<16>(a, s);
    case 32: return launch_dh<32>(a, s);
    case 64: return launch_dh<64>(a, s);
    case 128: return launch_dh<128>(a, s);
    case 256: return launch_dh<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dg
