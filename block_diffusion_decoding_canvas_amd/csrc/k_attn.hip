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
// Up to head_dim 128 (the generic kernel) there are 4 waves (one per SIMD), each holding 32 query
// rows as two 16-row MFMA tiles, so every K and V^T fragment read from LDS feeds two MFMAs; each
// wave computes S^T = K Q^T, so the probabilities come out of the MFMA in the lane layout that
// the P V product takes as its B operand (O^T = V^T P^T) with no shuffle.  Head_dim 256 has a
// kernel of its own (score waves and P V waves, below).
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
  static_assert(DH <= 128, "head_dim 256 runs the score / P V kernel");
  static constexpr int QT = 2;                  // 16-row query tiles per wave
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

// fp8 KV cache: K tiles are e4m3 bytes in LDS (S^T = K Q^T on the 16x16x128 e4m3 MFMA, Q
// quantised per query row in the prologue), V tiles are converted to bf16 as they are staged
// (exact) and P V stays on the bf16 MFMA, with the value row scales applied to P
template <int DH>
struct AttnF8Cfg {
  static constexpr int K8S = DH + 32;        // bytes per K row in LDS (stride / 16 = 2 mod 4)
  static constexpr int NKB = DH / 128;       // 128-wide dh blocks of QK^T
  static constexpr int PCH = DH / 16;        // 16-byte pieces (16 values) per key row
  static constexpr int NPC = KT * PCH;       // pieces per tile
  static constexpr int PIT = (NPC + AttnCfg<DH>::NTHR - 1) / AttnCfg<DH>::NTHR;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// CDNA4 transposing LDS read of 16-bit data: within each group of 16 lanes, lane 4a + b receives
// element b of the 8-byte pieces addressed by lanes a, a + 4, a + 8 and a + 12 (in that order)
// streaming (non-temporal) 16-byte load for the bf16 K/V tiles of the head_dim-256 kernel: a step
// reads each cached row once, and with the hint the 67 MB of cache rows of a layer stop displacing
// the rows other kernels re-read from L2 (a decoder step measured 11.81 against 11.91 ms).  The
// e4m3 tiles keep plain loads: on 4 x 131,072-key caches the hint cost 1% of attention time
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

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

template <int DH, bool F8>
__global__ __launch_bounds__(AttnCfg<DH>::NTHR) void k_attn(AttnArgs a) {
  using C = AttnCfg<DH>;
  using C8 = AttnF8Cfg<DH>;
  constexpr int QT = C::QT, NTHR = C::NTHR;
  __shared__ __align__(16) uint16_t ks[2][F8 ? 8 : C::KBUF];
  __shared__ __align__(16) uint8_t ks8[2][F8 ? KT * C8::K8S : 16];
  __shared__ __align__(16) float sks[2][F8 ? KT : 4];   // fp8: key row scales of the tile
  __shared__ __align__(16) float svs[2][F8 ? KT : 4];   // fp8: value row scales of the tile
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
  int ntiles = (nk + KT - 1) / KT;
  if (a.causal) {
    // the block's last canvas position: canvas keys past it are masked for every query of the
    // block, so their tiles are not visited (the rows of a block are consecutive positions of
    // one query head unless the block straddles two heads)
    const int r0 = qblk * QB, r1 = min(R, r0 + QB) - 1;
    const int qmax = (r0 / a.C == r1 / a.C) ? r1 % a.C : a.C - 1;
    ntiles = min(ntiles, (nc + qmax + 1 + KT - 1) / KT);
  }
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
    if constexpr (!F8) {
#pragma unroll
      for (int ks_ = 0; ks_ < C::NKS; ++ks_) {
        const int d0 = ks_ * 32 + lg * 8;
        qf[ks_][q] = (d0 < DH) ? ld16(qp + d0) : zero4;
      }
    }
  }
  // fp8: the query row's e4m3 codes with its scale amax / 448 (decided in binary32); lane
  // (r16, lg) holds dh 128 kb + 16 lg + [0, 16) and 128 kb + 64 + 16 lg + [0, 16) of its row for
  // every 128-wide block kb (the MFMA only needs the K fragments in the same k order; this one
  // makes each 16-byte K read a 16-byte lane stride, as in the bf16 kernel)
  u32x4 qf8[F8 ? C8::NKB : 1][QT][2];
  float sq[QT];
  if constexpr (F8) {
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      const uint16_t* qp = a.qkv + qrow[q] * ldqkv + h[q] * DH;
      u32x4 raw[C8::NKB][4];
      float amax = 0.f;
#pragma unroll
      for (int kb = 0; kb < C8::NKB; ++kb)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          raw[kb][m] = ld16(qp + 128 * kb + (m >> 1) * 64 + 16 * lg + 8 * (m & 1));
#pragma unroll
          for (int w = 0; w < 4; ++w)
            amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(raw[kb][m][w] << 16)),
                                     fabsf(__uint_as_float(raw[kb][m][w] & 0xffff0000u))));
        }
      amax = lanes_max4(amax);
      sq[q] = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
      for (int kb = 0; kb < C8::NKB; ++kb)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // 8 bf16 -> 8 codes (2 dwords) of the 32-byte fragment
          uint32_t c[4];
#pragma unroll
          for (int w = 0; w < 4; ++w)
            c[w] = f2e4m3(__uint_as_float(raw[kb][m][w] << 16) / sq[q]) |
                   (f2e4m3(__uint_as_float(raw[kb][m][w] & 0xffff0000u) / sq[q]) << 8);
          const uint32_t lo = c[0] | (c[1] << 16), hi = c[2] | (c[3] << 16);
          u32x4& dst = qf8[kb][q][m >> 1];
          if (m & 1) {
            dst.z = lo;
            dst.w = hi;
          } else {
            dst.x = lo;
            dst.y = hi;
          }
        }
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

  const uint16_t* kcache = a.kc + (static_cast<long long>(a.kvb[b]) * a.Hkv + g) * a.cap * DH;
  const uint16_t* vcache = a.vc + (static_cast<long long>(a.kvb[b]) * a.Hkv + g) * a.cap * DH;
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
  // K pieces: 16 bytes of a key row (8 bf16, or 16 e4m3 codes).  V pieces: 8 values of a row (16
  // bf16 bytes, or 8 e4m3 codes that become 16 bf16 bytes in LDS, so that consecutive lanes store
  // consecutive 16-byte pieces either way)
  constexpr int PIT = F8 ? C8::PIT : C::PIT;
  constexpr int NPC = F8 ? C8::NPC : C::NPC;
  constexpr int PCH = F8 ? C8::PCH : C::KCH;   // K pieces per key row
  constexpr bool PFULL = NPC % NTHR == 0;      // every thread has all its K pieces
  constexpr bool VFULL = C::NPC % NTHR == 0;   // ... and all its V pieces
  // piece -> key in the tile and its first dh
  int p_key[PIT], p_off[PIT], v_key[C::PIT], v_off[C::PIT];
#pragma unroll
  for (int it = 0; it < PIT; ++it) {
    const int pc = min(tid + it * NTHR, NPC - 1);
    p_key[it] = pc / PCH;
    p_off[it] = (pc % PCH) * (F8 ? 16 : 8);
  }
#pragma unroll
  for (int it = 0; it < C::PIT; ++it) {
    const int pc = min(tid + it * NTHR, C::NPC - 1);
    v_key[it] = pc / C::KCH;
    v_off[it] = (pc % C::KCH) * 8;
  }
  // fp8: rows of e4m3 codes (cache, or the call's quantised canvas rows) and their scales
  const uint8_t* kcache8 = reinterpret_cast<const uint8_t*>(a.kc) +
                           (static_cast<long long>(a.kvb[b]) * a.Hkv + g) * a.cap * DH;
  const uint8_t* vcache8 = reinterpret_cast<const uint8_t*>(a.vc) +
                           (static_cast<long long>(a.kvb[b]) * a.Hkv + g) * a.cap * DH;
  const float* kcs = a.ksc + (static_cast<long long>(a.kvb[b]) * a.Hkv + g) * a.cap;
  const float* vcs = a.vsc + (static_cast<long long>(a.kvb[b]) * a.Hkv + g) * a.cap;
  const long long cq0 = static_cast<long long>(b) * a.C * a.Hkv + g;   // canvas row (i = 0)
  auto kv_row8 = [&](int kk, const uint8_t* cache, const uint8_t* canvas) -> const uint8_t* {
    const int kc = min(kk, nk - 1);
    const uintptr_t pc = reinterpret_cast<uintptr_t>(
        cache + static_cast<long long>(c_lo + max(min(kc, nc - 1), 0)) * DH);
    const uintptr_t pn = reinterpret_cast<uintptr_t>(
        canvas + (cq0 + static_cast<long long>(max(kc - nc, 0)) * a.Hkv) * DH);
    const uintptr_t m = -static_cast<uintptr_t>(kc < nc);
    return reinterpret_cast<const uint8_t*>((pc & m) | (pn & ~m));
  };
  auto row_scale = [&](int kk, const float* cache, const float* canvas) -> float {
    const int kc = min(kk, nk - 1);
    const uintptr_t pc = reinterpret_cast<uintptr_t>(cache + c_lo + max(min(kc, nc - 1), 0));
    const uintptr_t pn = reinterpret_cast<uintptr_t>(
        canvas + cq0 + static_cast<long long>(max(kc - nc, 0)) * a.Hkv);
    const uintptr_t m = -static_cast<uintptr_t>(kc < nc);
    return *reinterpret_cast<const float*>((pc & m) | (pn & ~m));
  };
  u32x4 pk[PIT], pv[C::PIT];
  uint2 pv8[F8 ? C::PIT : 1];
  float pks = 0.f, pvsc = 0.f;                 // fp8: thread t < KT stages key t's scales
  auto fetch_k = [&](int tt) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < PIT; ++it) {
      if constexpr (F8)
        pk[it] = ld16(kv_row8(tt * KT + p_key[it], kcache8, a.kq) + p_off[it]);
      else
        pk[it] = ld16(kv_row(tt * KT + p_key[it], kcache, kcanvas) + p_off[it]);
    }
    if constexpr (F8) {
      if (tid < KT) pks = row_scale(tt * KT + tid, kcs, a.kqs);
    }
  };
  auto fetch_v = [&](int tt) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < C::PIT; ++it) {
      if constexpr (F8)
        pv8[it] = *reinterpret_cast<const uint2*>(
            kv_row8(tt * KT + v_key[it], vcache8, a.vq) + v_off[it]);
      else
        pv[it] = ld16(kv_row(tt * KT + v_key[it], vcache, vcanvas) + v_off[it]);
    }
    if constexpr (F8) {
      if (tid < KT) pvsc = row_scale(tt * KT + tid, vcs, a.vqs);
    }
  };
  auto stage = [&](uint16_t* dst, const u32x4 (&pr)[C::PIT], const int (&key)[C::PIT],
                   const int (&off)[C::PIT]) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < C::PIT; ++it) {
      if (!VFULL && tid + it * NTHR >= C::NPC) continue;
      st16(dst + key[it] * C::KS_STRIDE + off[it], pr[it]);
    }
  };
  auto stage_k = [&](int buf) __attribute__((always_inline)) {
    if constexpr (F8) {
#pragma unroll
      for (int it = 0; it < PIT; ++it) {
        if (!PFULL && tid + it * NTHR >= NPC) continue;
        st16(&ks8[buf][p_key[it] * C8::K8S + p_off[it]], pk[it]);
      }
      if (tid < KT) sks[buf][tid] = pks;
    } else {
      stage(ks[buf], pk, p_key, p_off);
    }
  };
  auto stage_v = [&](int buf) __attribute__((always_inline)) {
    if constexpr (F8) {
      // 8 codes of one key row -> their values in bf16 (exact: an e4m3 value has 4 significant
      // bits); the row's scale is applied to the probabilities instead
#pragma unroll
      for (int it = 0; it < C::PIT; ++it) {
        if (!VFULL && tid + it * NTHR >= C::NPC) continue;
        uint32_t w[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int x = static_cast<int>(h2 ? pv8[it].y : pv8[it].x);
          w[2 * h2] = __builtin_bit_cast(
              uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
          w[2 * h2 + 1] = __builtin_bit_cast(
              uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
        }
        st16(vs[buf] + v_key[it] * C::KS_STRIDE + v_off[it], u32x4{w[0], w[1], w[2], w[3]});
      }
      if (tid < KT) svs[buf][tid] = pvsc;
    } else {
      stage(vs[buf], pv, v_key, v_off);
    }
  };

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
  for (int q = 0; q < QT; ++q) {
    if constexpr (F8) {
#pragma unroll
      for (int kb = 0; kb < C8::NKB; ++kb) {
        asm volatile("" : "+v"(qf8[kb][q][0]));
        asm volatile("" : "+v"(qf8[kb][q][1]));
      }
    } else {
#pragma unroll
      for (int ks_ = 0; ks_ < C::NKS; ++ks_) asm volatile("" : "+v"(qf[ks_][q]));
    }
  }
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
    f32x4 s[QT][4];
#pragma unroll
    for (int q = 0; q < QT; ++q)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) s[q][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (F8) {
      // S^T on the 16x16x128 e4m3 MFMA: fragment i = (dh block i / 4, key sub-tile i % 4), 32
      // bytes per lane from two 16-byte LDS reads (dh 16 lg + [0, 16) and 64 + 16 lg + [0, 16)
      // of the block, the query fragments' order); then each raw product is scaled by its key's
      // row scale (the query's scale is folded into the softmax multiplier below)
      constexpr int NS8 = 4 * C8::NKB;
      const uint8_t* k8b = ks8[cur] + r16 * C8::K8S + 16 * lg;
      u32x4 kr8[NS8][2];
#pragma unroll
      for (int i = 0; i < NS8; ++i) {
        const uint8_t* p = k8b + (i % 4) * 16 * C8::K8S + (i / 4) * 128;
        kr8[i][0] = ld16(p);
        kr8[i][1] = ld16(p + 64);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < NS8; ++i)
#pragma unroll
        for (int q = 0; q < QT; ++q)
          s[q][i % 4] = mfma_f8_128(kr8[i][0], kr8[i][1], qf8[i / 4][q][0], qf8[i / 4][q][1],
                                    s[q][i % 4]);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float4 skv = *reinterpret_cast<const float4*>(&sks[cur][nt * 16 + 4 * lg]);
#pragma unroll
        for (int q = 0; q < QT; ++q) {
          s[q][nt][0] *= skv.x;
          s[q][nt][1] *= skv.y;
          s[q][nt][2] *= skv.z;
          s[q][nt][3] *= skv.w;
        }
      }
    } else {
      constexpr int NS = 4 * C::NKS;
      auto kfrag = [&](int i) -> u32x4 {
        const int d0 = (i / 4) * 32 + lg * 8;
        return (d0 < DH) ? ld16(ksb + ((i % 4) * 16 + r16) * C::KS_STRIDE + d0) : zero4;
      };
      constexpr int KR = C::RING < NS ? C::RING : NS;
      u32x4 kr[KR];
#pragma unroll
      for (int i = 0; i < KR; ++i) kr[i] = kfrag(i);
      // a wave in an MFMA loop takes issue priority over a wave sharing its SIMD, which is then
      // left to its softmax
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
#pragma unroll
        for (int q = 0; q < QT; ++q)
          s[q][i % 4] = mfma16x16x32(kr[i % KR], qf[i / 4][q], s[q][i % 4]);
        if (i + KR < NS) kr[i % KR] = kfrag(i + KR);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
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
    // fp8: the value row scales of this lane's keys (nt*16 + 4 lg + j), applied to P
    float4 svk[4];
    if constexpr (F8) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        svk[nt] = *reinterpret_cast<const float4*>(&svs[cur][nt * 16 + 4 * lg]);
    }
    u32x4 pb[QT][2];
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      // fp8: the query row's scale joins the softmax multiplier (it is > 0, so the max commutes)
      float scq = sc;
      if constexpr (F8) scq = sc * sq[q];
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
      const float m_new = fmaxf(m_run[q], tmax * scq);
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
          lo[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[q][2 * kp][j], scq, neg_m));
          hi[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[q][2 * kp + 1][j], scq, neg_m));
        }
        l_run[q] += (lo[0] + lo[1]) + (lo[2] + lo[3]) + (hi[0] + hi[1]) + (hi[2] + hi[3]);
        if constexpr (F8) {
          const float4 a0 = svk[2 * kp], a1 = svk[2 * kp + 1];
          lo[0] *= a0.x; lo[1] *= a0.y; lo[2] *= a0.z; lo[3] *= a0.w;
          hi[0] *= a1.x; hi[1] *= a1.y; hi[2] *= a1.z; hi[3] *= a1.w;
        }
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

// e4m3 rows of the canvas keys and values: one wave per (token, KV head, K or V) row of dh <= 256
// values, 4 per lane; scale amax / 448 and codes e4m3(x / s), decided in binary32
__global__ __launch_bounds__(256) void k_kv_quant(AttnArgs a, uint8_t* kq, uint8_t* vq,
                                                  float* kqs, float* vqs, uint8_t* kc,
                                                  uint8_t* vc, float* ksc, float* vsc) {
  const long long nrow = static_cast<long long>(a.B) * a.C * a.Hkv * 2;
  const long long row = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= nrow) return;
  const int lane = threadIdx.x & 63;
  const int dh = a.dh;
  const int kind = static_cast<int>(row & 1);          // 0: key, 1: value
  const long long tg = row >> 1;                       // token * Hkv + g
  const int g = static_cast<int>(tg % a.Hkv);
  const long long t = tg / a.Hkv;
  const uint16_t* src =
      a.qkv + t * ((a.Hq + 2 * a.Hkv) * dh) + (a.Hq + kind * a.Hkv + g) * dh;
  const int c = lane * 4;
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < dh) {
    const uint2 u = *reinterpret_cast<const uint2*>(src + c);
    x = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                    __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
  const float amax =
      wave_max(fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  const uint32_t codes = f2e4m3(x.x / sc) | (f2e4m3(x.y / sc) << 8) | (f2e4m3(x.z / sc) << 16) |
                         (f2e4m3(x.w / sc) << 24);
  if (c < dh) *reinterpret_cast<uint32_t*>((kind ? vq : kq) + tg * dh + c) = codes;
  if (lane == 0) (kind ? vqs : kqs)[tg] = sc;
  if (kc) {   // encoder pass: the row also goes into the cache at position len + i
    const int b = static_cast<int>(t / a.C), i = static_cast<int>(t % a.C);
    const long long crow = (static_cast<long long>(a.kvb[b]) * a.Hkv + g) * a.cap + a.len[b] + i;
    if (c < dh) *reinterpret_cast<uint32_t*>((kind ? vc : kc) + crow * dh + c) = codes;
    if (lane == 0) (kind ? vsc : ksc)[crow] = sc;
  }
}

// ---------------------------------------------------------------------------------------------
// head_dim 256: score waves and P V waves.
//
// At head_dim 256 a wave cannot hold 32 query rows of S^T and their 32 x 256 O^T together, and
// a wave of 16 rows feeds every K and V^T fragment it reads from LDS to a single MFMA.  Here the
// two waves that share a SIMD (waves w and w + 4) take different roles:
//   * waves 0-3 (score waves) compute S^T = K Q^T and the online softmax for 32 query rows each
//     (each K fragment feeds two MFMAs) and write P (bf16) and the rescale factors to LDS;
//   * waves 4-7 (P V waves) each own O^T for 64 of the 256 dh over all 128 query rows of the
//     block (each V^T fragment feeds 8 MFMAs and each P fragment 4), one key tile behind, and
//     stage the K and V tiles (the score waves' softmax is the longer chain).
// While a score wave runs its softmax, the P V wave beside it keeps the SIMD's MFMA unit busy,
// and the LDS bytes read per flop are 40% fewer than with every wave computing both products.
// Keys go in tiles of 32 with one barrier per tile: in phase p the score waves take tile p and
// the P V waves tile p - 1.  K, V and P are double buffered in LDS.  The staging loads of a tile
// are spread over the P V MFMAs of one phase into one of two register sets and stored to LDS at
// the end of the next phase.  The visible cached keys and the canvas keys are tiled separately,
// so that the rows of a tile are equally spaced in one buffer: a uniform base and stride, and a
// per-lane row clamped to the tile's last valid one.  P is stored in the key order of the B
// operand that the transposing V^T reads pair with, so that one 16-byte LDS write and one
// 16-byte read move a lane's 8 probabilities.  A row's reference maximum moves only when a tile
// exceeds it by more than a factor 2^8, so the P V waves rarely rescale O (with 128 rows per
// wave, some row gains a new maximum in almost every tile).
constexpr int PP_KT = 32;                  // keys per tile
constexpr int PP_DH = 256;
constexpr int PP_NTHR = 512;               // 8 waves
constexpr int PP_KS = PP_DH + 16;          // bf16 per K / V row in LDS (544 B, /16 = 2 mod 4)
constexpr int PP_K8S = PP_DH + 32;         // bytes per e4m3 K row (288 B, /16 = 2 mod 4)
constexpr int PP_PST = PP_KT + 16;         // bf16 per P row (96 B, /16 = 2 mod 4)
constexpr float PP_LAZY = 8.f;             // rescale threshold of the running maximum (log2 units)

template <bool F8>
__global__ __launch_bounds__(PP_NTHR) void k_attn_pp(AttnArgs a) {
  constexpr int DH = PP_DH, KTP = PP_KT, KSS = PP_KS;
  constexpr int EB = F8 ? 1 : 2;           // bytes per cached K / V element
  __shared__ __align__(16) uint16_t ks[2][F8 ? 8 : KTP * KSS];
  __shared__ __align__(16) uint8_t ks8[2][F8 ? KTP * PP_K8S : 16];
  __shared__ __align__(16) float sks[2][F8 ? KTP : 4];   // fp8: key row scales of the tile
  __shared__ __align__(16) float svs[2][F8 ? KTP : 4];   // fp8: value row scales of the tile
  __shared__ __align__(16) uint16_t vs[2][KTP * KSS];
  __shared__ __align__(16) uint16_t ps[2][QB * PP_PST];  // P of the tile [query row][key slot]
  __shared__ __align__(16) float al[2][16 * 8];          // rescale factors [r16][query tile]
  __shared__ float lsum[QB];                             // final softmax sums

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
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  const int hpg = a.Hq / a.Hkv;
  const int ldqkv = (a.Hq + 2 * a.Hkv) * DH;

  const int len = a.len[b];
  const int c_lo = a.window > 0 ? max(0, len - a.window + 1) : 0;
  const int nc = len - c_lo;           // cache keys in the union of the visible ranges
  const int nk = nc + a.C;             // + canvas keys
  // tiles: ceil(nc / 32) of cached keys (from c_lo), then the canvas keys that some query of the
  // block sees (causal: canvas keys past the block's last canvas position are masked for all of
  // its queries); keys are numbered cache first (0 .. nc - 1), then canvas (nc .. nk - 1)
  const int tcache = (nc + KTP - 1) / KTP;
  int cv = a.C;
  if (a.causal) {
    const int r0 = qblk * QB, r1 = min(R, r0 + QB) - 1;
    cv = ((r0 / a.C == r1 / a.C) ? r1 % a.C : a.C - 1) + 1;
  }
  const int ntiles = tcache + (cv + KTP - 1) / KTP;
  const int per = (ntiles + a.n_split - 1) / a.n_split;
  const int t_beg = min(ntiles, split * per);
  const int t_end = min(ntiles, t_beg + per);
  const int n = t_end - t_beg;         // tiles of this split (>= 0)
  const float sc = a.scale_log2e;

  if (wave >= 4) {
    // ---------------- P V waves: staging, and O^T for dh 64 pw + [0, 64) of all 128 rows -----
    const int pw = wave - 4, vt = tid - 256;
    // staging by the 256 P V threads: K in pieces of 16 bytes (8 bf16 or 16 codes), V in pieces
    // of 8 values (16 bf16 bytes, or 8 codes that become 16 bf16 bytes in LDS); threads 0-31 also
    // stage the key's K and V scales (fp8)
    constexpr int KPIT = F8 ? 2 : 4;
    constexpr int KPR = DH * EB / 16;            // K pieces per key row
    constexpr int VPR = DH / 8;                  // V pieces per key row
    constexpr int VB = 8 * EB;                   // bytes per V piece in the cache
    const long long cb = (static_cast<long long>(a.kvb[b]) * a.Hkv + g) * a.cap;
    const uint8_t* kc_base = reinterpret_cast<const uint8_t*>(a.kc) + (cb + c_lo) * (DH * EB);
    const uint8_t* vc_base = reinterpret_cast<const uint8_t*>(a.vc) + (cb + c_lo) * (DH * EB);
    const long long cq0 = static_cast<long long>(b) * a.C * a.Hkv + g;   // fp8 canvas row (i = 0)
    const uint8_t* kcan = F8 ? a.kq + cq0 * DH
                             : reinterpret_cast<const uint8_t*>(a.qkv + static_cast<long long>(b) *
                                                                a.C * ldqkv + (a.Hq + g) * DH);
    const uint8_t* vcan = F8 ? a.vq + cq0 * DH
                             : reinterpret_cast<const uint8_t*>(a.qkv + static_cast<long long>(b) *
                                                                a.C * ldqkv + (a.Hq + a.Hkv + g) * DH);
    const long long can_stride = F8 ? static_cast<long long>(a.Hkv) * DH : 2ll * ldqkv;   // bytes
    int k_key[KPIT], v_key[4], k_col[KPIT], v_col[4];   // key in the tile, byte in the row
#pragma unroll
    for (int it = 0; it < KPIT; ++it) {
      const int pc = vt + it * 256;
      k_key[it] = pc / KPR;
      k_col[it] = (pc % KPR) * 16;
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int pc = vt + it * 256;
      v_key[it] = pc / VPR;
      v_col[it] = (pc % VPR) * VB;
    }
    // tile tt: first row address, row stride (bytes) and the last valid row of the tile (uniform);
    // every staging load is unconditional: a key past the range reads the range's last key,
    // finite data whose score is masked
    struct TileRows {
      const uint8_t* k;
      const uint8_t* v;
      long long stride;
      int last;
    };
    auto tile_rows = [&](int tt) -> TileRows {
      TileRows t;
      if (tt < tcache) {
        const long long r0 = static_cast<long long>(tt) * KTP;
        t.k = kc_base + r0 * (DH * EB);
        t.v = vc_base + r0 * (DH * EB);
        t.stride = DH * EB;
        t.last = nc - 1 - tt * KTP;
      } else {
        const long long r0 = static_cast<long long>(tt - tcache) * KTP;
        t.k = kcan + r0 * can_stride;
        t.v = vcan + r0 * can_stride;
        t.stride = can_stride;
        t.last = a.C - 1 - (tt - tcache) * KTP;
      }
      return t;
    };
    const float* ksc_base = F8 ? a.ksc + cb + c_lo : nullptr;
    const float* vsc_base = F8 ? a.vsc + cb + c_lo : nullptr;

    // two register sets, alternating by phase parity
    u32x4 pk[2][KPIT];
    u32x4 pv[2][F8 ? 1 : 4];
    uint2 pv8[2][F8 ? 4 : 1];
    float pks[2] = {0.f, 0.f}, pvs[2] = {0.f, 0.f};
    // piece it of tile tt (rows t) into set S; K piece 0 also brings the fp8 scales
    auto load_k = [&](const TileRows& t, int tt, int it, auto set_tag) __attribute__((always_inline)) {
      constexpr int S = decltype(set_tag)::value;
      const uint8_t* kp = t.k + (static_cast<uint32_t>(min(k_key[it], t.last)) *
                                     static_cast<uint32_t>(t.stride) +
                                 static_cast<uint32_t>(k_col[it]));
      pk[S][it] = F8 ? ld16(kp) : ld16_stream(kp);
      if constexpr (F8) {
        if (it != 0) return;
        if (vt < KTP) {
          const int rr = min(vt, t.last);
          if (tt < tcache) {
            pks[S] = ksc_base[tt * KTP + rr];
            pvs[S] = vsc_base[tt * KTP + rr];
          } else {
            const long long ci = cq0 + static_cast<long long>((tt - tcache) * KTP + rr) * a.Hkv;
            pks[S] = a.kqs[ci];
            pvs[S] = a.vqs[ci];
          }
        }
      }
    };
    auto load_v = [&](const TileRows& t, int it, auto set_tag) __attribute__((always_inline)) {
      constexpr int S = decltype(set_tag)::value;
      const uint8_t* p = t.v + (static_cast<uint32_t>(min(v_key[it], t.last)) *
                                    static_cast<uint32_t>(t.stride) +
                                static_cast<uint32_t>(v_col[it]));
      if constexpr (F8)
        pv8[S][it] = *reinterpret_cast<const uint2*>(p);
      else
        pv[S][it] = ld16_stream(p);
    };
    // the pieces of K of tile tk and V of tile tv into set S, all at once
    auto fetch = [&](int tk, int tv, auto set_tag) __attribute__((always_inline)) {
      const TileRows rk = tile_rows(tk), rv = tile_rows(tv);
#pragma unroll
      for (int it = 0; it < KPIT; ++it) load_k(rk, tk, it, set_tag);
#pragma unroll
      for (int it = 0; it < 4; ++it) load_v(rv, it, set_tag);
    };
    auto store_k = [&](int buf, auto set_tag) __attribute__((always_inline)) {
      constexpr int S = decltype(set_tag)::value;
#pragma unroll
      for (int it = 0; it < KPIT; ++it) {
        const int col = k_col[it];
        if constexpr (F8)
          st16(&ks8[buf][k_key[it] * PP_K8S + col], pk[S][it]);
        else
          st16(reinterpret_cast<uint8_t*>(ks[buf]) + k_key[it] * (KSS * 2) + col, pk[S][it]);
      }
      if constexpr (F8) {
        if (vt < KTP) {
          sks[buf][vt] = pks[S];
          svs[buf][vt] = pvs[S];
        }
      }
    };
    auto store_v = [&](int buf, auto set_tag) __attribute__((always_inline)) {
      constexpr int S = decltype(set_tag)::value;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int col = v_col[it] / EB;   // element
        if constexpr (F8) {
          // 8 codes -> their bf16 values (exact); the row's scale goes onto P
          uint32_t w[4];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int x = static_cast<int>(h2 ? pv8[S][it].y : pv8[S][it].x);
            w[2 * h2] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
            w[2 * h2 + 1] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
          }
          st16(vs[buf] + v_key[it] * KSS + col, u32x4{w[0], w[1], w[2], w[3]});
        } else {
          st16(vs[buf] + v_key[it] * KSS + col, pv[S][it]);
        }
      }
    };

    f32x4 o[4][8];
#pragma unroll
    for (int dl = 0; dl < 4; ++dl)
#pragma unroll
      for (int qt = 0; qt < 8; ++qt) o[dl][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    using J0 = std::integral_constant<int, 0>;
    using J1 = std::integral_constant<int, 1>;
    if (n > 0) {
      fetch(t_beg, t_beg, J0{});
      store_k(0, J0{});
      fetch(min(t_beg + 1, t_end - 1), t_beg, J0{});
    }
    __syncthreads();   // the first K tile
    const uint16_t* vlane0 = &vs[0][0] + (4 * lg + (r16 >> 2)) * KSS + 4 * (r16 & 3) + pw * 64;
    const uint16_t* pl0 = &ps[0][0] + r16 * PP_PST + 8 * lg;
    // phase i (parity P): P V of tile i - 1 with the pieces of K of tile i + 2 and V of tile i + 1
    // loaded into set P ^ 1 spread over its MFMAs, and K of tile i + 1 and V of tile i (loaded in
    // the phase before, set P) stored to LDS among them (clamped: the last phases re-stage valid
    // tiles that are never read)
    auto vphase = [&](int i, auto par) __attribute__((always_inline)) {
      constexpr int P = decltype(par)::value;
      using NX = std::integral_constant<int, P ^ 1>;
      const int fk = min(t_beg + i + 2, t_end - 1), fv = min(t_beg + i + 1, t_end - 1);
      if (i == 0) {
        if (n > 0) fetch(fk, fv, NX{});
      } else {
        const TileRows rk = tile_rows(fk), rv = tile_rows(fv);
        const int prev = (i - 1) & 1;
        // rescale by the factors of tile i - 1, per query tile (wave-uniform tests)
        const float4 a0 = *reinterpret_cast<const float4*>(&al[prev][r16 * 8]);
        const float4 a1 = *reinterpret_cast<const float4*>(&al[prev][r16 * 8 + 4]);
        const float alr[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int qt = 0; qt < 8; ++qt) {
          if (__builtin_amdgcn_ballot_w64(alr[qt] != 1.f)) {
#pragma unroll
            for (int dl = 0; dl < 4; ++dl) o[dl][qt] *= alr[qt];
          }
        }
        // V^T fragment of dh tile 4 pw + dl: lane (dh r16, group lg) gets keys 4 lg + [0, 4) and
        // 16 + 4 lg + [0, 4); the P fragment of query tile qt holds the same keys in that order
        const uint16_t* vlane = vlane0 + prev * (KTP * KSS);
        u32x4 vf[4];
#pragma unroll
        for (int dl = 0; dl < 4; ++dl) {
          const s16x4 lo = lds_read_tr16(vlane + dl * 16);
          const s16x4 hi = lds_read_tr16(vlane + 16 * KSS + dl * 16);
          vf[dl] = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        const uint16_t* pl = pl0 + prev * (QB * PP_PST);
        u32x4 pr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[j] = ld16(pl + j * 16 * PP_PST);
#pragma unroll
        for (int qt = 0; qt < 8; ++qt) {
#pragma unroll
          for (int dl = 0; dl < 4; ++dl) o[dl][qt] = mfma16x16x32(vf[dl], pr[qt % 4], o[dl][qt]);
          if (qt + 4 < 8) pr[qt % 4] = ld16(pl + (qt + 4) * 16 * PP_PST);
          if (qt < KPIT) load_k(rk, fk, qt, NX{});
          else if (qt < KPIT + 4) load_v(rv, qt - KPIT, NX{});
          // K of tile i + 1 and V of tile i go to LDS among the MFMAs rather than after them.
          // The K buffer was last read by the score waves in phase i - 1 and the V buffer by
          // these waves in phase i - 1, so both are free once this phase has begun.  bf16: after
          // query tiles 2 and 3 (56.3 against 58.4 us per call at the decoder shape).  e4m3:
          // after query tiles 5 and 6, later since its V stores carry the code conversion (953
          // against 938 TFLOP/s on the long-context step; after tiles 2 and 3: 847 against 877)
          if (qt == (F8 ? 5 : 2)) store_k((i + 1) & 1, par);
          if (qt == (F8 ? 6 : 3)) store_v(i & 1, par);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (n > 0 && i == 0) {
        store_k((i + 1) & 1, par);
        store_v(i & 1, par);
      }
      __syncthreads();
    };
    int i = 0;
    for (; i + 1 <= n; i += 2) {
      vphase(i, J0{});
      vphase(i + 1, J1{});
    }
    if (i <= n) vphase(i, J0{});
    __syncthreads();   // the score waves' sums
#pragma unroll
    for (int qt = 0; qt < 8; ++qt) {
      const int rr = qblk * QB + 16 * qt + r16;
      if (rr >= R) continue;
      const int qi = rr % a.C, h = g * hpg + rr / a.C;
      const long long qrow = static_cast<long long>(b) * a.C + qi;
      if (a.n_split == 1) {
        const float lq = lsum[16 * qt + r16];
        const float inv = lq > 0.f ? 1.f / lq : 0.f;
        uint16_t* op = a.out + qrow * (a.Hq * DH) + h * DH + pw * 64;
#pragma unroll
        for (int dl = 0; dl < 4; ++dl) {
          uint2 pk2;
          pk2.x = pack_bf2(o[dl][qt][0] * inv, o[dl][qt][1] * inv);
          pk2.y = pack_bf2(o[dl][qt][2] * inv, o[dl][qt][3] * inv);
          *reinterpret_cast<uint2*>(op + dl * 16 + 4 * lg) = pk2;
        }
      } else {
        const long long prow = ((static_cast<long long>(split) * a.B + b) * a.Hkv + g) * R + rr;
        uint16_t* op = a.o_part + prow * DH + pw * 64;
#pragma unroll
        for (int dl = 0; dl < 4; ++dl) {
          uint2 pk2;
          pk2.x = pack_bf2(o[dl][qt][0], o[dl][qt][1]);
          pk2.y = pack_bf2(o[dl][qt][2], o[dl][qt][3]);
          *reinterpret_cast<uint2*>(op + dl * 16 + 4 * lg) = pk2;
        }
      }
    }
    return;
  }

  // ---------------- score waves: rows 32 sw + 16 q + r16 of the block -------------------------
  const int sw = wave;
  int r[2], qi[2], h[2], win_lo[2];
  long long qrow[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    r[q] = qblk * QB + 32 * sw + 16 * q + r16;
    const int rr = r[q] < R ? r[q] : R - 1;
    qi[q] = rr % a.C;
    h[q] = g * hpg + rr / a.C;
    qrow[q] = static_cast<long long>(b) * a.C + qi[q];
    win_lo[q] = len + qi[q] - a.window + 1;   // first visible cache position (windowed)
  }
  // query fragments: bf16 (dh 32 ks + 8 lg + [0, 8)), or e4m3 codes with the row scale (lane
  // holds dh 128 kb + 16 lg + [0, 16) and 128 kb + 64 + 16 lg + [0, 16))
  u32x4 qf[F8 ? 1 : 8][2];
  u32x4 qf8[F8 ? 2 : 1][2][2];
  float sq[2] = {1.f, 1.f};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint16_t* qp = a.qkv + qrow[q] * ldqkv + h[q] * DH;
    if constexpr (!F8) {
#pragma unroll
      for (int k2 = 0; k2 < 8; ++k2) qf[k2][q] = ld16(qp + k2 * 32 + lg * 8);
    } else {
      u32x4 raw[2][4];
      float amax = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          raw[kb][m] = ld16(qp + 128 * kb + (m >> 1) * 64 + 16 * lg + 8 * (m & 1));
#pragma unroll
          for (int w = 0; w < 4; ++w)
            amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(raw[kb][m][w] << 16)),
                                     fabsf(__uint_as_float(raw[kb][m][w] & 0xffff0000u))));
        }
      amax = lanes_max4(amax);
      sq[q] = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint32_t c[4];
#pragma unroll
          for (int w = 0; w < 4; ++w)
            c[w] = f2e4m3(__uint_as_float(raw[kb][m][w] << 16) / sq[q]) |
                   (f2e4m3(__uint_as_float(raw[kb][m][w] & 0xffff0000u) / sq[q]) << 8);
          const uint32_t lo = c[0] | (c[1] << 16), hi = c[2] | (c[3] << 16);
          u32x4& dst = qf8[kb][q][m >> 1];
          if (m & 1) {
            dst.z = lo;
            dst.w = hi;
          } else {
            dst.x = lo;
            dst.y = hi;
          }
        }
    }
  }
  // wave-uniform range of the wave's canvas positions (tiles every query sees entirely need no
  // per-element mask)
  int qi_lo = min(qi[0], qi[1]), qi_hi = max(qi[0], qi[1]);
#pragma unroll
  for (int o2 = 1; o2 < 64; o2 <<= 1) {
    qi_lo = min(qi_lo, __shfl_xor(qi_lo, o2, 64));
    qi_hi = max(qi_hi, __shfl_xor(qi_hi, o2, 64));
  }
  qi_lo = __builtin_amdgcn_readfirstlane(qi_lo);
  qi_hi = __builtin_amdgcn_readfirstlane(qi_hi);

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // the query fragments stay in registers for the whole key range
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if constexpr (F8) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        asm volatile("" : "+v"(qf8[kb][q][0]));
        asm volatile("" : "+v"(qf8[kb][q][1]));
      }
    } else {
#pragma unroll
      for (int k2 = 0; k2 < 8; ++k2) asm volatile("" : "+v"(qf[k2][q]));
    }
  }
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  __syncthreads();
  // phase i (parity P = i & 1): scores and softmax of tile i from buffer P
  auto phase = [&](int i, auto par) __attribute__((always_inline)) {
    constexpr int cur = decltype(par)::value;
    const int tt = t_beg + i;
    const bool cache_tile = tt < tcache;
    const int kbase = cache_tile ? tt * KTP : nc + (tt - tcache) * KTP;   // first key
    const int klim = cache_tile ? nc : nk;                                 // keys >= klim: none
    f32x4 s[2][2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) s[q][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (F8) {
      // fragment j = (dh block j / 2, key sub-tile j % 2): 32 bytes per lane, two reads
      const uint8_t* k8b = ks8[cur] + r16 * PP_K8S + 16 * lg;
      u32x4 kr8[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint8_t* p = k8b + (j % 2) * 16 * PP_K8S + (j / 2) * 128;
        kr8[j][0] = ld16(p);
        kr8[j][1] = ld16(p + 64);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          s[q][j % 2] = mfma_f8_128(kr8[j][0], kr8[j][1], qf8[j / 2][q][0], qf8[j / 2][q][1],
                                    s[q][j % 2]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float4 skv = *reinterpret_cast<const float4*>(&sks[cur][nt * 16 + 4 * lg]);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          s[q][nt][0] *= skv.x;
          s[q][nt][1] *= skv.y;
          s[q][nt][2] *= skv.z;
          s[q][nt][3] *= skv.w;
        }
      }
    } else {
      // 16 K fragments (dh step j / 2, key sub-tile j % 2) through a 4-deep register ring, each
      // read 4 fragments (8 MFMAs) ahead of use; each feeds both query tiles
      const uint16_t* kl = ks[cur] + r16 * KSS + lg * 8;
      auto kfrag = [&](int j) -> u32x4 { return ld16(kl + (j % 2) * 16 * KSS + (j / 2) * 32); };
      u32x4 kr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) kr[j] = kfrag(j);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
#pragma unroll
        for (int q = 0; q < 2; ++q) s[q][j % 2] = mfma16x16x32(kr[j % 4], qf[j / 2][q], s[q][j % 2]);
        if (j + 4 < 16) kr[j % 4] = kfrag(j + 4);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // visibility (the lane's keys: nt * 16 + 4 lg + j)
    const bool full =
        kbase + KTP <= klim &&
        (cache_tile ? (a.window == 0 || c_lo + kbase >= len + qi_hi - a.window + 1)
                    : (!a.causal || kbase + KTP - 1 - nc <= qi_lo));
    float4 svk[2];
    if constexpr (F8) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        svk[nt] = *reinterpret_cast<const float4*>(&svs[cur][nt * 16 + 4 * lg]);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float scq = sc;
      if constexpr (F8) scq = sc * sq[q];
      float tmax = -INFINITY;
      if (full) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          tmax = fmaxf(tmax, fmaxf(fmaxf(s[q][nt][0], s[q][nt][1]), fmaxf(s[q][nt][2], s[q][nt][3])));
      } else {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kk = kbase + nt * 16 + 4 * lg + j;
            bool vis = kk < klim;
            if (cache_tile) {
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
      // the row's reference maximum moves only when the tile's maximum exceeds it by more
      // than PP_LAZY (log2 units), so the probabilities stay <= 2^PP_LAZY and the P V waves
      // rescale O only at the first tiles of a row (a wave-uniform test per query tile)
      const float t_m = tmax * scq;
      const float m_new = (t_m > m_run[q] + PP_LAZY) ? t_m : m_run[q];
      const float neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[q] + neg_m);   // m_run = -inf: 0
      m_run[q] = m_new;
      f32x4 lo, hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[q][0][j], scq, neg_m));
        hi[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[q][1][j], scq, neg_m));
      }
      l_run[q] = l_run[q] * alpha +
                 ((lo[0] + lo[1]) + (lo[2] + lo[3]) + (hi[0] + hi[1]) + (hi[2] + hi[3]));
      if constexpr (F8) {
        lo[0] *= svk[0].x; lo[1] *= svk[0].y; lo[2] *= svk[0].z; lo[3] *= svk[0].w;
        hi[0] *= svk[1].x; hi[1] *= svk[1].y; hi[2] *= svk[1].z; hi[3] *= svk[1].w;
      }
      // keys 4 lg + [0, 4) and 16 + 4 lg + [0, 4) go to slots 8 lg + [0, 8) of the row
      st16(&ps[cur][(32 * sw + 16 * q + r16) * PP_PST + 8 * lg],
           u32x4{cvt_pk_bf16(lo[0], lo[1]), cvt_pk_bf16(lo[2], lo[3]),
                 cvt_pk_bf16(hi[0], hi[1]), cvt_pk_bf16(hi[2], hi[3])});
      if (lg == 0) al[cur][r16 * 8 + 2 * sw + q] = alpha;
    }
    __syncthreads();
  };
  int i = 0;
  for (; i + 1 < n; i += 2) {
    phase(i, I0{});
    phase(i + 1, I1{});
  }
  if (i < n) phase(i, I0{});
  __syncthreads();   // the P V waves take the last tile
  float l[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    l[q] = lanes_sum4(l_run[q]);
    if (lg == 0) lsum[32 * sw + 16 * q + r16] = l[q];
  }
  if (a.n_split > 1) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (r[q] >= R || lg != 0) continue;
      const long long prow = ((static_cast<long long>(split) * a.B + b) * a.Hkv + g) * R + r[q];
      a.ml_part[prow * 2] = m_run[q];
      a.ml_part[prow * 2 + 1] = l[q];
    }
  }
  __syncthreads();
}

template <bool F8>
hipError_t launch_pp(const AttnArgs& a, hipStream_t s) {
  const int R = (a.Hq / a.Hkv) * a.C;
  int grid = ((R + QB - 1) / QB) * a.Hkv * a.B * a.n_split;
  grid = (grid + 7) & ~7;
  hipLaunchKernelGGL(k_attn_pp<F8>, dim3(grid), dim3(PP_NTHR), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const long long n = static_cast<long long>(a.B) * a.Hkv * R * (PP_DH / 4);
  hipLaunchKernelGGL(k_attn_merge<PP_DH>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

template <int DH, bool F8>
hipError_t launch_dh(const AttnArgs& a, hipStream_t s) {
  const int R = (a.Hq / a.Hkv) * a.C;
  int grid = ((R + QB - 1) / QB) * a.Hkv * a.B * a.n_split;
  grid = (grid + 7) & ~7;
  hipLaunchKernelGGL((k_attn<DH, F8>), dim3(grid), dim3(AttnCfg<DH>::NTHR), 0, s, a);
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
  if (a.f8) {
    switch (a.dh) {   // the e4m3 QK^T runs 128 dh per MFMA
      case 128: return launch_dh<128, true>(a, s);
      case 256: return launch_pp<true>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.dh) {
    case 16: return launch_dh<16, false>(a, s);
    case 32: return launch_dh<32, false>(a, s);
    case 64: return launch_dh<64, false>(a, s);
    case 128: return launch_dh<128, false>(a, s);
    case 256: return launch_pp<false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_kv_quant(const AttnArgs& a, uint8_t* kq, uint8_t* vq, float* kqs, float* vqs,
                           uint8_t* kc, uint8_t* vc, float* ksc, float* vsc, hipStream_t s) {
  if (a.dh > 256 || a.dh % 4) return hipErrorInvalidValue;
  const long long nrow = static_cast<long long>(a.B) * a.C * a.Hkv * 2;
  if (nrow == 0) return hipSuccess;
  hipLaunchKernelGGL(k_kv_quant, dim3(static_cast<unsigned>((nrow + 3) / 4)), dim3(256), 0, s, a,
                     kq, vq, kqs, vqs, kc, vc, ksc, vsc);
  return hipGetLastError();
}

}  // namespace dg
