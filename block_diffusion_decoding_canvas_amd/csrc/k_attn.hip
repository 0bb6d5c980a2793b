// Canvas attention: every canvas query attends, in one softmax, to the visible cached keys and
// to the canvas keys (DiffusionGemma model card, "Model overview": bidirectional attention over
// the canvas plus cross-attention to the cached context; the encoder reads a finished canvas
// causally).  GQA: query head h reads KV head floor(h * Hkv / Hq); scale 1/sqrt(head_dim).
// Sliding-window layers: canvas query i at absolute position len + i sees cache position j
// only if (len + i) - j < window (model card dimension table: 1,024-token window).
//
// Layout of the work: one workgroup = (canvas b, KV head g, 128 query rows, one split of the
// key range).  The query rows of a KV head are its Hq/Hkv query heads times the canvas
// positions, so the K/V tiles staged in LDS serve every query head that reads them.  Keys are
// processed in tiles of 64 (K tile [key][dh] and V tile transposed [dh][key] in LDS).  Each wave
// holds 16 query rows and computes S^T = K Q^T, so the probabilities come out of the MFMA in the
// lane layout that the P V product takes as its B operand (O^T = V^T P^T) with no shuffle.
// Splits of the key range write unnormalised partial outputs with their running max and sum,
// merged afterwards by log-sum-exp.
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int KT = 64;        // keys per tile
constexpr int NWAVE = 8;      // waves per workgroup
constexpr int QB = NWAVE * 16; // query rows per workgroup
constexpr int NTHR = NWAVE * 64;

template <int DH>
struct AttnCfg {
  static constexpr int KS_STRIDE = DH + 8;   // bf16 per K row in LDS
  static constexpr int VT_STRIDE = KT + 8;   // bf16 per transposed V row in LDS
  static constexpr int NKS = (DH + 31) / 32; // 32-wide dh steps of QK^T
  static constexpr int NDT = DH / 16;        // 16-row dh tiles of O^T
  static constexpr int LDS_BYTES = (KT * KS_STRIDE + DH * VT_STRIDE) * 2;
};

template <int DH>
__global__ __launch_bounds__(NTHR) void k_attn(AttnArgs a) {
  using C = AttnCfg<DH>;
  constexpr int ITEMS = (KT / 2) * (DH / 8) / NTHR;  // (key pair, 8-dh chunk) items per thread
  constexpr int IT = ITEMS >= 1 ? ITEMS : 1;
  __shared__ __align__(16) uint16_t ks[KT * C::KS_STRIDE];
  __shared__ __align__(16) uint16_t vt[DH * C::VT_STRIDE];

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

  // this lane's query row (B operand column)
  const int r = qblk * QB + wave * 16 + r16;
  const bool r_ok = r < R;
  const int rr = r_ok ? r : R - 1;
  const int hl = rr / a.C, qi = rr % a.C;
  const int h = g * hpg + hl;
  const long long qrow = static_cast<long long>(b) * a.C + qi;

  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  u32x4 qf[C::NKS];
  {
    const uint16_t* qp = a.qkv + qrow * ldqkv + h * DH;
#pragma unroll
    for (int ks_ = 0; ks_ < C::NKS; ++ks_) {
      const int d0 = ks_ * 32 + lg * 8;
      qf[ks_] = (d0 < DH) ? ld16(qp + d0) : zero4;
    }
  }

  f32x4 o[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* kcache = a.kc + (static_cast<long long>(b) * a.Hkv + g) * a.cap * DH;
  const uint16_t* vcache = a.vc + (static_cast<long long>(b) * a.Hkv + g) * a.cap * DH;
  const uint16_t* kcanvas = a.qkv + static_cast<long long>(b) * a.C * ldqkv + (a.Hq + g) * DH;
  const uint16_t* vcanvas = kcanvas + a.Hkv * DH;
  const int win_lo = len + qi - a.window + 1;  // first visible cache position (windowed layers)

  // wave-uniform range of this wave's canvas positions (tiles that no query of the wave sees
  // partially are processed without per-element masks)
  int qi_lo = qi, qi_hi = qi;
#pragma unroll
  for (int o2 = 1; o2 < 64; o2 <<= 1) {
    qi_lo = min(qi_lo, __shfl_xor(qi_lo, o2, 64));
    qi_hi = max(qi_hi, __shfl_xor(qi_hi, o2, 64));
  }
  qi_lo = __builtin_amdgcn_readfirstlane(qi_lo);
  qi_hi = __builtin_amdgcn_readfirstlane(qi_hi);

  // staging items: (key pair p, dh chunk c): two keys' rows of K, and of V written transposed;
  // the next tile's rows are prefetched into registers while the current one is computed
  constexpr int ITEMS_ALL = (KT / 2) * (DH / 8);
  u32x4 pk0[IT], pk1[IT], pv0[IT], pv1[IT];
  auto key_ptr = [&](int kk, const uint16_t* cache, const uint16_t* canvas) -> const uint16_t* {
    return kk < nc ? cache + static_cast<long long>(c_lo + kk) * DH
                   : canvas + static_cast<long long>(kk - nc) * ldqkv;
  };
  auto fetch = [&](int tt) __attribute__((always_inline)) {
    const int kt0 = tt * KT;
    if (kt0 + KT <= nc) {
      // every key of the tile is a cache row: two consecutive rows per item
      const long long base = static_cast<long long>(c_lo + kt0) * DH;
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int idx = tid + it * NTHR;
        const int pp = idx % (KT / 2), c = idx / (KT / 2);
        const long long off = base + static_cast<long long>(2 * pp) * DH + c * 8;
        if (idx < ITEMS_ALL) {
          pk0[it] = ld16(kcache + off);
          pk1[it] = ld16(kcache + off + DH);
          pv0[it] = ld16(vcache + off);
          pv1[it] = ld16(vcache + off + DH);
        }
      }
      return;
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = tid + it * NTHR;
      const bool on = idx < ITEMS_ALL;
      const int pp = idx % (KT / 2), c = idx / (KT / 2);
      const int k0 = kt0 + 2 * pp;
      pk0[it] = pk1[it] = pv0[it] = pv1[it] = zero4;
      if (on && k0 < nk) {
        pk0[it] = ld16(key_ptr(k0, kcache, kcanvas) + c * 8);
        pv0[it] = ld16(key_ptr(k0, vcache, vcanvas) + c * 8);
      }
      if (on && k0 + 1 < nk) {
        pk1[it] = ld16(key_ptr(k0 + 1, kcache, kcanvas) + c * 8);
        pv1[it] = ld16(key_ptr(k0 + 1, vcache, vcanvas) + c * 8);
      }
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = tid + it * NTHR;
      if (idx >= ITEMS_ALL) continue;
      const int pp = idx % (KT / 2), c = idx / (KT / 2);
      st16(ks + (2 * pp) * C::KS_STRIDE + c * 8, pk0[it]);
      st16(ks + (2 * pp + 1) * C::KS_STRIDE + c * 8, pk1[it]);
      // V^T[dh][key]: each 32-bit store holds keys 2p and 2p+1 of one dh
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a0 = pv0[it][e], a1 = pv1[it][e];
        uint32_t* row0 = reinterpret_cast<uint32_t*>(vt + (c * 8 + 2 * e) * C::VT_STRIDE) + pp;
        uint32_t* row1 = reinterpret_cast<uint32_t*>(vt + (c * 8 + 2 * e + 1) * C::VT_STRIDE) + pp;
        *row0 = __builtin_amdgcn_perm(a1, a0, 0x05040100u);   // low halves: key 2p, key 2p+1
        *row1 = __builtin_amdgcn_perm(a1, a0, 0x07060302u);   // high halves
      }
    }
  };

  const float sc = a.scale_log2e;
  // the next tile's K/V rows are fetched into registers while the current tile is computed
  if (t_beg < t_end) fetch(t_beg);
  for (int tt = t_beg; tt < t_end; ++tt) {
    const int kbase = tt * KT;
    __syncthreads();  // previous tile fully consumed
    stage();
    __syncthreads();
    if (tt + 1 < t_end) fetch(tt + 1);

    // S^T[key][q] for 4 sub-tiles of 16 keys (raw dot products).  The 4 NKS MFMAs run ks-major
    // (consecutive MFMAs update different accumulators) with a 4-deep ring of K fragments read
    // from LDS ahead of use, pinned by scheduling barriers so each MFMA waits only for its own
    constexpr int NS = 4 * C::NKS;
    auto kfrag = [&](int i) -> u32x4 {
      const int d0 = (i / 4) * 32 + lg * 8;
      return (d0 < DH) ? ld16(ks + ((i % 4) * 16 + r16) * C::KS_STRIDE + d0) : zero4;
    };
    f32x4 s[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) s[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 kr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[i] = kfrag(i);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      s[i % 4] = mfma16x16x32(kr[i % 4], qf[i / 4], s[i % 4]);
      if (i + 4 < NS) kr[i % 4] = kfrag(i + 4);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first V^T fragments of the P V product, read while the softmax below runs
    constexpr int NP = 2 * C::NDT;
    auto vfrag = [&](int i) -> u32x4 {
      const uint16_t* vrow = vt + ((i % C::NDT) * 16 + r16) * C::VT_STRIDE + (i / C::NDT) * 32 + 4 * lg;
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    };
    u32x4 vr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = vfrag(i);
    // visibility: a tile inside the canvas or inside the cache that every query of this wave
    // sees entirely needs no per-element mask (the lane's keys: nt*16 + 4 lg + j)
    const bool in_cache = kbase + KT <= nc;
    const bool full =
        kbase + KT <= nk &&
        (in_cache ? (a.window == 0 || c_lo + kbase >= len + qi_hi - a.window + 1)
                  : (kbase >= nc && (!a.causal || kbase + KT - 1 - nc <= qi_lo)));
    float tmax = -INFINITY;
    if (full) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        tmax = fmaxf(tmax, fmaxf(fmaxf(s[nt][0], s[nt][1]), fmaxf(s[nt][2], s[nt][3])));
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kk = kbase + nt * 16 + 4 * lg + j;
          bool vis = kk < nk;
          if (kk < nc) {
            if (a.window > 0) vis = vis && (c_lo + kk >= win_lo);
          } else if (a.causal) {
            vis = vis && (kk - nc <= qi);
          }
          s[nt][j] = vis ? s[nt][j] : -INFINITY;
          tmax = fmaxf(tmax, s[nt][j]);
        }
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // running max in scaled (log2) units; the scale is > 0, so it commutes with the max
    const float m_new = fmaxf(m_run, tmax * sc);
    const float neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run + neg_m);   // m_run = -inf: 0
    m_run = m_new;
    // rescale only when some lane's maximum moved (a wave-uniform branch)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) o[dt] *= alpha;
    }
    u32x4 pb[2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      f32x4 lo, hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * kp][j], sc, neg_m));
        hi[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * kp + 1][j], sc, neg_m));
      }
      l_run += (lo[0] + lo[1]) + (lo[2] + lo[3]) + (hi[0] + hi[1]) + (hi[2] + hi[3]);
      pb[kp] = u32x4{cvt_pk_bf16(lo[0], lo[1]), cvt_pk_bf16(lo[2], lo[3]),
                     cvt_pk_bf16(hi[0], hi[1]), cvt_pk_bf16(hi[2], hi[3])};
    }
    // O^T[dh][q] += V^T[dh][keys] P^T[keys][q]; the B operand's 8 keys per lane are
    // {32 kp + 4 lg + 0..3, 32 kp + 16 + 4 lg + 0..3}; the A operand reads the same keys.
    // kp-major (consecutive MFMAs update different accumulators), 4-deep V^T fragment ring.
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      o[i % C::NDT] = mfma16x16x32(vr[i % 4], pb[i / C::NDT], o[i % C::NDT]);
      if (i + 4 < NP) vr[i % 4] = vfrag(i + 4);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // row sum over the 4 lanes that share this query
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!r_ok) return;
  if (a.n_split == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* op = a.out + qrow * (a.Hq * DH) + h * DH;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      uint2 pk;
      pk.x = pack_bf2(o[dt][0] * inv, o[dt][1] * inv);
      pk.y = pack_bf2(o[dt][2] * inv, o[dt][3] * inv);
      *reinterpret_cast<uint2*>(op + dt * 16 + 4 * lg) = pk;
    }
  } else {
    const long long prow = ((static_cast<long long>(split) * a.B + b) * a.Hkv + g) * R + r;
    float* op = a.o_part + prow * DH;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
      *reinterpret_cast<float4*>(op + dt * 16 + 4 * lg) =
          make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (lg == 0) {
      a.ml_part[prow * 2] = m_run;
      a.ml_part[prow * 2 + 1] = l_run;
    }
  }
}

// merge of split partials: one thread per (query row, 4 dh values)
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
  float mmax = -INFINITY;
  for (int sp = 0; sp < a.n_split; ++sp) mmax = fmaxf(mmax, a.ml_part[(sp * stride + row) * 2]);
  float l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // splits merged in split order; each group of 8 is loaded together (clamped split index,
  // zero weight past the last split)
  for (int sp0 = 0; sp0 < a.n_split; sp0 += 8) {
    float2 ml[8];
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const long long r2 = static_cast<long long>(min(sp0 + u, a.n_split - 1)) * stride + row;
      ml[u] = *reinterpret_cast<const float2*>(a.ml_part + r2 * 2);
      v[u] = *reinterpret_cast<const float4*>(a.o_part + r2 * DH + c4);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (sp0 + u < a.n_split) {  // uniform; the loads above are already in flight
        const float m = ml[u].x;
        const float w = (m == -INFINITY) ? 0.f : exp2f(m - mmax);
        l += w * ml[u].y;
        acc.x += w * v[u].x;
        acc.y += w * v[u].y;
        acc.z += w * v[u].z;
        acc.w += w * v[u].w;
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
  hipLaunchKernelGGL(k_attn<DH>, dim3(grid), dim3(NTHR), 0, s, a);
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
