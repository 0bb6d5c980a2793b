// Per-token kernels of the decoder step:
//   embed     h[t] = E[token t] (row gather, fp32 residual stream)
//   rmsnorm   u = bf16(h / sqrt(mean(h^2) + eps) * gain); in the fp8 configuration also the
//             row's e4m3 codes and scale (amax / 448), decided in binary32
//   topk      router: top-k experts by logit (lowest id on ties, descending order), gates =
//             softmax weights renormalised over the top-k
//   permute   stable counting sort of the (token, slot) pairs by expert; emits the row order,
//             its inverse and the tile list the grouped expert GEMMs read (the shared expert's
//             tiles last)
//   combine   h[t] += sum_j gate_tj Y[row(t, j)] (fixed j order) + Y_shared[t]; optionally the
//             next RMSNorm of the same row
//   kv_write  the canvas keys/values of one layer into the cache at [len, len + C)
// The MoE is 8 of 128 routed experts plus 1 shared (DiffusionGemma model card, dimension table).
#include "dg_internal.h"

namespace dg {
namespace {

struct TokMap {
  int C, n;        // n > 0: row t reads tokens[idx[t / C] * C + t % C]
  int idx[64];
};

// token ids outside [0, vocab) are clamped into range (no out-of-bounds gather)
__global__ __launch_bounds__(256) void k_embed(const int32_t* tokens, const uint16_t* embed,
                                               float* h, int ntok, int d, int vocab, TokMap mp) {
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const int per = d / 8;
  if (idx >= static_cast<long long>(ntok) * per) return;
  const int t = static_cast<int>(idx / per), c = static_cast<int>(idx % per) * 8;
  const long long src = mp.n > 0 ? static_cast<long long>(mp.idx[t / mp.C]) * mp.C + t % mp.C : t;
  const int tok = min(max(tokens[src], 0), vocab - 1);
  const uint4 v = *reinterpret_cast<const uint4*>(embed + static_cast<long long>(tok) * d + c);
  float4* o = reinterpret_cast<float4*>(h + static_cast<long long>(t) * d + c);
  o[0] = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
  o[1] = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xffff0000u),
                     __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xffff0000u));
}

// ---- per-token row kernels -------------------------------------------------------------------
// One workgroup of 256 threads per token row of d <= 8192 fp32 values; thread i owns the float4
// chunks at columns 4 i + 1024 n, n < NC = ceil(d / 1024).  Every load a row needs (the
// residual, its addends, the norm gain) is issued before its first use and the row stays in
// registers through the norm, so a token costs one memory round trip and two workgroup
// reductions.

// sum over the workgroup's 4 waves (wave order), broadcast to every thread
__device__ __forceinline__ float block_sum4(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__device__ __forceinline__ float block_max4(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(fmaxf(red[0], red[1]), red[2]), red[3]);
}

__device__ __forceinline__ float4 bf4(uint2 v) {
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}

// u = bf16(x / sqrt(mean(x^2) + eps) * gain) of the thread's chunks; with q8 also the e4m3 codes
// of the same fp32 values, quantised with the row scale amax / 448 (1 for an all-zero row, decided
// in binary32), and that scale.  red: 8 floats of LDS.
template <int NC>
__device__ __forceinline__ void row_norm(const float4 (&x)[NC], const uint2 (&gn)[NC], int d,
                                         float eps, uint16_t* u, uint8_t* q8, float* q8s,
                                         float* red) {
  const int c0 = threadIdx.x * 4;
  float ss = 0.f;
#pragma unroll
  for (int n = 0; n < NC; ++n)
    if (c0 + 1024 * n < d) {
      const float4 v = x[n];
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  const float rs = rsqrtf(block_sum4(ss, red) / d + eps);
  float4 y[NC];
  float amax = 0.f;
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    const int c = c0 + 1024 * n;
    if (c < d) {
      const float4 v = x[n], g = bf4(gn[n]);
      y[n] = make_float4(v.x * rs * g.x, v.y * rs * g.y, v.z * rs * g.z, v.w * rs * g.w);
      uint2 pk;
      pk.x = pack_bf2(y[n].x, y[n].y);
      pk.y = pack_bf2(y[n].z, y[n].w);
      *reinterpret_cast<uint2*>(u + c) = pk;
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(y[n].x), fabsf(y[n].y)),
                               fmaxf(fabsf(y[n].z), fabsf(y[n].w))));
    }
  }
  if (!q8) return;
  amax = block_max4(amax, red + 4);
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    const int c = c0 + 1024 * n;
    if (c < d)
      *reinterpret_cast<uint32_t*>(q8 + c) =
          f2e4m3(y[n].x / sc) | (f2e4m3(y[n].y / sc) << 8) | (f2e4m3(y[n].z / sc) << 16) |
          (f2e4m3(y[n].w / sc) << 24);
  }
  if (threadIdx.x == 0) *q8s = sc;
}

template <int NC>
__device__ __forceinline__ void load_gain(const uint16_t* gain, int d, uint2 (&gn)[NC]) {
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    const int c = threadIdx.x * 4 + 1024 * n;
    gn[n] = c < d ? *reinterpret_cast<const uint2*>(gain + c) : make_uint2(0u, 0u);
  }
}

// u = RMSNorm(h[t]) with the given gain
template <int NC>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* h, const uint16_t* gain, uint16_t* u,
                                                 int d, float eps, uint8_t* q8, float* q8s) {
  __shared__ float red[8];
  const int t = blockIdx.x, c0 = threadIdx.x * 4;
  const float* x = h + static_cast<long long>(t) * d;
  float4 v[NC];
  uint2 gn[NC];
#pragma unroll
  for (int n = 0; n < NC; ++n)
    if (c0 + 1024 * n < d) v[n] = *reinterpret_cast<const float4*>(x + c0 + 1024 * n);
  load_gain<NC>(gain, d, gn);
  row_norm<NC>(v, gn, d, eps, u + static_cast<long long>(t) * d,
               q8 ? q8 + static_cast<long long>(t) * d : nullptr, q8 ? q8s + t : nullptr, red);
}

// one wave per token; n_exp <= 64 KV <= 256, top_k <= 16.  The router logits arrive as ksplit
// fp32 partial planes [ksplit][ntok][n_exp], summed here in split order.  Selection by rank:
// expert e ranks behind every expert with a larger logit and every expert with an equal logit and
// a lower id (a NaN logit ranks as -inf, -0 as +0), so the experts of rank < top_k are the top-k
// in descending order with the lowest id first on ties, and each writes itself to slot rank.  The
// order is one unsigned comparison of 64-bit keys (an order-preserving image of the logit, then
// the complement of the id), and the ranks take one pass over the token's keys read back from
// LDS (every lane the same address) instead of top_k rounds of cross-lane reductions.
__device__ __forceinline__ uint64_t rank_key(float x, int e) {
  const float y = x != x ? -INFINITY : (x == 0.f ? 0.f : x);
  const uint32_t b = __float_as_uint(y);
  const uint32_t mono = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(mono) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}

template <int KV>
__global__ __launch_bounds__(256) void k_topk(const float* logits, int ksplit, int ntok,
                                              int n_exp, int top_k, int32_t* idx, float* gates,
                                              float* logits_out) {
  __shared__ __align__(16) uint64_t key[4][64 * KV];
  __shared__ float sel_val[4][16];
  __shared__ int sel_idx[4][16];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  const bool live = t < ntok;   // waves past the last token only join the barriers
  float v[KV];
  uint64_t my[KV];
#pragma unroll
  for (int k = 0; k < KV; ++k) {
    const int e = lane + 64 * k;
    float x = -INFINITY;
    if (live && e < n_exp) {
      // the k-split partial planes, summed in plane order; groups of 8 loads are issued
      // together (clamped plane index, zero weight past the last plane)
      x = 0.f;
      for (int sp0 = 0; sp0 < ksplit; sp0 += 8) {
        float part[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          part[u] = logits[(static_cast<long long>(min(sp0 + u, ksplit - 1)) * ntok + t) * n_exp + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) x += (sp0 + u < ksplit) ? part[u] : 0.f;
      }
      if (logits_out) logits_out[static_cast<long long>(t) * n_exp + e] = x;
    }
    v[k] = x;
    my[k] = e < n_exp ? rank_key(x, e) : 0ull;   // padding sorts below every expert
    key[w][e] = my[k];
  }
  __syncthreads();
  if (live) {
    int rank[KV];
#pragma unroll
    for (int k = 0; k < KV; ++k) rank[k] = 0;
    for (int e0 = 0; e0 < 64 * KV; e0 += 2) {
      const uint4 q = *reinterpret_cast<const uint4*>(&key[w][e0]);
      const uint64_t q0 = (static_cast<uint64_t>(q.y) << 32) | q.x;
      const uint64_t q1 = (static_cast<uint64_t>(q.w) << 32) | q.z;
#pragma unroll
      for (int k = 0; k < KV; ++k) rank[k] += (q0 > my[k]) + (q1 > my[k]);
    }
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      const int e = lane + 64 * k;
      if (e < n_exp && rank[k] < top_k) {
        sel_val[w][rank[k]] = v[k] != v[k] ? -INFINITY : v[k];
        sel_idx[w][rank[k]] = e;
      }
    }
  }
  __syncthreads();
  if (live && lane == 0) {
    // renormalised softmax weights: exp(r_j - r_max) / sum over the selected
    float s = 0.f;
    for (int j = 0; j < top_k; ++j) s += __expf(sel_val[w][j] - sel_val[w][0]);
    for (int j = 0; j < top_k; ++j) {
      idx[static_cast<long long>(t) * top_k + j] = sel_idx[w][j];
      gates[static_cast<long long>(t) * top_k + j] = __expf(sel_val[w][j] - sel_val[w][0]) / s;
    }
  }
}

// One workgroup of 1024 threads.  Pairs p = t * top_k + j are sorted stably by expert.  The
// expert counts are scanned into the experts' first rows; then, 2048 pairs at a time, every pair
// sets its bit in its expert's 2048-bit mask (LDS), one thread per expert turns its mask words
// into running popcount prefixes, and a pair's position is its expert's row offset plus the
// prefix of its word plus the bits below it in the word.  Rows [0, T k) hold the routed pairs
// sorted by (expert, p); rows [T k, T k + T) the shared expert's tokens.
constexpr int kPermBlock = 2048;          // pairs per mask block (2 per thread)
constexpr int kMaskStride = 68;           // words per expert row: 64 used, 16-byte aligned rows
                                          // on distinct bank groups
__global__ __launch_bounds__(1024) void k_permute(const int32_t* idx, int ntok, int top_k,
                                                  int n_exp, int tile_rows, int32_t* perm,
                                                  int32_t* inv, int32_t* chunks,
                                                  int32_t* n_chunks) {
  __shared__ int cnt[256];
  __shared__ int base[256];
  __shared__ int nch_off[257];
  __shared__ int row_off[257];
  __shared__ __align__(16) uint32_t mask[256 * kMaskStride];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int npairs = ntok * top_k;
  for (int e = tid; e < 256; e += 1024) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < npairs; p += 1024) atomicAdd(&cnt[idx[p]], 1);
  __syncthreads();
  // exclusive scans over the experts in one wave: first rows and tile offsets
  if (w == 0) {
    int run_rows = 0, run_tiles = 0;
    for (int e0 = 0; e0 < n_exp; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < n_exp ? cnt[e] : 0;
      const int nt = (c + tile_rows - 1) / tile_rows;
      int sr = c, st = nt;   // inclusive scans within the wave
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int ur = __shfl_up(sr, o, 64), ut = __shfl_up(st, o, 64);
        if (lane >= o) {
          sr += ur;
          st += ut;
        }
      }
      if (e < n_exp) {
        row_off[e] = base[e] = run_rows + sr - c;
        nch_off[e] = run_tiles + st - nt;
      }
      run_rows += __shfl(sr, 63, 64);
      run_tiles += __shfl(st, 63, 64);
    }
    if (lane == 0) {
      row_off[n_exp] = run_rows;
      nch_off[n_exp] = run_tiles;
    }
  }
  for (int blk = 0; blk < npairs; blk += kPermBlock) {
    for (int i = tid; i < n_exp * kMaskStride; i += 1024) mask[i] = 0u;
    __syncthreads();
    int pe[2], pw[2];
    uint32_t pbit[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = tid + 1024 * h;           // pair within the block
      const int p = blk + q;
      pe[h] = p < npairs ? idx[p] : -1;
      pw[h] = q >> 5;
      pbit[h] = 1u << (q & 31);
      if (pe[h] >= 0) atomicOr(&mask[pe[h] * kMaskStride + pw[h]], pbit[h]);
    }
    __syncthreads();
    uint32_t word[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) word[h] = pe[h] >= 0 ? mask[pe[h] * kMaskStride + pw[h]] : 0u;
    __syncthreads();
    if (tid < n_exp) {
      // the expert's 64 mask words -> exclusive running popcounts (in place); base advances
      uint4* row = reinterpret_cast<uint4*>(&mask[tid * kMaskStride]);
      uint4 m[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) m[i] = row[i];
      uint32_t run = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint4 o;
        o.x = run; run += __popc(m[i].x);
        o.y = run; run += __popc(m[i].y);
        o.z = run; run += __popc(m[i].z);
        o.w = run; run += __popc(m[i].w);
        row[i] = o;
      }
      cnt[tid] = static_cast<int>(run);   // this block's pairs of the expert
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (pe[h] < 0) continue;
      const int p = blk + tid + 1024 * h;
      const int pos = base[pe[h]] + static_cast<int>(mask[pe[h] * kMaskStride + pw[h]]) +
                      __popc(word[h] & (pbit[h] - 1u));
      perm[pos] = p / top_k;
      inv[p] = pos;
    }
    __syncthreads();
    if (tid < n_exp) base[tid] += cnt[tid];
  }
  for (int t = tid; t < ntok; t += 1024) perm[npairs + t] = t;
  __syncthreads();
  // tile list: ceil(n_e / tile_rows) tiles per expert in expert order, then the shared tiles;
  // one thread per (expert, tile range)
  for (int e = tid; e <= n_exp; e += 1024) {
    const int row0 = e < n_exp ? row_off[e] : npairs;
    const int n = e < n_exp ? row_off[e + 1] - row_off[e] : ntok;
    const int k0 = nch_off[e];
    for (int c = 0; c * tile_rows < n; ++c) {
      chunks[3 * (k0 + c)] = e;
      chunks[3 * (k0 + c) + 1] = row0 + c * tile_rows;
      chunks[3 * (k0 + c) + 2] = min(tile_rows, n - c * tile_rows);
    }
    if (e == n_exp) *n_chunks = k0 + (n + tile_rows - 1) / tile_rows;
  }
}

// h[t] += sum over k-splits of the projection partials (split order), then u = RMSNorm(h[t])
// with the given gain.  The partial planes are read in groups of 4 (clamped plane index, zero
// weight past the last plane), every load of a group issued together.
template <int NC>
__global__ __launch_bounds__(256) void k_resid_norm(float* h, const float* part, int ksplit,
                                                    int ntok, int d, const uint16_t* gain,
                                                    uint16_t* u, float eps, uint8_t* q8,
                                                    float* q8s) {
  __shared__ float red[8];
  const int t = blockIdx.x, c0 = threadIdx.x * 4;
  float* x = h + static_cast<long long>(t) * d;
  const long long plane = static_cast<long long>(ntok) * d;
  const float* pt = part + static_cast<long long>(t) * d + c0;
  float4 acc[NC];
  uint2 gn[NC];
#pragma unroll
  for (int n = 0; n < NC; ++n)
    if (c0 + 1024 * n < d) acc[n] = *reinterpret_cast<const float4*>(x + c0 + 1024 * n);
  load_gain<NC>(gain, d, gn);
  for (int sp0 = 0; sp0 < ksplit; sp0 += 4) {
    float4 p[4][NC];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int n = 0; n < NC; ++n)
        if (c0 + 1024 * n < d)
          p[q][n] = *reinterpret_cast<const float4*>(pt + min(sp0 + q, ksplit - 1) * plane + 1024 * n);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (sp0 + q < ksplit) {   // uniform; the loads above are already in flight
#pragma unroll
        for (int n = 0; n < NC; ++n) {
          acc[n].x += p[q][n].x;
          acc[n].y += p[q][n].y;
          acc[n].z += p[q][n].z;
          acc[n].w += p[q][n].w;
        }
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NC; ++n)
    if (c0 + 1024 * n < d) *reinterpret_cast<float4*>(x + c0 + 1024 * n) = acc[n];
  row_norm<NC>(acc, gn, d, eps, u + static_cast<long long>(t) * d,
               q8 ? q8 + static_cast<long long>(t) * d : nullptr, q8 ? q8s + t : nullptr, red);
}

// h[t] += sum_j gate_tj Y[row(t, j)] (j order) + Y[shared row of t], then optionally the next
// RMSNorm of the same row.  KM >= top_k: the routed rows are read for j < KM with the index
// clamped to top_k - 1, so every load is issued before the first use; rows j >= top_k are not
// added.
template <int NC, int KM>
__global__ __launch_bounds__(256) void k_combine(float* h, const uint16_t* Y, const int32_t* inv,
                                                 const float* gates, int ntok, int top_k, int d,
                                                 const uint16_t* next_gain, uint16_t* u_next,
                                                 float eps, uint8_t* q8, float* q8s) {
  __shared__ float red[8];
  const int t = blockIdx.x, c0 = threadIdx.x * 4;
  float* x = h + static_cast<long long>(t) * d;
  const int32_t* inv_t = inv + static_cast<long long>(t) * top_k;
  const float* g_t = gates + static_cast<long long>(t) * top_k;
  float4 acc[NC];
  uint2 y[KM][NC], ys[NC], gn[NC];
#pragma unroll
  for (int n = 0; n < NC; ++n)
    if (c0 + 1024 * n < d) acc[n] = *reinterpret_cast<const float4*>(x + c0 + 1024 * n);
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const uint16_t* yr = Y + static_cast<long long>(inv_t[min(j, top_k - 1)]) * d + c0;
#pragma unroll
    for (int n = 0; n < NC; ++n)
      if (c0 + 1024 * n < d) y[j][n] = *reinterpret_cast<const uint2*>(yr + 1024 * n);
  }
  const uint16_t* yrs = Y + (static_cast<long long>(ntok) * top_k + t) * d + c0;
#pragma unroll
  for (int n = 0; n < NC; ++n)
    if (c0 + 1024 * n < d) ys[n] = *reinterpret_cast<const uint2*>(yrs + 1024 * n);
  if (next_gain) load_gain<NC>(next_gain, d, gn);
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    if (c0 + 1024 * n >= d) continue;
    float4 mix = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < top_k) {   // uniform
        const float gj = g_t[j];
        const float4 v = bf4(y[j][n]);
        mix.x += gj * v.x;
        mix.y += gj * v.y;
        mix.z += gj * v.z;
        mix.w += gj * v.w;
      }
    }
    const float4 vs = bf4(ys[n]);
    acc[n].x += mix.x + vs.x;
    acc[n].y += mix.y + vs.y;
    acc[n].z += mix.z + vs.z;
    acc[n].w += mix.w + vs.w;
    *reinterpret_cast<float4*>(x + c0 + 1024 * n) = acc[n];
  }
  if (!next_gain) return;
  row_norm<NC>(acc, gn, d, eps, u_next + static_cast<long long>(t) * d,
               q8 ? q8 + static_cast<long long>(t) * d : nullptr, q8 ? q8s + t : nullptr, red);
}

struct KvWriteArgs {
  const uint16_t* qkv;
  uint16_t* kc;
  uint16_t* vc;
  int B, C, Hq, Hkv, dh, cap;
  int len[64];
};

__global__ __launch_bounds__(256) void k_kv_write(KvWriteArgs a) {
  const int per = a.dh / 8;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const long long total = static_cast<long long>(a.B) * a.C * a.Hkv * per;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % per) * 8;
  long long rest = idx / per;
  const int g = static_cast<int>(rest % a.Hkv);
  rest /= a.Hkv;
  const int i = static_cast<int>(rest % a.C);
  const int b = static_cast<int>(rest / a.C);
  const int ld = (a.Hq + 2 * a.Hkv) * a.dh;
  const uint16_t* src = a.qkv + (static_cast<long long>(b) * a.C + i) * ld;
  const long long dst = ((static_cast<long long>(b) * a.Hkv + g) * a.cap + a.len[b] + i) * a.dh + c;
  *reinterpret_cast<uint4*>(a.kc + dst) =
      *reinterpret_cast<const uint4*>(src + (a.Hq + g) * a.dh + c);
  *reinterpret_cast<uint4*>(a.vc + dst) =
      *reinterpret_cast<const uint4*>(src + (a.Hq + a.Hkv + g) * a.dh + c);
}

}  // namespace

hipError_t launch_embed(const int32_t* tokens, const uint16_t* embed, float* h, int ntok, int d,
                        int vocab, hipStream_t s, int C, int n_map, const int* map) {
  TokMap mp;
  mp.C = C;
  mp.n = n_map > 0 ? n_map : 0;
  for (int i = 0; i < mp.n && i < 64; ++i) mp.idx[i] = map[i];
  const long long n = static_cast<long long>(ntok) * (d / 8);
  hipLaunchKernelGGL(k_embed, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     tokens, embed, h, ntok, d, vocab, mp);
  return hipGetLastError();
}

// the row kernels are instantiated for NC = ceil(d / 1024) in 1..8
#define DG_ROW_SWITCH(d, CALL)                    \
  switch ((d + 1023) / 1024) {                    \
    case 1: { constexpr int NC = 1; CALL; } break; \
    case 2: { constexpr int NC = 2; CALL; } break; \
    case 3: { constexpr int NC = 3; CALL; } break; \
    case 4: { constexpr int NC = 4; CALL; } break; \
    case 5: { constexpr int NC = 5; CALL; } break; \
    case 6: { constexpr int NC = 6; CALL; } break; \
    case 7: { constexpr int NC = 7; CALL; } break; \
    case 8: { constexpr int NC = 8; CALL; } break; \
    default: return hipErrorInvalidValue;         \
  }

hipError_t launch_rmsnorm(const float* h, const uint16_t* gain, uint16_t* u, int ntok, int d,
                          float eps, uint8_t* q8, float* q8s, hipStream_t s) {
  if (ntok <= 0) return hipSuccess;
  DG_ROW_SWITCH(d, hipLaunchKernelGGL(k_rmsnorm<NC>, dim3(ntok), dim3(256), 0, s, h, gain, u, d,
                                      eps, q8, q8s))
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int ksplit, int ntok, int n_exp, int top_k,
                       int32_t* idx, float* gates, float* logits_out, hipStream_t s) {
  if (ntok <= 0) return hipSuccess;
  const dim3 grid((ntok + 3) / 4);
  switch ((n_exp + 63) / 64) {
    case 1: hipLaunchKernelGGL(k_topk<1>, grid, dim3(256), 0, s, logits, ksplit, ntok, n_exp, top_k,
                               idx, gates, logits_out); break;
    case 2: hipLaunchKernelGGL(k_topk<2>, grid, dim3(256), 0, s, logits, ksplit, ntok, n_exp, top_k,
                               idx, gates, logits_out); break;
    case 3: hipLaunchKernelGGL(k_topk<3>, grid, dim3(256), 0, s, logits, ksplit, ntok, n_exp, top_k,
                               idx, gates, logits_out); break;
    case 4: hipLaunchKernelGGL(k_topk<4>, grid, dim3(256), 0, s, logits, ksplit, ntok, n_exp, top_k,
                               idx, gates, logits_out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_resid_norm(float* h, const float* part, int ksplit, int ntok, int d,
                             const uint16_t* gain, uint16_t* u, float eps, uint8_t* q8,
                             float* q8s, hipStream_t s) {
  if (ntok <= 0) return hipSuccess;
  DG_ROW_SWITCH(d, hipLaunchKernelGGL(k_resid_norm<NC>, dim3(ntok), dim3(256), 0, s, h, part,
                                      ksplit, ntok, d, gain, u, eps, q8, q8s))
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int ntok, int top_k, int n_exp, int tile_rows,
                          int32_t* perm, int32_t* inv, int32_t* chunks, int32_t* n_chunks,
                          int max_chunks, hipStream_t s) {
  (void)max_chunks;
  hipLaunchKernelGGL(k_permute, dim3(1), dim3(1024), 0, s, idx, ntok, top_k, n_exp, tile_rows,
                     perm, inv, chunks, n_chunks);
  return hipGetLastError();
}

hipError_t launch_combine(float* h, const uint16_t* Y, const int32_t* inv, const float* gates,
                          int ntok, int top_k, int d, const uint16_t* next_gain,
                          uint16_t* u_next, float eps, uint8_t* q8, float* q8s, hipStream_t s) {
  if (ntok <= 0) return hipSuccess;
  if (top_k <= 8) {
    DG_ROW_SWITCH(d, hipLaunchKernelGGL((k_combine<NC, 8>), dim3(ntok), dim3(256), 0, s, h, Y, inv,
                                        gates, ntok, top_k, d, next_gain, u_next, eps, q8, q8s))
  } else {
    DG_ROW_SWITCH(d, hipLaunchKernelGGL((k_combine<NC, 16>), dim3(ntok), dim3(256), 0, s, h, Y,
                                        inv, gates, ntok, top_k, d, next_gain, u_next, eps, q8,
                                        q8s))
  }
  return hipGetLastError();
}

hipError_t launch_kv_write(const uint16_t* qkv, uint16_t* kc, uint16_t* vc, int B, int C, int Hq,
                           int Hkv, int dh, int cap, const int* len, hipStream_t s) {
  KvWriteArgs a;
  a.qkv = qkv;
  a.kc = kc;
  a.vc = vc;
  a.B = B;
  a.C = C;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.dh = dh;
  a.cap = cap;
  for (int b = 0; b < B && b < 64; ++b) a.len[b] = len[b];
  const long long n = static_cast<long long>(B) * C * Hkv * (dh / 8);
  hipLaunchKernelGGL(k_kv_write, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dg
