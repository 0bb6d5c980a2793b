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

// token ids outside [0, vocab) are clamped into range (no out-of-bounds gather)
__global__ __launch_bounds__(256) void k_embed(const int32_t* tokens, const uint16_t* embed,
                                               float* h, int ntok, int d, int vocab) {
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const int per = d / 8;
  if (idx >= static_cast<long long>(ntok) * per) return;
  const int t = static_cast<int>(idx / per), c = static_cast<int>(idx % per) * 8;
  const int tok = min(max(tokens[t], 0), vocab - 1);
  const uint4 v = *reinterpret_cast<const uint4*>(embed + static_cast<long long>(tok) * d + c);
  float4* o = reinterpret_cast<float4*>(h + static_cast<long long>(t) * d + c);
  o[0] = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
  o[1] = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xffff0000u),
                     __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xffff0000u));
}

__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int k = 0; k < static_cast<int>(blockDim.x >> 6); ++k) s += red[k];
  return s;
}

__device__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float m = 0.f;
  for (int k = 0; k < static_cast<int>(blockDim.x >> 6); ++k) m = fmaxf(m, red[k]);
  return m;
}

// four normed values x * rs * gain of row x at column c
__device__ __forceinline__ float4 normed4(const float* x, float rs, const uint16_t* gain, int c) {
  const float4 v = *reinterpret_cast<const float4*>(x + c);
  const uint2 gg = *reinterpret_cast<const uint2*>(gain + c);
  return make_float4(v.x * rs * __uint_as_float(gg.x << 16), v.y * rs * __uint_as_float(gg.x & 0xffff0000u),
                     v.z * rs * __uint_as_float(gg.y << 16), v.w * rs * __uint_as_float(gg.y & 0xffff0000u));
}

// Writes u = bf16(x * rs * gain) for one row (the whole workgroup); with q8, also the e4m3
// codes of the same fp32 values, quantised with the row scale amax / 448 (1 for an all-zero
// row), and that scale.  The quantisation is decided in binary32.
__device__ void norm_out(const float* x, float rs, const uint16_t* gain, uint16_t* o, int d,
                         uint8_t* q8, float* q8s, float* red) {
  float amax = 0.f;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const float4 y = normed4(x, rs, gain, c);
    uint2 pk;
    pk.x = pack_bf2(y.x, y.y);
    pk.y = pack_bf2(y.z, y.w);
    *reinterpret_cast<uint2*>(o + c) = pk;
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w))));
  }
  if (!q8) return;
  amax = block_max(amax, red);
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const float4 y = normed4(x, rs, gain, c);
    *reinterpret_cast<uint32_t*>(q8 + c) = f2e4m3(y.x / sc) | (f2e4m3(y.y / sc) << 8) |
                                           (f2e4m3(y.z / sc) << 16) | (f2e4m3(y.w / sc) << 24);
  }
  if (threadIdx.x == 0) *q8s = sc;
}

// one workgroup per token
__global__ __launch_bounds__(256) void k_rmsnorm(const float* h, const uint16_t* gain, uint16_t* u,
                                                 int d, float eps, uint8_t* q8, float* q8s) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const float* x = h + static_cast<long long>(t) * d;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(x + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  const float rs = rsqrtf(block_sum(ss, red) / d + eps);
  norm_out(x, rs, gain, u + static_cast<long long>(t) * d, d,
           q8 ? q8 + static_cast<long long>(t) * d : nullptr, q8 ? q8s + t : nullptr, red);
}

// one wave per token; n_exp <= 256, top_k <= 16.  The router logits arrive as ksplit fp32
// partial planes [ksplit][ntok][n_exp], summed here in split order.
__global__ __launch_bounds__(256) void k_topk(const float* logits, int ksplit, int ntok,
                                              int n_exp, int top_k, int32_t* idx, float* gates,
                                              float* logits_out) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= ntok) return;
  float v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = lane + 64 * k;
    float x = -INFINITY;
    if (e < n_exp) {
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
  }
  float sel_val[16];
  int sel_idx[16];
  for (int j = 0; j < top_k; ++j) {
    // (max value, lowest index) over the remaining entries
    float bv = v[0];
    int bi = lane;
#pragma unroll
    for (int k = 1; k < 4; ++k)
      if (v[k] > bv) {
        bv = v[k];
        bi = lane + 64 * k;
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    sel_val[j] = bv;
    sel_idx[j] = bi;
    if ((bi & 63) == lane) v[bi >> 6] = -INFINITY;
  }
  if (lane == 0) {
    // renormalised softmax weights: exp(r_j - r_max) / sum over the selected
    float s = 0.f;
    for (int j = 0; j < top_k; ++j) s += __expf(sel_val[j] - sel_val[0]);
    for (int j = 0; j < top_k; ++j) {
      idx[static_cast<long long>(t) * top_k + j] = sel_idx[j];
      gates[static_cast<long long>(t) * top_k + j] = __expf(sel_val[j] - sel_val[0]) / s;
    }
  }
}

// One workgroup of 1024 threads.  Pairs p = t * top_k + j (in p order) are ranked within their
// expert: a 1024-pair block is split in 16 wave segments; inside a segment lanes with the same
// expert are ranked with ballots; segment counts are scanned per expert.  Rows [0, T k) hold
// the routed pairs sorted by (expert, p); rows [T k, T k + T) the shared expert's tokens.
__global__ __launch_bounds__(1024) void k_permute(const int32_t* idx, int ntok, int top_k,
                                                  int n_exp, int tile_rows, int32_t* perm,
                                                  int32_t* inv, int32_t* chunks,
                                                  int32_t* n_chunks) {
  __shared__ int cnt[256];
  __shared__ int base[256];
  __shared__ int wcnt[16][256];
  __shared__ int nch_off[257];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int npairs = ntok * top_k;
  for (int e = tid; e < 256; e += 1024) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < npairs; p += 1024) atomicAdd(&cnt[idx[p]], 1);
  __syncthreads();
  if (w == 0) {  // exclusive scan of the expert counts in one wave
    int run = 0;
    for (int e0 = 0; e0 < n_exp; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < n_exp ? cnt[e] : 0;
      int sc = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(sc, o, 64);
        if (lane >= o) sc += u;
      }
      if (e < n_exp) base[e] = run + sc - c;
      run += __shfl(sc, 63, 64);
    }
  }
  __syncthreads();
  for (int blk = 0; blk < npairs; blk += 1024) {
    for (int e = tid; e < 16 * 256; e += 1024) wcnt[e >> 8][e & 255] = 0;
    __syncthreads();
    const int p = blk + tid;
    const bool ok = p < npairs;
    const int e = ok ? idx[p] : -1;
    uint64_t todo = __ballot(ok);
    int rank = 0;
    while (todo) {
      const int leader = __ffsll(static_cast<unsigned long long>(todo)) - 1;
      const int le = __shfl(e, leader, 64);
      const uint64_t m = __ballot(e == le);
      if (e == le) rank = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == leader) wcnt[w][le] = __popcll(m);
      todo &= ~m;
    }
    __syncthreads();
    // per-expert exclusive scan over the 16 segments, then advance the expert's base
    for (int ex = tid; ex < n_exp; ex += 1024) {
      int s = base[ex];
      for (int k = 0; k < 16; ++k) {
        const int c = wcnt[k][ex];
        wcnt[k][ex] = s;
        s += c;
      }
      base[ex] = s;
    }
    __syncthreads();
    if (ok) {
      const int pos = wcnt[w][e] + rank;
      perm[pos] = p / top_k;
      inv[p] = pos;
    }
    __syncthreads();
  }
  for (int t = tid; t < ntok; t += 1024) perm[npairs + t] = t;
  // tile list: ceil(n_e / tile_rows) tiles per expert in expert order, then the shared tiles.
  // Exclusive scans over the experts (row offsets and tile offsets) in one wave.
  __shared__ int row_off[257];
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
        row_off[e] = run_rows + sr - c;
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
  __syncthreads();
  // one thread per (expert, tile): experts use their own tile range
  for (int e = tid; e <= n_exp; e += 1024) {
    const int row0 = e < n_exp ? row_off[e] : npairs;
    const int n = e < n_exp ? cnt[e] : ntok;
    const int k0 = nch_off[e];
    for (int c = 0; c * tile_rows < n; ++c) {
      chunks[3 * (k0 + c)] = e;
      chunks[3 * (k0 + c) + 1] = row0 + c * tile_rows;
      chunks[3 * (k0 + c) + 2] = min(tile_rows, n - c * tile_rows);
    }
    if (e == n_exp) *n_chunks = k0 + (n + tile_rows - 1) / tile_rows;
  }
}

// one workgroup per token: h[t] += sum over k-splits of the projection partials (split order),
// then u = RMSNorm(h[t]) with the given gain
__global__ __launch_bounds__(256) void k_resid_norm(float* h, const float* part, int ksplit,
                                                    int ntok, int d, const uint16_t* gain,
                                                    uint16_t* u, float eps, uint8_t* q8,
                                                    float* q8s) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  float* x = h + static_cast<long long>(t) * d;
  const long long plane = static_cast<long long>(ntok) * d;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    float4 acc = *reinterpret_cast<const float4*>(x + c);
    // the k-split partial planes, added in plane order; each group of 4 loads is issued
    // together (clamped plane index, zero weight past the last plane)
    for (int sp0 = 0; sp0 < ksplit; sp0 += 4) {
      float4 p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        p[u] = *reinterpret_cast<const float4*>(part + min(sp0 + u, ksplit - 1) * plane +
                                                static_cast<long long>(t) * d + c);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (sp0 + u < ksplit) {   // uniform; the loads above are already in flight
          acc.x += p[u].x;
          acc.y += p[u].y;
          acc.z += p[u].z;
          acc.w += p[u].w;
        }
      }
    }
    *reinterpret_cast<float4*>(x + c) = acc;
    ss += acc.x * acc.x + acc.y * acc.y + acc.z * acc.z + acc.w * acc.w;
  }
  const float rs = rsqrtf(block_sum(ss, red) / d + eps);
  norm_out(x, rs, gain, u + static_cast<long long>(t) * d, d,
           q8 ? q8 + static_cast<long long>(t) * d : nullptr, q8 ? q8s + t : nullptr, red);
}

// one workgroup per token
__global__ __launch_bounds__(256) void k_combine(float* h, const uint16_t* Y, const int32_t* inv,
                                                 const float* gates, int ntok, int top_k, int d,
                                                 const uint16_t* next_gain, uint16_t* u_next,
                                                 float eps, uint8_t* q8, float* q8s) {
  __shared__ float red[4];
  __shared__ int rows[17];
  __shared__ float gw[16];
  const int t = blockIdx.x;
  if (threadIdx.x < top_k) {
    rows[threadIdx.x] = inv[static_cast<long long>(t) * top_k + threadIdx.x];
    gw[threadIdx.x] = gates[static_cast<long long>(t) * top_k + threadIdx.x];
  }
  if (threadIdx.x == 0) rows[top_k] = ntok * top_k + t;  // shared expert row
  __syncthreads();
  float* x = h + static_cast<long long>(t) * d;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    float4 acc = *reinterpret_cast<const float4*>(x + c);
    float4 mix = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < top_k; ++j) {
      const uint2 y = *reinterpret_cast<const uint2*>(Y + static_cast<long long>(rows[j]) * d + c);
      const float gj = gw[j];
      mix.x += gj * __uint_as_float(y.x << 16);
      mix.y += gj * __uint_as_float(y.x & 0xffff0000u);
      mix.z += gj * __uint_as_float(y.y << 16);
      mix.w += gj * __uint_as_float(y.y & 0xffff0000u);
    }
    const uint2 ys = *reinterpret_cast<const uint2*>(Y + static_cast<long long>(rows[top_k]) * d + c);
    acc.x += mix.x + __uint_as_float(ys.x << 16);
    acc.y += mix.y + __uint_as_float(ys.x & 0xffff0000u);
    acc.z += mix.z + __uint_as_float(ys.y << 16);
    acc.w += mix.w + __uint_as_float(ys.y & 0xffff0000u);
    *reinterpret_cast<float4*>(x + c) = acc;
    ss += acc.x * acc.x + acc.y * acc.y + acc.z * acc.z + acc.w * acc.w;
  }
  if (!next_gain) return;
  const float rs = rsqrtf(block_sum(ss, red) / d + eps);
  norm_out(x, rs, next_gain, u_next + static_cast<long long>(t) * d, d,
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
                        int vocab, hipStream_t s) {
  const long long n = static_cast<long long>(ntok) * (d / 8);
  hipLaunchKernelGGL(k_embed, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     tokens, embed, h, ntok, d, vocab);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* h, const uint16_t* gain, uint16_t* u, int ntok, int d,
                          float eps, uint8_t* q8, float* q8s, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(ntok), dim3(256), 0, s, h, gain, u, d, eps, q8, q8s);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int ksplit, int ntok, int n_exp, int top_k,
                       int32_t* idx, float* gates, float* logits_out, hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3((ntok + 3) / 4), dim3(256), 0, s, logits, ksplit, ntok, n_exp,
                     top_k, idx, gates, logits_out);
  return hipGetLastError();
}

hipError_t launch_resid_norm(float* h, const float* part, int ksplit, int ntok, int d,
                             const uint16_t* gain, uint16_t* u, float eps, uint8_t* q8,
                             float* q8s, hipStream_t s) {
  hipLaunchKernelGGL(k_resid_norm, dim3(ntok), dim3(256), 0, s, h, part, ksplit, ntok, d, gain, u,
                     eps, q8, q8s);
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
  hipLaunchKernelGGL(k_combine, dim3(ntok), dim3(256), 0, s, h, Y, inv, gates, ntok, top_k, d,
                     next_gain, u_next, eps, q8, q8s);
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
