// Entropy-bound sampler kernels (DiffusionGemma model card, Best Practices section 1; diffusers
// DiffusionGemmaPipeline docs, "Schedulers" and "Adaptive stopping").
//
//   logit_stats  bf16 logits -> per-(row, chunk) softmax statistics of y = z / T_s   (HBM bound)
//   stats_merge  chunk statistics -> entropy (nats) and argmax per position
//   eb_commit    one workgroup per canvas: stability, stop / finalise, stable sort of the
//                uncommitted entropies, fp64 running sum against the bound, Philox renoise
//   candidates   Gumbel-max draw over the vocabulary, only for rows committed by the bound
//   cand_apply   merge the candidate partials and write the committed tokens
//   canvas_init  uniform placeholder tokens (uniform corruption, no mask token)
#include <float.h>

#include "dg_internal.h"

namespace dg {

namespace {

constexpr int kStatsThreads = 64;    // one wave per statistics workgroup
constexpr int kStatsChunk = 4096;    // vocabulary entries per statistics workgroup (8 groups of 8 per lane)
constexpr int kCandThreads = 256;
constexpr int kCandChunk = 4096;     // vocabulary entries per candidate workgroup

constexpr int kStatsGroups = kStatsChunk / (kStatsThreads * 8);   // groups of 8 per thread

__device__ __forceinline__ void unpack8(const uint4 raw, float (&z)[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    z[2 * k] = __uint_as_float(w[k] << 16);
    z[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}

// Batch map of a compacted step: compact canvas b of the call is canvas map_b(b) of the state,
// outputs and logits; the workspace arrays (partials, flags, candidates) stay compact.
__device__ __forceinline__ int map_b(const EbArgs& a, int b) { return a.mapped ? a.bmap[b] : b; }
__device__ __forceinline__ size_t map_row(const EbArgs& a, int row) {
  return a.mapped ? static_cast<size_t>(a.bmap[row / a.C]) * a.C + row % a.C
                  : static_cast<size_t>(row);
}

__device__ __forceinline__ SoftStats stats_empty() { return SoftStats{-INFINITY, 0x7fffffff, 0.f, 0.f}; }

__device__ __forceinline__ SoftStats stats_merge_nan(SoftStats x, SoftStats y) {
  const bool nan = isnan(x.r) || isnan(y.r);
  SoftStats w = stats_merge(x, y);
  if (nan) w.r = NAN;
  return w;
}

// workgroup-wide merge of per-thread statistics (fixed tree order); result valid in thread 0
__device__ SoftStats stats_block_reduce(SoftStats s) {
  __shared__ SoftStats red[kStatsThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s = stats_merge_nan(s, stats_shfl_xor(s, o));
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) red[wv] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < static_cast<int>(blockDim.x >> 6); ++k) s = stats_merge_nan(s, red[k]);
  }
  return s;
}

// Statistics of one thread's entries of a chunk: its groups of 8 (group g at v0 + (g * threads +
// thread) * 8, ascending in g) are all loaded first; pass 1 finds the thread's maximum M of z and
// the first group G holding it; pass 2 sums 2^d and d 2^d (d = z c - M c, one fma, hardware exp2
// with d <= 0) over the other groups against that final maximum, so no rescaling and no
// per-entry test is needed (group G's offset is a huge negative number, which sends its terms to
// 0); group G is then re-read (from L2) and folded with its first maximum left out of the sums,
// which gives the index (lowest on ties) and keeps R = sum over the other entries exact to
// rounding however small it is.  Non-finite inputs need no separate test: +inf makes d = inf -
// inf, a NaN propagates, and -inf gives d * e = -inf * 0, so r or a ends NaN (checked once per
// thread).  FULL: the chunk holds kStatsChunk entries (every group is in range).
template <bool FULL>
__device__ __forceinline__ SoftStats chunk_stats(const uint16_t* z, int v0, int v1, float c) {
  constexpr int NG = kStatsGroups;
  const int tid = threadIdx.x;
  auto base = [&](int g) { return v0 + (g * kStatsThreads + tid) * 8; };
  auto valid = [&](int g) { return FULL || base(g) < v1; };
  if (!valid(0)) return stats_empty();          // no entries for this thread
  uint4 raw[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g)
    raw[g] = *reinterpret_cast<const uint4*>(z + (FULL ? base(g) : min(base(g), v1 - 8)));
  // pass 1
  float gmax[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float x[8];
    unpack8(raw[g], x);
    const float gm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                           fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    gmax[g] = valid(g) ? gm : -INFINITY;
  }
  float M = gmax[0];
#pragma unroll
  for (int g = 1; g < NG; ++g) M = fmaxf(M, gmax[g]);
  int G = NG - 1;
#pragma unroll
  for (int g = NG - 2; g >= 0; --g) G = (gmax[g] == M) ? g : G;
  const int vG = min(base(G), v1 - 8);
  const uint4 rawG = *reinterpret_cast<const uint4*>(z + vG);   // in flight during pass 2
  // pass 2
  const float neg_m = -(M * c);
  float r = 0.f, acc = 0.f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float x[8];
    unpack8(raw[g], x);
    const float nm = (g == G || !valid(g)) ? -3.0e38f : neg_m;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float d = __builtin_fmaf(x[k], c, nm);
      const float e = __builtin_amdgcn_exp2f(d);
      r += e;
      acc = __builtin_fmaf(d, e, acc);
    }
  }
  // group G
  float x[8];
  unpack8(rawG, x);
  int gi = 7;
#pragma unroll
  for (int k = 6; k >= 0; --k) gi = (x[k] == M) ? k : gi;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float d = __builtin_fmaf(x[k], c, neg_m);
    const float e = (k == gi) ? 0.f : __builtin_amdgcn_exp2f(d);
    r += e;
    acc = __builtin_fmaf(d, e, acc);
  }
  SoftStats st;
  st.m = -neg_m;
  st.idx = vG + gi;
  st.r = (r != r || acc != acc) ? NAN : r;
  st.a = acc;
  return st;
}

__global__ __launch_bounds__(kStatsThreads) void k_logit_stats(EbArgs a) {
  const int row = blockIdx.x;
  const int chunk = blockIdx.y;
  const int v0 = chunk * kStatsChunk;
  const int v1 = min(a.V, v0 + kStatsChunk);
  const uint16_t* z = a.logits + static_cast<size_t>(row) * a.V;
  SoftStats s = (v1 - v0 == kStatsChunk) ? chunk_stats<true>(z, v0, v1, a.inv_t_log2e)
                                         : chunk_stats<false>(z, v0, v1, a.inv_t_log2e);
  s = stats_block_reduce(s);
  if (threadIdx.x == 0) a.part[static_cast<size_t>(row) * a.n_part + chunk] = s;
}

// one wave per row
__global__ __launch_bounds__(256) void k_stats_merge(EbArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.B * a.C) return;
  const SoftStats* p = a.part + static_cast<size_t>(row) * a.n_part;
  SoftStats s = stats_empty();
  for (int k = lane; k < a.n_part; k += 64) s = stats_merge_nan(s, p[k]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s = stats_merge_nan(s, stats_shfl_xor(s, o));
  if (lane == 0) {
    float h = log1pf(s.r) - 0.69314718055994531f * s.a / (1.0f + s.r);
    h = (h < 0.f) ? 0.f : h;  // keeps NaN
    const size_t rr = map_row(a, row);
    a.out.entropy[rr] = h;
    a.out.argmax[rr] = s.idx;
    if (a.row) a.row[row] = s;
  }
}

// one workgroup of 1024 threads per canvas; position i = thread i (C <= 1024)
__global__ __launch_bounds__(1024) void k_eb_commit(EbArgs a) {
  __shared__ uint64_t keys[1024];
  __shared__ double dsum[1024];
  __shared__ uint8_t sel[1024];
  __shared__ int n_sel;
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool live = i < a.C;
  const size_t at = static_cast<size_t>(b) * a.C + i;
  const int rb = map_b(a, b);
  const size_t ra = static_cast<size_t>(rb) * a.C + i;
  const int32_t* done_p = a.st.done + rb;
  if (*done_p) {  // a frozen canvas never changes
    if (live) {
      a.out.commit_now[ra] = 0;
      a.need_cand[at] = 0;
    }
    return;
  }
  const float h = live ? a.out.entropy[ra] : 0.f;
  const int am = live ? a.out.argmax[ra] : 0;
  const bool committed = live ? (a.st.committed[ra] != 0) : true;
  const int prev = live ? a.st.prev_argmax[ra] : 0;

  const int bad = __syncthreads_or(live && !(fabsf(h) <= FLT_MAX));
  if (bad) {  // non-finite logits: sticky status, the canvas is frozen unchanged
    if (live) {
      a.out.commit_now[ra] = 0;
      a.need_cand[at] = 0;
    }
    if (i == 0) {
      if (a.st.dev_status) atomicExch(a.st.dev_status, static_cast<int>(DG_ERR_NONFINITE));
      a.st.done[rb] = 1;
    }
    return;
  }
  const int all_same = __syncthreads_and(!live || am == prev);
  const int stable = (a.step >= 1 && all_same) ? a.st.stable_count[rb] + 1 : 0;
  if (live) a.st.prev_argmax[ra] = am;

  // mean entropy: fp64 sum in a fixed tree order
  dsum[i] = live ? static_cast<double>(h) : 0.0;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (i < o) dsum[i] += dsum[i + o];
    __syncthreads();
  }
  const double mean_h = dsum[0] / a.C;
  const int any_unc = __syncthreads_or(live && !committed);
  const bool stop = a.stop_entropy >= 0.0 && stable >= a.stability && mean_h < a.stop_entropy;
  if (i == 0) a.st.stable_count[rb] = stable;

  if (stop || a.step == a.max_steps - 1 || !any_unc) {  // finalise: remaining take the argmax
    if (live) {
      a.need_cand[at] = 0;
      if (!committed) {
        a.st.canvas[ra] = am;
        a.st.committed[ra] = 1;
        a.out.commit_now[ra] = 1;
      } else {
        a.out.commit_now[ra] = 0;
      }
    }
    if (i == 0) a.st.done[rb] = 1;
    return;
  }

  // ascending (entropy, position) order of the uncommitted positions; entropies are >= 0,
  // so their binary32 patterns order like their values
  keys[i] = (live && !committed)
                ? ((static_cast<uint64_t>(__float_as_uint(h)) << 32) | static_cast<uint32_t>(i))
                : ~0ull;
  sel[i] = 0;
  __syncthreads();
  for (int k = 2; k <= 1024; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int p = i ^ j;
      if (p > i) {
        const uint64_t x = keys[i], y = keys[p];
        const bool up = (i & k) == 0;
        if ((x > y) == up) {
          keys[i] = y;
          keys[p] = x;
        }
      }
      __syncthreads();
    }
  }
  if (i == 0) {  // longest prefix whose fp64 running sum stays <= bound (sequential order)
    double acc = 0.0;
    int n = 0;
    for (; n < 1024; ++n) {
      const uint64_t kk = keys[n];
      if (kk == ~0ull) break;
      const double hv = static_cast<double>(__uint_as_float(static_cast<uint32_t>(kk >> 32)));
      if (acc + hv <= a.bound) {
        acc += hv;
      } else {
        break;
      }
    }
    n_sel = n;
  }
  __syncthreads();
  if (i < n_sel) sel[static_cast<uint32_t>(keys[i])] = 1;
  __syncthreads();
  const bool chosen = live && sel[i];
  if (live) {
    if (!committed) {
      if (chosen) {
        a.need_cand[at] = 1;
        a.out.commit_now[ra] = 1;
        a.st.committed[ra] = 1;
      } else {  // full renoise: a fresh uniform token
        a.need_cand[at] = 0;
        a.out.commit_now[ra] = 0;
        a.st.canvas[ra] = uniform_token(a.seed, a.st.canvas_id[rb], static_cast<uint32_t>(a.step),
                                        static_cast<uint32_t>(i), static_cast<uint32_t>(a.V));
      }
    } else {
      a.need_cand[at] = 0;
      a.out.commit_now[ra] = 0;
    }
  }
  const int all_committed = __syncthreads_and(!live || committed || chosen);
  if (i == 0 && all_committed) a.st.done[rb] = 1;
}

// Gumbel-max over one vocabulary chunk of one row: score_v = z_v * (1/T) + g_v in fp64,
// g_v = -ln(-ln u_v), u_v = (x_v + 0.5) 2^-32 from Philox stream 1, word v & 3 of counter
// (v >> 2, position, step, (canvas_id << 1) | 1).
__global__ __launch_bounds__(kCandThreads) void k_candidates(EbArgs a) {
  const int row = blockIdx.x;
  if (!a.need_cand[row]) return;
  const int chunk = blockIdx.y;
  const int b = row / a.C, pos = row % a.C;
  const uint32_t cid = a.st.canvas_id[map_b(a, b)];
  const uint32_t k0 = static_cast<uint32_t>(a.seed), k1 = static_cast<uint32_t>(a.seed >> 32);
  const uint16_t* z = a.logits + map_row(a, row) * a.V;
  const double inv_t = static_cast<double>(a.inv_t);
  const int v0 = chunk * kCandChunk;
  const int v1 = min(a.V, v0 + kCandChunk);
  double best = -INFINITY;
  int best_v = 0x7fffffff;
  for (int v = v0 + threadIdx.x * 8; v < v1; v += kCandThreads * 8) {
    const uint4 raw = *reinterpret_cast<const uint4*>(z + v);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    const Philox4 r0 = philox10(static_cast<uint32_t>(v >> 2), pos, a.step, (cid << 1) | 1u, k0, k1);
    const Philox4 r1 = philox10(static_cast<uint32_t>((v >> 2) + 1), pos, a.step, (cid << 1) | 1u,
                                k0, k1);
    const uint32_t x[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float zf = __uint_as_float(k & 1 ? (w[k >> 1] & 0xffff0000u) : (w[k >> 1] << 16));
      const double u = (static_cast<double>(x[k]) + 0.5) * 0x1p-32;
      const double g = -log(-log(u));
      const double sc = static_cast<double>(zf) * inv_t + g;
      if (sc > best) {
        best = sc;
        best_v = v + k;
      }
    }
  }
  // reduce (max score, lowest index)
  __shared__ double rs[kCandThreads / 64];
  __shared__ int ri[kCandThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double ob = __shfl_xor(best, o, 64);
    const int ov = __shfl_xor(best_v, o, 64);
    if (ob > best || (ob == best && ov < best_v)) {
      best = ob;
      best_v = ov;
    }
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) {
    rs[wv] = best;
    ri[wv] = best_v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kCandThreads / 64; ++k) {
      if (rs[k] > best || (rs[k] == best && ri[k] < best_v)) {
        best = rs[k];
        best_v = ri[k];
      }
    }
    a.cand_score[static_cast<size_t>(row) * a.n_cand_chunks + chunk] = best;
    a.cand_idx[static_cast<size_t>(row) * a.n_cand_chunks + chunk] = best_v;
  }
}

__global__ __launch_bounds__(256) void k_cand_apply(EbArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.B * a.C || !a.need_cand[row]) return;
  double best = -INFINITY;
  int best_v = 0x7fffffff;
  for (int k = lane; k < a.n_cand_chunks; k += 64) {
    const double sc = a.cand_score[static_cast<size_t>(row) * a.n_cand_chunks + k];
    const int v = a.cand_idx[static_cast<size_t>(row) * a.n_cand_chunks + k];
    if (sc > best || (sc == best && v < best_v)) {
      best = sc;
      best_v = v;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double ob = __shfl_xor(best, o, 64);
    const int ov = __shfl_xor(best_v, o, 64);
    if (ob > best || (ob == best && ov < best_v)) {
      best = ob;
      best_v = ov;
    }
  }
  if (lane == 0) {
    if (a.kind == SCHED_BLOCK_REFINEMENT)
      a.cand[row] = best_v;       // the commit kernel decides whether it is taken
    else
      a.st.canvas[map_row(a, row)] = best_v;  // entropy bound: committed rows; DDIM: new token
  }
}

// ---- block refinement and DDIM -----------------------------------------------------------------
// (diffusers DiffusionGemmaPipeline docs, "Schedulers" and "Predictor-corrector sampling")

// ascending bitonic sort of 1024 keys in LDS by a workgroup of 1024 threads
__device__ __forceinline__ void sort1024(uint64_t* keys) {
  const int i = threadIdx.x;
  __syncthreads();
  for (int k = 2; k <= 1024; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int p = i ^ j;
      if (p > i) {
        const uint64_t x = keys[i], y = keys[p];
        const bool up = (i & k) == 0;
        if ((x > y) == up) {
          keys[i] = y;
          keys[p] = x;
        }
      }
      __syncthreads();
    }
  }
}

// p(v) of a row under softmax(z * inv_t) from its merged statistics (log2 units): one fp32 exp2
__device__ __forceinline__ float row_prob(float zv, float c, const SoftStats& st) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(zv, c, -st.m)) / (1.0f + st.r);
}

// One workgroup of 1024 threads per canvas: stability, the adaptive stop and finalisation (the
// pipeline's rule, as for the entropy bound), then which rows draw a token this step.
//   block refinement: every uncommitted row (and, with editing, every committed row) draws a
//     candidate; with temperature 0 the candidate is the argmax and nothing is drawn;
//   DDIM predictor: every row draws from its posterior; corrector: the corrector_k rows with the
//     lowest p(current token) (lower position first on ties); final step: finalise.
__global__ __launch_bounds__(1024) void k_sched_prepare(EbArgs a) {
  __shared__ uint64_t keys[1024];
  __shared__ double dsum[1024];
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool live = i < a.C;
  const size_t at = static_cast<size_t>(b) * a.C + i;
  const int rb = map_b(a, b);
  const size_t ra = static_cast<size_t>(rb) * a.C + i;
  if (a.st.done[rb]) {  // a frozen canvas never changes
    if (live) {
      a.out.commit_now[ra] = 0;
      a.need_cand[at] = 0;
    }
    return;
  }
  const float h = live ? a.out.entropy[ra] : 0.f;
  const int am = live ? a.out.argmax[ra] : 0;
  const bool committed = live ? (a.st.committed[ra] != 0) : true;
  const int prev = live ? a.st.prev_argmax[ra] : 0;
  const int bad = __syncthreads_or(live && !(fabsf(h) <= FLT_MAX));
  if (bad) {  // non-finite logits: sticky status, the canvas is frozen unchanged
    if (live) {
      a.out.commit_now[ra] = 0;
      a.need_cand[at] = 0;
    }
    if (i == 0) {
      if (a.st.dev_status) atomicExch(a.st.dev_status, static_cast<int>(DG_ERR_NONFINITE));
      a.st.done[rb] = 1;
    }
    return;
  }
  const int all_same = __syncthreads_and(!live || am == prev);
  const int stable = (a.step >= 1 && all_same) ? a.st.stable_count[rb] + 1 : 0;
  if (live) a.st.prev_argmax[ra] = am;
  dsum[i] = live ? static_cast<double>(h) : 0.0;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (i < o) dsum[i] += dsum[i + o];
    __syncthreads();
  }
  const double mean_h = dsum[0] / a.C;
  const int any_unc = __syncthreads_or(live && !committed);
  const bool stop = a.stop_entropy >= 0.0 && stable >= a.stability && mean_h < a.stop_entropy;
  if (i == 0) a.st.stable_count[rb] = stable;
  const bool ddim = a.kind == SCHED_DDIM;
  if (stop || (ddim && a.phase == DDIM_FINAL) || (!ddim && !any_unc && !a.editing)) {
    if (live) {  // finalise: every uncommitted position takes its argmax
      a.need_cand[at] = 0;
      a.out.commit_now[ra] = committed ? 0 : 1;
      if (!committed) {
        a.st.canvas[ra] = am;
        a.st.committed[ra] = 1;
      }
    }
    if (i == 0) a.st.done[rb] = 1;
    return;
  }
  if (!ddim) {  // block refinement
    if (live) {
      a.need_cand[at] = (!a.greedy && (!committed || a.editing)) ? 1 : 0;
      if (a.greedy) a.cand[at] = am;
    }
    return;
  }
  if (live) a.out.commit_now[ra] = 0;
  if (a.phase == DDIM_PREDICT) {
    if (live) a.need_cand[at] = 1;
    return;
  }
  // corrector sweep: ascending (p(current token), position); probabilities are >= 0, so their
  // binary32 patterns order like their values
  float conf = 0.f;
  if (live) {
    const int x = a.st.canvas[ra];
    const SoftStats st = a.row[at];
    if (a.greedy) {
      conf = (x == st.idx) ? 1.f : 0.f;
    } else {
      const float zx = bf2f(a.logits[ra * static_cast<size_t>(a.V) + min(max(x, 0), a.V - 1)]);
      conf = row_prob(zx, a.inv_t_log2e, st);
    }
  }
  keys[i] = live ? ((static_cast<uint64_t>(__float_as_uint(conf)) << 32) | static_cast<uint32_t>(i))
                 : ~0ull;
  sort1024(keys);
  if (live) a.need_cand[at] = 0;
  __syncthreads();
  if (i < a.corrector_k && i < a.C) a.need_cand[static_cast<size_t>(b) * a.C +
                                                static_cast<uint32_t>(keys[i])] = 1;
}

// DDIM draw for one vocabulary chunk of one row (predictor posterior or corrector conditional).
// Both are affine in the model's probabilities: w_v = A + B p_v for v != j and A_j + B_j p_j at
// the current token j (coefficients below, fp64).  The draw is argmax_v (ln w_v + g_v) with the
// entropy-bound sampler's Gumbel noise g_v = -ln(-ln u_v); it is taken as argmax_v w_v / E_v with
// E_v = -ln u_v, the same order (exp of the score), one logarithm per entry.
__global__ __launch_bounds__(kCandThreads) void k_ddim_candidates(EbArgs a) {
  const int row = blockIdx.x;
  if (!a.need_cand[row]) return;
  const int chunk = blockIdx.y;
  const int b = row / a.C, pos = row % a.C;
  const uint32_t cid = a.st.canvas_id[map_b(a, b)];
  const uint32_t k0 = static_cast<uint32_t>(a.seed), k1 = static_cast<uint32_t>(a.seed >> 32);
  const uint16_t* z = a.logits + map_row(a, row) * a.V;
  const SoftStats st = a.row[row];
  const float c = a.inv_t_log2e;
  const int j = min(max(a.st.canvas[map_row(a, row)], 0), a.V - 1);
  const double pj = a.greedy ? (j == st.idx ? 1.0 : 0.0)
                             : static_cast<double>(row_prob(bf2f(z[j]), c, st));
  const double V = static_cast<double>(a.V);
  const double al = a.alpha_t;
  const double d_same = al + (1.0 - al) / V, d_diff = (1.0 - al) / V;
  const double s0 = pj / d_same + (1.0 - pj) / d_diff;
  double A, B, Aj, Bj;
  if (a.phase == DDIM_PREDICT) {
    // sum_m p(m) q(x_next = v | x_t = j, x_0 = m): the one-step transition back to j times the
    // forward transition to the next level applied to r(m) = p(m) / q(j | m)
    const double bn = a.alpha_next, as = a.a_step;
    const double step_same = as + (1.0 - as) / V, step_diff = (1.0 - as) / V;
    A = step_diff * (1.0 - bn) * s0 / V;
    B = step_diff * bn / d_diff;
    Aj = step_same * (1.0 - bn) * s0 / V;
    Bj = step_same * bn / d_same;
  } else {
    // alpha p_loo(v) + (1 - alpha) / V with p_loo(v) = p(v) / (q(j | v) s0)
    A = Aj = (1.0 - al) / V;
    B = al / (d_diff * s0);
    Bj = al / (d_same * s0);
  }
  const int v0 = chunk * kCandChunk;
  const int v1 = min(a.V, v0 + kCandChunk);
  double best = -1.0;
  int best_v = 0x7fffffff;
  for (int v = v0 + threadIdx.x * 8; v < v1; v += kCandThreads * 8) {
    const uint4 raw = *reinterpret_cast<const uint4*>(z + v);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    const Philox4 r0 = philox10(static_cast<uint32_t>(v >> 2), pos, a.step, (cid << 1) | 1u, k0, k1);
    const Philox4 r1 = philox10(static_cast<uint32_t>((v >> 2) + 1), pos, a.step, (cid << 1) | 1u,
                                k0, k1);
    const uint32_t x[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int vk = v + k;
      const float zf = __uint_as_float(k & 1 ? (w[k >> 1] & 0xffff0000u) : (w[k >> 1] << 16));
      const double p = a.greedy ? (vk == st.idx ? 1.0 : 0.0)
                                : static_cast<double>(row_prob(zf, c, st));
      const double wv = (vk == j) ? Aj + Bj * p : A + B * p;
      const double u = (static_cast<double>(x[k]) + 0.5) * 0x1p-32;
      const double sc = wv / (-log(u));
      if (sc > best) {
        best = sc;
        best_v = vk;
      }
    }
  }
  __shared__ double rs[kCandThreads / 64];
  __shared__ int ri[kCandThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double ob = __shfl_xor(best, o, 64);
    const int ov = __shfl_xor(best_v, o, 64);
    if (ob > best || (ob == best && ov < best_v)) {
      best = ob;
      best_v = ov;
    }
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) {
    rs[wv] = best;
    ri[wv] = best_v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kCandThreads / 64; ++k) {
      if (rs[k] > best || (rs[k] == best && ri[k] < best_v)) {
        best = rs[k];
        best_v = ri[k];
      }
    }
    // the score kept by the merge is ln(w / E), the Gumbel score itself
    a.cand_score[static_cast<size_t>(row) * a.n_cand_chunks + chunk] = log(best);
    a.cand_idx[static_cast<size_t>(row) * a.n_cand_chunks + chunk] = best_v;
  }
}

// Block refinement commit, one workgroup of 1024 threads per canvas (canvases finalised or
// frozen by k_sched_prepare are done and skipped): confidence = p(candidate); the uncommitted
// positions in descending (confidence, then ascending position) order; the step commits every
// one above the threshold plus `quota` more (every remaining one at the last step); with editing,
// committed positions take a different candidate whose confidence is above edit_threshold; the
// other uncommitted positions are renoised.
__global__ __launch_bounds__(1024) void k_br_commit(EbArgs a) {
  __shared__ uint64_t keys[1024];
  __shared__ uint8_t sel[1024];
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int rb = map_b(a, b);
  if (a.st.done[rb]) return;
  const bool live = i < a.C;
  const size_t at = static_cast<size_t>(b) * a.C + i;
  const size_t ra = static_cast<size_t>(rb) * a.C + i;
  const bool committed = live ? (a.st.committed[ra] != 0) : true;
  const bool needs = live && (!committed || a.editing);
  int cand = 0;
  float conf = 0.f;
  if (needs) {
    cand = min(max(a.cand[at], 0), a.V - 1);
    const float zc = bf2f(a.logits[ra * static_cast<size_t>(a.V) + cand]);
    conf = row_prob(zc, a.inv_t_log2e, a.row[at]);
  }
  const bool unc = live && !committed;
  keys[i] = unc ? ((static_cast<uint64_t>(~__float_as_uint(conf)) << 32) | static_cast<uint32_t>(i))
                : ~0ull;
  sel[i] = 0;
  const bool above = unc && static_cast<double>(conf) > a.threshold;
  const int n_above = __syncthreads_count(above);
  const int n_unc = __syncthreads_count(unc);
  sort1024(keys);
  const bool last = a.step == a.max_steps - 1;
  const int n = last ? n_unc : min(n_unc, n_above + a.quota);
  if (i < n) sel[static_cast<uint32_t>(keys[i])] = 1;
  __syncthreads();
  if (live) {
    if (unc) {
      if (sel[i]) {
        a.st.canvas[ra] = cand;
        a.st.committed[ra] = 1;
        a.out.commit_now[ra] = 1;
      } else {  // full renoise: a fresh uniform token
        a.out.commit_now[ra] = 0;
        a.st.canvas[ra] = uniform_token(a.seed, a.st.canvas_id[rb], static_cast<uint32_t>(a.step),
                                        static_cast<uint32_t>(i), static_cast<uint32_t>(a.V));
      }
    } else {
      a.out.commit_now[ra] = 0;
      if (a.editing && cand != a.st.canvas[ra] && static_cast<double>(conf) > a.edit_threshold)
        a.st.canvas[ra] = cand;
    }
  }
  const int all_committed = __syncthreads_and(!live || committed || sel[i]);
  if (i == 0 && (last || (all_committed && !a.editing))) a.st.done[rb] = 1;
}

__global__ __launch_bounds__(256) void k_canvas_init(uint64_t seed, dg_eb_state st, int B, int C,
                                                     int V) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= B * C) return;
  const int b = t / C, i = t % C;
  st.canvas[t] = uniform_token(seed, st.canvas_id[b], kInitStepTag, static_cast<uint32_t>(i),
                               static_cast<uint32_t>(V));
  st.committed[t] = 0;
  st.prev_argmax[t] = 0;
  if (i == 0) {
    st.stable_count[b] = 0;
    st.done[b] = 0;
  }
  if (t == 0 && st.dev_status) *st.dev_status = 0;
}

}  // namespace

int logit_stats_chunks(int V) { return (V + kStatsChunk - 1) / kStatsChunk; }
int cand_chunks(int V) { return (V + kCandChunk - 1) / kCandChunk; }

hipError_t launch_logit_stats(const EbArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.C, logit_stats_chunks(a.V));
  hipLaunchKernelGGL(k_logit_stats, grid, dim3(kStatsThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stats_merge(const EbArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_stats_merge, dim3((a.B * a.C + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_eb_commit(const EbArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_eb_commit, dim3(a.B), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_candidates(const EbArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.C, a.n_cand_chunks);
  hipLaunchKernelGGL(k_candidates, grid, dim3(kCandThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cand_apply(const EbArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_cand_apply, dim3((a.B * a.C + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sched_prepare(const EbArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_sched_prepare, dim3(a.B), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ddim_candidates(const EbArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.C, a.n_cand_chunks);
  hipLaunchKernelGGL(k_ddim_candidates, grid, dim3(kCandThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_br_commit(const EbArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_br_commit, dim3(a.B), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_canvas_init(uint64_t seed, dg_eb_state st, int B, int C, int V, hipStream_t s) {
  hipLaunchKernelGGL(k_canvas_init, dim3((B * C + 255) / 256), dim3(256), 0, s, seed, st, B, C, V);
  return hipGetLastError();
}

}  // namespace dg
