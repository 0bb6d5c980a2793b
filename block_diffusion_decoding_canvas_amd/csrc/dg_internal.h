// Internal declarations shared by the HIP translation units of libdg.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "dg.h"

namespace dg {

// ---------------------------------------------------------------------------------------------
// device helpers

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// native 16-byte vector (register-friendly; HIP's uint4 struct can force private-memory copies)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round to nearest even; NaN stays NaN
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return static_cast<uint32_t>(f2bf(a)) | (static_cast<uint32_t>(f2bf(b)) << 16);
}

// hardware round-to-nearest-even pair conversion (v_cvt_pk_bf16_f32); a in the low half
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// one 16x16x128 OCP-e4m3 MFMA (format 0 for both operands, no block scales): a lane's 32 bytes
// of A are a0 then a1, of B b0 then b1.  A and B must list the same k in the same order; which
// 32 k a lane group holds is otherwise free.  Measured here at twice the rate of the 16x16x32
// e4m3 form, which runs at the bf16 rate.
__device__ __forceinline__ f32x4 mfma_f8_128(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x4 c) {
  const i32x8 a = {static_cast<int>(a0.x), static_cast<int>(a0.y), static_cast<int>(a0.z),
                   static_cast<int>(a0.w), static_cast<int>(a1.x), static_cast<int>(a1.y),
                   static_cast<int>(a1.z), static_cast<int>(a1.w)};
  const i32x8 b = {static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z),
                   static_cast<int>(b0.w), static_cast<int>(b1.x), static_cast<int>(b1.y),
                   static_cast<int>(b1.z), static_cast<int>(b1.w)};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// binary32 -> OCP e4m3 code: nearest, ties to even; magnitudes >= 448 saturate to 448 (0x7E);
// NaN -> 0x7F.  Normals keep 3 mantissa bits (bias 7); below 2^-6 the quantum is 2^-9.
__device__ __forceinline__ uint32_t f2e4m3(float f) {
  const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
  const float a = fabsf(f);
  if (!(a == a)) return sign | 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  const uint32_t ua = __float_as_uint(a);
  const uint32_t r = (ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20;  // exponent and 3 mantissa bits
  return sign | (r - (120u << 3));                                  // rebias 127 -> 7
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// XCD-aware slot remap: hardware hands consecutive workgroup ids to the 8 XCDs round-robin;
// this maps them so that consecutive *logical* ids land on the same XCD (and share its L2).
__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  const int per = grid >> 3;  // grid is a multiple of 8
  return (bid & 7) * per + (bid >> 3);
}

// Running softmax statistics of a set of scaled logits y (in log2 units), merged exactly:
//   m = max y, idx = lowest index holding m, R = sum over the other entries of 2^(y - m),
//   A = sum over all entries of (y - m) 2^(y - m).
// Entropy in nats of softmax over the set: ln(1 + R) - ln2 * A / (1 + R).
struct SoftStats {
  float m;
  int idx;
  float r;
  float a;
};

__device__ __forceinline__ SoftStats stats_merge(SoftStats x, SoftStats y) {
  const bool y_wins = (y.m > x.m) || (y.m == x.m && y.idx < x.idx);
  SoftStats w = y_wins ? y : x;
  SoftStats l = y_wins ? x : y;
  if (l.m == -INFINITY) return w;
  const float d = l.m - w.m;  // <= 0
  const float s = __builtin_amdgcn_exp2f(d);
  w.r = w.r + (1.0f + l.r) * s;
  w.a = w.a + (l.a + d * (1.0f + l.r)) * s;
  return w;
}

__device__ __forceinline__ SoftStats stats_shfl_xor(SoftStats s, int o) {
  SoftStats t;
  t.m = __shfl_xor(s.m, o, 64);
  t.idx = __shfl_xor(s.idx, o, 64);
  t.r = __shfl_xor(s.r, o, 64);
  t.a = __shfl_xor(s.a, o, 64);
  return t;
}

// ---------------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): multipliers 0xD2511F53 / 0xCD9E8D57, Weyl key
// increments 0x9E3779B9 / 0xBB67AE85, ten rounds, key advanced between rounds.
struct Philox4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ Philox4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                            uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0;
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{c0, c1, c2, c3};
}

// Sampler counter layout: (w0, position, step tag, (canvas_id << 1) | stream).
constexpr uint32_t kInitStepTag = 0xFFFFFFFFu;

__device__ __forceinline__ int32_t uniform_token(uint64_t seed, uint32_t canvas_id,
                                                 uint32_t step_tag, uint32_t pos,
                                                 uint32_t vocab) {
  const Philox4 r = philox10(0u, pos, step_tag, (canvas_id << 1) | 0u,
                             static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  return static_cast<int32_t>((static_cast<uint64_t>(r.x) * vocab) >> 32);
}

// ---------------------------------------------------------------------------------------------
// host-side launch interface (implemented in the .hip files)

struct WGemmArgs {
  const uint16_t* X;      // token rows (bf16)
  int ldx;
  const int32_t* x_rows;  // gather: X row of tile row r (NULL = r)
  const uint16_t* W;      // weights [experts][N][K] (bf16)
  long long w_estride;    // elements between experts
  const uint16_t* W_sh;   // shared expert weights (expert id == n_experts)
  int K;
  int K_sh;               // shared expert's K
  int N;                  // output features (paired: F, the gate/up split)
  int N_sh;               // shared expert's N
  int n_experts;
  int ksplit;             // dense fp32 epilogue: k splits (partials summed by the consumer)
  int k_per_split;        // set by the launcher
  long long split_stride; // elements between split partial planes
  const int32_t* chunks;  // grouped tiles: [slot] = (expert, row0, nrows); NULL = dense
  const int32_t* n_chunks;
  int ntok;               // dense: rows
  int n_nblk;             // N blocks per tile
  int grid_tiles;         // tile slots
  void* out;
  int ldo;
  // LM-head statistics epilogue
  float inv_t_log2e;      // log2(e) / T as fp32
  SoftStats* part;        // [rows][n_nblk]
  // e4m3 operands: X holds e4m3 codes with one scale per X row, W packed e4m3 codes with one
  // scale per weight row; output = accumulator * x_scale * w_scale
  const float* x_scale;   // indexed like the X rows (through x_rows when gathered)
  const float* w_scale;   // [experts][weight rows]
  long long wsc_estride;  // scales between experts
  const float* w_scale_sh;
  // 1 KiB of readable device memory (workspace) that the weight ring's past-the-end loads read
  // instead of weights; its contents are never used
  const uint8_t* hot;
  // grouped products: the shared expert's tiles (the last sh_tiles of the tile list; 0 = none)
  // are ordered token tile fastest, so its weights are read into one L2 per row block
  int sh_tiles;
  // LM head of a compacted step: token row r is written to output row
  // omap[r / omap_C] * omap_C + r % omap_C (omap_C = 0: row r)
  int omap_C;
  int omap[64];
};

enum Epi { EPI_BF16 = 0, EPI_F32 = 2, EPI_SWIGLU = 3, EPI_LMHEAD = 4 };

// launchers; each returns the hip error of the launch
// router projection: fp32 k-split partial planes [ksplit][ntok][N], any N
hipError_t launch_gemm_dense_f32(const WGemmArgs& a, hipStream_t s);
hipError_t launch_lmhead_packed(const WGemmArgs& a, hipStream_t s);       // logits + stats
int gemm_lmhead_rows_per_block();
// expert products over fragment-major ("packed") weights, in tiles of tile_rows gathered rows:
// moe_tile_rows(ntok) (32, or 128 once a call routes ntok >= 1,024 tokens, about 64 rows per
// expert and more), moe_tile_rows_min() for sizing
hipError_t launch_moe_gateup(const WGemmArgs& a, int tile_rows, hipStream_t s);  // SwiGLU act
hipError_t launch_moe_down(const WGemmArgs& a, int tile_rows, hipStream_t s);    // Y rows bf16
int moe_tile_rows(int ntok);
int moe_tile_rows_min();
// dense products over packed weights, 64-token tiles (bf16 out, or fp32 k-split partials)
hipError_t launch_dense_packed_bf16(const WGemmArgs& a, hipStream_t s);
hipError_t launch_dense_packed_f32(const WGemmArgs& a, hipStream_t s);
hipError_t launch_pack(const void* src, void* dst, long long rows, long long cols, hipStream_t s);
// e4m3 variants (X and W e4m3 codes, per-row scales); gate/up writes the fp32 SwiGLU output
hipError_t launch_moe_gateup_fp8(const WGemmArgs& a, int tile_rows, hipStream_t s);  // fp32 act
hipError_t launch_moe_down_fp8(const WGemmArgs& a, int tile_rows, hipStream_t s);    // Y rows bf16
hipError_t launch_lmhead_packed_fp8(const WGemmArgs& a, hipStream_t s);   // logits + stats
hipError_t launch_pack_fp8(const void* src, void* dst, long long rows, long long cols,
                           hipStream_t s);
// per-row e4m3 quantisation: rows [0, rows_a) have cols_a columns, rows [rows_a, rows) cols_b
hipError_t launch_quant_rows(const void* src, bool src_f32, long long ld_src, uint8_t* codes,
                             long long ld_codes, float* scales, long long rows, long long rows_a,
                             int cols_a, int cols_b, hipStream_t s);

struct AttnArgs {
  const uint16_t* qkv;    // [B*C][(Hq+2Hkv)*dh]
  const uint16_t* kc;     // this layer's cache K [B][Hkv][cap][dh]
  const uint16_t* vc;
  int cap;
  int B, C, Hq, Hkv, dh;
  int len[64];            // visible cache length per canvas (host copy)
  int kvb[64];            // cache batch index of each canvas of the call
  int window;             // 0 = global
  int causal;             // encoder: canvas key j visible to query i iff j <= i
  float scale_log2e;      // log2(e) / sqrt(dh)
  int n_split;
  uint16_t* o_part;       // [n_split][B][Hkv][R][dh] bf16 (R = Hq/Hkv * C)
  float* ml_part;         // [n_split][B][Hkv][R][2]
  uint16_t* out;          // [B*C][Hq*dh]
  // fp8 KV cache: kc / vc hold e4m3 codes (bytes, same layout) with one fp32 scale per row in
  // ksc / vsc [B][Hkv][cap]; the call's canvas keys and values are read as e4m3 rows too, from
  // kq / vq [B*C][Hkv][dh] with scales kqs / vqs [B*C][Hkv]
  int f8;
  const float* ksc;
  const float* vsc;
  const uint8_t* kq;
  const uint8_t* vq;
  const float* kqs;
  const float* vqs;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// e4m3 rows of the call's canvas keys and values (one scale per token and KV head) from the
// bf16 QKV product into kq / vq (+ scales); with kc != NULL they are also written into the cache
// at [len[b] + i] (kc/vc codes, ksc/vsc scales of this layer)
hipError_t launch_kv_quant(const AttnArgs& a, uint8_t* kq, uint8_t* vq, float* kqs, float* vqs,
                           uint8_t* kc, uint8_t* vc, float* ksc, float* vsc, hipStream_t s);
int attention_pick_split(int B, int C, int Hq, int Hkv, int max_keys);

// per-token kernels
// h[t] = E[token t]; with n_map > 0 (compacted step) the token of row t is
// tokens[map[t / C] * C + t % C]
hipError_t launch_embed(const int32_t* tokens, const uint16_t* embed, float* h, int ntok, int d,
                        int vocab, hipStream_t s, int C = 0, int n_map = 0,
                        const int* map = nullptr);
// norms: u = bf16(RMSNorm(h) * gain); with q8 != NULL also the e4m3 codes of the fp32 normed
// row and its scale (q8s)
hipError_t launch_rmsnorm(const float* h, const uint16_t* gain, uint16_t* u, int ntok, int d,
                          float eps, uint8_t* q8, float* q8s, hipStream_t s);
hipError_t launch_topk(const float* logits, int ksplit, int ntok, int n_exp, int top_k,
                       int32_t* idx, float* gates, float* logits_out, hipStream_t s);
hipError_t launch_resid_norm(float* h, const float* part, int ksplit, int ntok, int d,
                             const uint16_t* gain, uint16_t* u, float eps, uint8_t* q8,
                             float* q8s, hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int ntok, int top_k, int n_exp, int tile_rows,
                          int32_t* perm, int32_t* inv, int32_t* chunks, int32_t* n_chunks,
                          int max_chunks, hipStream_t s);
hipError_t launch_combine(float* h, const uint16_t* Y, const int32_t* inv, const float* gates,
                          int ntok, int top_k, int d, const uint16_t* next_gain,
                          uint16_t* u_next, float eps, uint8_t* q8, float* q8s, hipStream_t s);
hipError_t launch_kv_write(const uint16_t* qkv, uint16_t* kc, uint16_t* vc, int B, int C,
                           int Hq, int Hkv, int dh, int cap, const int* len, hipStream_t s);
hipError_t launch_copy(void* dst, const void* src, size_t n, hipStream_t s);
hipError_t launch_read_stream(const void* src, size_t n, uint32_t* out, hipStream_t s);
hipError_t launch_mfma_loop(int iters, float* out, hipStream_t s);
int mfma_loop_blocks();

// sampler kernels
enum SchedKind { SCHED_EB = 0, SCHED_BLOCK_REFINEMENT = 1, SCHED_DDIM = 2 };
enum DdimPhase { DDIM_PREDICT = 0, DDIM_CORRECT = 1, DDIM_FINAL = 2 };

struct EbArgs {
  int B, C, V, step, max_steps;
  float inv_t;            // fp32 multiplier of the logits: 1 / T_s (EB), 1 / T or 1 (greedy)
  float inv_t_log2e;      // fp32(inv_t * log2 e)
  double bound;
  double stop_entropy;
  int stability;
  uint64_t seed;
  dg_eb_state st;
  dg_step_out out;
  const uint16_t* logits;
  SoftStats* part;        // [B*C][n_part]
  int n_part;
  uint8_t* need_cand;     // [B*C] rows that take a Gumbel candidate this step
  double* cand_score;     // [B*C][n_cand_chunks]
  int32_t* cand_idx;
  int n_cand_chunks;
  // the other schedulers
  int kind;               // SchedKind
  SoftStats* row;         // [B*C] merged statistics of each row (m, argmax, R, A)
  int32_t* cand;          // [B*C] block refinement: each row's candidate token
  int greedy;             // temperature 0: the candidate is the argmax
  double threshold;       // block refinement: commit above this confidence
  double edit_threshold;  // block refinement: re-edit above this confidence (editing != 0)
  int editing;
  int quota;              // block refinement: this step's even share of the canvas
  int phase;              // DDIM: DdimPhase of this call step
  double a_step;          // DDIM predictor: alpha(t) / alpha(t_next)
  double alpha_t;         // DDIM: alpha at the current level
  double alpha_next;      // DDIM predictor: alpha at the next level
  int corrector_k;        // DDIM corrector: positions resampled per sweep
  // compacted step: compact canvas b is canvas bmap[b] of the state, outputs and logits
  int mapped;
  int bmap[64];
};
hipError_t launch_logit_stats(const EbArgs& a, hipStream_t s);   // partials from logits
int logit_stats_chunks(int V);
hipError_t launch_stats_merge(const EbArgs& a, hipStream_t s);   // partials -> H, argmax
hipError_t launch_eb_commit(const EbArgs& a, hipStream_t s);     // stop / select / renoise
hipError_t launch_candidates(const EbArgs& a, hipStream_t s);    // Gumbel-max partials
hipError_t launch_cand_apply(const EbArgs& a, hipStream_t s);    // write candidates
int cand_chunks(int V);
hipError_t launch_canvas_init(uint64_t seed, dg_eb_state st, int B, int C, int V, hipStream_t s);
// block refinement and DDIM: stop / finalise and the rows needing a draw; the DDIM draw; the
// block-refinement commit (threshold + quota, editing, renoise)
hipError_t launch_sched_prepare(const EbArgs& a, hipStream_t s);
hipError_t launch_ddim_candidates(const EbArgs& a, hipStream_t s);
hipError_t launch_br_commit(const EbArgs& a, hipStream_t s);

}  // namespace dg
