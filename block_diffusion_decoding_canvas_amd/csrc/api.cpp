// C ABI of libdg.so: host-side validation, workspace layout and kernel sequencing.
// The HIP kernels live in the k_*.hip files; every step of the path runs in them.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "dg_internal.h"

struct dg_model {
  dg_dims dims;
  std::vector<dg_layer_w> layers;
  const uint16_t* embed;
  const uint16_t* final_norm;
  const void* w_lm;        // packed bf16, or packed e4m3 codes (fp8 configuration)
  const float* s_lm;       // fp8: per-row scales of w_lm
  bool fp8() const { return dims.wdtype == DG_FP8_E4M3; }
};

namespace {

thread_local char g_err[512] = "";

dg_status fail(dg_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

#define DG_HIP(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(DG_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_));         \
  } while (0)

// ---------------------------------------------------------------------------------------------
// kernel timing (HIP events around launches of the enabled classes, on the launch stream)

enum ProfClass {
  PC_EMBED, PC_RMSNORM, PC_GEMM_QKV, PC_ATTENTION, PC_GEMM_O, PC_GEMM_ROUTER, PC_TOPK,
  PC_PERMUTE, PC_MOE_GATEUP, PC_MOE_DOWN, PC_COMBINE, PC_LMHEAD, PC_STATS, PC_STATS_MERGE,
  PC_EB_COMMIT, PC_CANDIDATES, PC_CAND_APPLY, PC_KV_WRITE, PC_COPY, PC_QUANT, PC_COUNT
};
const char* kProfNames[PC_COUNT] = {
    "embed", "rmsnorm", "gemm_qkv", "attention", "gemm_o", "gemm_router", "topk",
    "permute", "moe_gateup", "moe_down", "combine", "lmhead", "logit_stats", "stats_merge",
    "eb_commit", "candidates", "cand_apply", "kv_write", "copy", "quant"};

struct Prof {
  std::mutex mu;
  uint32_t mask = 0;
  struct Pair {
    hipEvent_t a, b;
    int cls;
  };
  std::vector<Pair> pending;
  std::vector<hipEvent_t> free_events;
  double total_ms[PC_COUNT] = {};
  int64_t count[PC_COUNT] = {};
} g_prof;

hipEvent_t prof_event() {
  if (!g_prof.free_events.empty()) {
    hipEvent_t e = g_prof.free_events.back();
    g_prof.free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

dg_status prof_harvest() {
  for (auto& p : g_prof.pending) {
    DG_HIP(hipEventSynchronize(p.b));
    float ms = 0.f;
    DG_HIP(hipEventElapsedTime(&ms, p.a, p.b));
    g_prof.total_ms[p.cls] += ms;
    g_prof.count[p.cls] += 1;
    g_prof.free_events.push_back(p.a);
    g_prof.free_events.push_back(p.b);
  }
  g_prof.pending.clear();
  return DG_OK;
}

// Wraps one launch; records events around it when profiling is on.
template <class F>
dg_status launch(int cls, hipStream_t s, F&& f) {
  hipEvent_t ea = nullptr, eb = nullptr;
  if (g_prof.mask & (1u << cls)) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.pending.size() > 20000) {
      dg_status st = prof_harvest();
      if (st != DG_OK) return st;
    }
    ea = prof_event();
    eb = prof_event();
    if (ea) DG_HIP(hipEventRecord(ea, s));
  }
  hipError_t e = f();
  if (e != hipSuccess)
    return fail(DG_ERR_HIP, "%s launch failed: %s", kProfNames[cls], hipGetErrorString(e));
  if (ea && eb) {
    DG_HIP(hipEventRecord(eb, s));
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.pending.push_back({ea, eb, cls});
  }
  return DG_OK;
}

#define DG_LAUNCH(cls, stream, expr)                                   \
  do {                                                                 \
    dg_status st_ = launch(cls, stream, [&]() { return (expr); });     \
    if (st_ != DG_OK) return st_;                                      \
  } while (0)

// ---------------------------------------------------------------------------------------------
// workspace carving

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <class T>
  T* take(size_t n) {
    off = (off + 255) & ~static_cast<size_t>(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

struct EbWs {
  dg::SoftStats* part;
  int n_part;
  uint8_t* need;
  double* cand_score;
  int32_t* cand_idx;
  int n_cand;
  dg::SoftStats* row;   // merged statistics per row
  int32_t* cand;        // block refinement candidates per row
};

// The sampler's scratch, carved the same way for the standalone sampler and the decoder step.
EbWs carve_eb(Carver& c, int rows, int n_part, int vocab) {
  EbWs w;
  w.n_part = n_part;
  w.part = c.take<dg::SoftStats>(static_cast<size_t>(rows) * n_part);
  w.need = c.take<uint8_t>(rows);
  w.n_cand = dg::cand_chunks(vocab);
  w.cand_score = c.take<double>(static_cast<size_t>(rows) * w.n_cand);
  w.cand_idx = c.take<int32_t>(static_cast<size_t>(rows) * w.n_cand);
  w.row = c.take<dg::SoftStats>(rows);
  w.cand = c.take<int32_t>(rows);
  return w;
}

// the entropy-bound constants as scheduler parameters
dg_sched_params sched_from_eb(const dg_eb_params* p) {
  dg_sched_params q;
  memset(&q, 0, sizeof(q));
  q.kind = DG_SCHED_ENTROPY_BOUND;
  q.max_steps = p->max_steps;
  q.t_max = p->t_max;
  q.t_min = p->t_min;
  q.entropy_bound = p->entropy_bound;
  q.stop_entropy = p->stop_entropy;
  q.stability = p->stability;
  q.seed = p->seed;
  q.editing_threshold = -1.0;
  return q;
}

dg_status check_sched(const dg_sched_params* p, int32_t step) {
  if (!p) return fail(DG_ERR_NULL, "params is NULL");
  if (p->max_steps < 1) return fail(DG_ERR_STATE, "max_steps must be >= 1");
  if (step < 0 || step >= p->max_steps)
    return fail(DG_ERR_STATE, "step %d outside [0, %d)", step, p->max_steps);
  if (p->stability < 0) return fail(DG_ERR_STATE, "stability must be >= 0");
  switch (p->kind) {
    case DG_SCHED_ENTROPY_BOUND:
      if (!(p->t_max > 0.0) || !(p->t_min > 0.0))
        return fail(DG_ERR_STATE, "temperatures must be > 0");
      if (!(p->entropy_bound >= 0.0)) return fail(DG_ERR_STATE, "entropy_bound must be >= 0");
      return DG_OK;
    case DG_SCHED_BLOCK_REFINEMENT:
      if (!(p->temperature >= 0.0) || !(p->temperature < 1e30))
        return fail(DG_ERR_STATE, "temperature must be finite and >= 0");
      if (!(p->threshold == p->threshold)) return fail(DG_ERR_STATE, "threshold is NaN");
      if (!(p->editing_threshold == p->editing_threshold))
        return fail(DG_ERR_STATE, "editing_threshold is NaN");
      if (p->top_k != 0)
        return fail(DG_ERR_UNSUPPORTED, "top_k = %d: the vocabulary top-k filter is not built",
                    p->top_k);
      return DG_OK;
    case DG_SCHED_DISCRETE_DDIM:
      if (!(p->temperature >= 0.0) || !(p->temperature < 1e30))
        return fail(DG_ERR_STATE, "temperature must be finite and >= 0");
      if (p->corrector_steps < 0 || p->corrector_steps > p->max_steps - 1)
        return fail(DG_ERR_STATE, "corrector_steps = %d outside [0, max_steps - 1]",
                    p->corrector_steps);
      if (p->corrector_k < 0) return fail(DG_ERR_STATE, "corrector_k must be >= 0");
      return DG_OK;
    default:
      return fail(DG_ERR_STATE, "unknown scheduler kind %d", p->kind);
  }
}

dg_status check_params(const dg_eb_params* p, int32_t step) {
  if (!p) return fail(DG_ERR_NULL, "params is NULL");
  const dg_sched_params q = sched_from_eb(p);
  return check_sched(&q, step);
}

dg_status check_state(const dg_eb_state* s) {
  if (!s) return fail(DG_ERR_NULL, "state is NULL");
  if (!s->canvas || !s->committed || !s->prev_argmax || !s->stable_count || !s->done ||
      !s->canvas_id)
    return fail(DG_ERR_NULL, "a sampler state pointer is NULL");
  return DG_OK;
}

dg_status check_out(const dg_step_out* o, bool need_logits) {
  if (!o) return fail(DG_ERR_NULL, "out is NULL");
  if (!o->entropy || !o->argmax || !o->commit_now)
    return fail(DG_ERR_NULL, "an output pointer is NULL");
  if (need_logits && !o->logits) return fail(DG_ERR_NULL, "out->logits is NULL");
  return DG_OK;
}

// The fp32 multiplier of the logits.  Entropy bound: T_s = t_max + (t_min - t_max) s / (S - 1)
// in fp64; the others: the fixed temperature, 1 when greedy.  The kernels use fp32(1 / T).
void temperature(const dg_sched_params* p, int step, float* inv_t, float* inv_t_log2e) {
  double t = 1.0;
  if (p->kind == DG_SCHED_ENTROPY_BOUND) {
    t = p->t_max;
    if (p->max_steps > 1)
      t = p->t_max + (p->t_min - p->t_max) * static_cast<double>(step) /
                         static_cast<double>(p->max_steps - 1);
  } else if (p->temperature > 0.0) {
    t = p->temperature;
  }
  *inv_t = static_cast<float>(1.0 / t);
  *inv_t_log2e = static_cast<float>(static_cast<double>(*inv_t) * 1.4426950408889634);
}

dg::EbArgs eb_args(const dg_sched_params* p, int B, int C, int V, int step,
                   const dg_eb_state* st, const dg_step_out* out, const uint16_t* logits,
                   const EbWs& w) {
  dg::EbArgs a;
  memset(&a, 0, sizeof(a));
  a.B = B;
  a.C = C;
  a.V = V;
  a.step = step;
  a.max_steps = p->max_steps;
  temperature(p, step, &a.inv_t, &a.inv_t_log2e);
  a.bound = p->entropy_bound;
  a.stop_entropy = p->stop_entropy;
  a.stability = p->stability;
  a.seed = p->seed;
  a.st = *st;
  a.out = *out;
  a.logits = logits;
  a.part = w.part;
  a.n_part = w.n_part;
  a.need_cand = w.need;
  a.cand_score = w.cand_score;
  a.cand_idx = w.cand_idx;
  a.n_cand_chunks = w.n_cand;
  a.row = w.row;
  a.cand = w.cand;
  a.kind = p->kind == DG_SCHED_BLOCK_REFINEMENT ? dg::SCHED_BLOCK_REFINEMENT
           : p->kind == DG_SCHED_DISCRETE_DDIM  ? dg::SCHED_DDIM
                                                : dg::SCHED_EB;
  a.greedy = (p->kind != DG_SCHED_ENTROPY_BOUND && !(p->temperature > 0.0)) ? 1 : 0;
  if (p->kind == DG_SCHED_BLOCK_REFINEMENT) {
    a.threshold = p->threshold;
    a.editing = p->editing_threshold >= 0.0 ? 1 : 0;
    a.edit_threshold = p->editing_threshold;
    const long long S = p->max_steps, s = step, c = C;
    a.quota = static_cast<int>((s + 1) * c / S - s * c / S);
  }
  if (p->kind == DG_SCHED_DISCRETE_DDIM) {
    // P predictor steps from t = 1 (pure noise) to t = 0, alpha(t) = 1 - t, then the corrector
    // sweeps at the last noisy level t = 1 / P, then the final deterministic step
    const int S = p->max_steps, P = S - p->corrector_steps;
    a.corrector_k = p->corrector_k;
    if (step == S - 1) {
      a.phase = dg::DDIM_FINAL;
    } else if (step < P - 1) {
      const double t = 1.0 - static_cast<double>(step) / P;
      const double tn = 1.0 - static_cast<double>(step + 1) / P;
      a.phase = dg::DDIM_PREDICT;
      a.alpha_t = 1.0 - t;
      a.alpha_next = 1.0 - tn;
      a.a_step = a.alpha_t / a.alpha_next;
    } else {
      a.phase = dg::DDIM_CORRECT;
      a.alpha_t = 1.0 - 1.0 / P;
    }
  }
  return a;
}

// stats partials are ready: merge, then the scheduler's decisions and draws
dg_status run_sampler_tail(const dg::EbArgs& a, hipStream_t s) {
  DG_LAUNCH(PC_STATS_MERGE, s, dg::launch_stats_merge(a, s));
  switch (a.kind) {
    case dg::SCHED_BLOCK_REFINEMENT:
      DG_LAUNCH(PC_EB_COMMIT, s, dg::launch_sched_prepare(a, s));
      if (!a.greedy) {
        DG_LAUNCH(PC_CANDIDATES, s, dg::launch_candidates(a, s));
        DG_LAUNCH(PC_CAND_APPLY, s, dg::launch_cand_apply(a, s));
      }
      DG_LAUNCH(PC_EB_COMMIT, s, dg::launch_br_commit(a, s));
      return DG_OK;
    case dg::SCHED_DDIM:
      DG_LAUNCH(PC_EB_COMMIT, s, dg::launch_sched_prepare(a, s));
      DG_LAUNCH(PC_CANDIDATES, s, dg::launch_ddim_candidates(a, s));
      DG_LAUNCH(PC_CAND_APPLY, s, dg::launch_cand_apply(a, s));
      return DG_OK;
    default:
      DG_LAUNCH(PC_EB_COMMIT, s, dg::launch_eb_commit(a, s));
      DG_LAUNCH(PC_CANDIDATES, s, dg::launch_candidates(a, s));
      DG_LAUNCH(PC_CAND_APPLY, s, dg::launch_cand_apply(a, s));
      return DG_OK;
  }
}

}  // namespace

// ---------------------------------------------------------------------------------------------

extern "C" {

const char* dg_last_error(void) { return g_err; }

dg_status dg_model_create(const dg_dims* d, const dg_layer_w* layers, const void* embed,
                          const void* final_norm, const void* w_lm, const float* s_lm,
                          dg_model** out) {
  if (!d || !layers || !embed || !final_norm || !w_lm || !out)
    return fail(DG_ERR_NULL, "dg_model_create: NULL argument");
  *out = nullptr;
  if (d->wdtype != DG_BF16 && d->wdtype != DG_FP8_E4M3)
    return fail(DG_ERR_DTYPE, "wdtype must be DG_BF16 or DG_FP8_E4M3");
  const bool fp8 = d->wdtype == DG_FP8_E4M3;
  if (fp8 && (d->d_model % 64 || d->ffn_inner % 64 || d->shared_inner % 64))
    return fail(DG_ERR_SHAPE, "fp8 weights need d_model, ffn_inner, shared_inner multiples of 64");
  if (fp8 && !s_lm) return fail(DG_ERR_NULL, "fp8 weights need s_lm");
  if (d->n_layers < 1 || d->d_model < 32 || d->n_q_heads < 1 || d->n_kv_heads < 1 ||
      d->head_dim < 16)
    return fail(DG_ERR_SHAPE, "non-positive or too small dimension");
  if (d->d_model % 32 || d->ffn_inner % 32 || d->shared_inner % 32)
    return fail(DG_ERR_SHAPE, "d_model, ffn_inner and shared_inner must be multiples of 32");
  if (d->d_model > 8192) return fail(DG_ERR_SHAPE, "d_model must be <= 8192");
  if (d->head_dim != 16 && d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128 &&
      d->head_dim != 256)
    return fail(DG_ERR_SHAPE, "head_dim must be one of 16, 32, 64, 128, 256");
  if (d->n_q_heads % d->n_kv_heads) return fail(DG_ERR_SHAPE, "n_q_heads %% n_kv_heads != 0");
  if (((d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim) % 32 || (d->n_q_heads * d->head_dim) % 32)
    return fail(DG_ERR_SHAPE, "(Hq + 2 Hkv) head_dim and Hq head_dim must be multiples of 32");
  if (d->n_experts < 1 || d->n_experts > 256 || d->top_k < 1 || d->top_k > d->n_experts ||
      d->top_k > 16)
    return fail(DG_ERR_SHAPE, "need 1 <= top_k <= min(16, n_experts), n_experts <= 256");
  if (d->vocab < 256 || d->vocab % 256) return fail(DG_ERR_SHAPE, "vocab must be a multiple of 256");
  if (d->canvas_len < 1 || d->canvas_len > 1024)
    return fail(DG_ERR_SHAPE, "canvas_len must be in [1, 1024]");
  if (d->window < 0 || (d->window > 0 && d->window < d->canvas_len))
    return fail(DG_ERR_SHAPE, "window must be 0 or >= canvas_len");
  if (d->window > 0 && d->global_every < 1) return fail(DG_ERR_SHAPE, "global_every must be >= 1");
  if (!(d->norm_eps > 0.f)) return fail(DG_ERR_SHAPE, "norm_eps must be > 0");
  for (int l = 0; l < d->n_layers; ++l) {
    const dg_layer_w& w = layers[l];
    if (!w.attn_norm || !w.w_qkv || !w.w_o || !w.ffn_norm || !w.w_router || !w.w_gate_up ||
        !w.w_down || !w.ws_gate_up || !w.ws_down)
      return fail(DG_ERR_NULL, "layer %d has a NULL weight", l);
    if (fp8 && (!w.s_gate_up || !w.s_down || !w.ss_gate_up || !w.ss_down))
      return fail(DG_ERR_NULL, "layer %d: fp8 weights need their scales", l);
  }
  dg_model* m = new (std::nothrow) dg_model;
  if (!m) return fail(DG_ERR_HIP, "host allocation failed");
  m->dims = *d;
  m->layers.assign(layers, layers + d->n_layers);
  m->embed = static_cast<const uint16_t*>(embed);
  m->final_norm = static_cast<const uint16_t*>(final_norm);
  m->w_lm = w_lm;
  m->s_lm = fp8 ? s_lm : nullptr;
  *out = m;
  return DG_OK;
}

void dg_model_destroy(dg_model* m) { delete m; }

size_t dg_eb_workspace_bytes(int32_t B, int32_t C, int32_t V) {
  if (B < 1 || C < 1 || V < 256) return 0;
  Carver c(nullptr);
  carve_eb(c, B * C, dg::logit_stats_chunks(V), V);
  return c.off + 256;
}

dg_status dg_canvas_init(const dg_eb_params* p, dg_eb_state* st, int32_t B, int32_t C, int32_t V,
                         void* stream) {
  if (!p) return fail(DG_ERR_NULL, "params is NULL");
  dg_status s = check_state(st);
  if (s != DG_OK) return s;
  if (B < 1 || C < 1 || C > 1024 || V < 1) return fail(DG_ERR_SHAPE, "bad B/C/V");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  DG_LAUNCH(PC_EB_COMMIT, hs, dg::launch_canvas_init(p->seed, *st, B, C, V, hs));
  return DG_OK;
}

dg_status dg_sample(const uint16_t* logits, int32_t B, int32_t C, int32_t V, int32_t step,
                    const dg_sched_params* p, dg_eb_state* st, dg_step_out* out, void* ws,
                    size_t ws_bytes, void* stream) {
  if (!logits || !ws) return fail(DG_ERR_NULL, "logits or workspace is NULL");
  dg_status s = check_sched(p, step);
  if (s != DG_OK) return s;
  if ((s = check_state(st)) != DG_OK) return s;
  if ((s = check_out(out, false)) != DG_OK) return s;
  if (B < 1 || C < 1 || C > 1024 || V < 256 || V % 256)
    return fail(DG_ERR_SHAPE, "need B >= 1, 1 <= C <= 1024, V a multiple of 256");
  if (ws_bytes < dg_eb_workspace_bytes(B, C, V))
    return fail(DG_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes,
                dg_eb_workspace_bytes(B, C, V));
  hipStream_t hs = static_cast<hipStream_t>(stream);
  Carver c(ws);
  EbWs w = carve_eb(c, B * C, dg::logit_stats_chunks(V), V);
  dg::EbArgs a = eb_args(p, B, C, V, step, st, out, logits, w);
  DG_LAUNCH(PC_STATS, hs, dg::launch_logit_stats(a, hs));
  return run_sampler_tail(a, hs);
}

dg_status dg_eb_sample(const uint16_t* logits, int32_t B, int32_t C, int32_t V, int32_t step,
                       const dg_eb_params* p, dg_eb_state* st, dg_step_out* out, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!p) return fail(DG_ERR_NULL, "params is NULL");
  const dg_sched_params q = sched_from_eb(p);
  return dg_sample(logits, B, C, V, step, &q, st, out, ws, ws_bytes, stream);
}

}  // extern "C"

// ---- the sampler without a caller workspace ------------------------------------------------
// Its scratch (chunk statistics, candidate flags and candidate partials) lives in this
// file-scope device array, one copy per GPU, held until the process ends.  In host code the
// array's name is only a host-side stand-in: its device address is looked up once per device
// with hipGetSymbolAddress and only that address is passed to kernels.

namespace {

constexpr size_t kNoAllocScratchBytes = 8u << 20;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dg_status scratch_ptr(void** out) {
  int dev = -1;
  DG_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DG_ERR_UNSUPPORTED, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DG_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DG_OK;
}

}  // namespace

extern "C" {

size_t dg_eb_sample_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

dg_status dg_eb_sample_noalloc(const uint16_t* logits, int32_t B, int32_t C, int32_t V,
                               int32_t step, const dg_eb_params* p, dg_eb_state* st,
                               dg_step_out* out, void* stream) {
  if (!logits) return fail(DG_ERR_NULL, "logits is NULL");
  if (B < 1 || C < 1 || C > 1024 || V < 256 || V % 256)
    return fail(DG_ERR_SHAPE, "need B >= 1, 1 <= C <= 1024, V a multiple of 256");
  const size_t need = dg_eb_workspace_bytes(B, C, V);
  if (need > kNoAllocScratchBytes)
    return fail(DG_ERR_WORKSPACE, "B = %d, C = %d, V = %d need %zu bytes of scratch; the "
                "built-in scratch holds %zu", B, C, V, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  dg_status s = scratch_ptr(&ws);
  if (s != DG_OK) return s;
  // every scratch entry a kernel reads is written earlier in the same call: nothing to clear
  return dg_eb_sample(logits, B, C, V, step, p, st, out, ws, kNoAllocScratchBytes, stream);
}

dg_status dg_pack_weight(const void* src, void* dst, int64_t rows, int64_t cols, void* stream) {
  if (!src || !dst) return fail(DG_ERR_NULL, "NULL pointer");
  if (rows < 16 || cols < 32 || rows % 16 || cols % 32)
    return fail(DG_ERR_SHAPE, "rows must be a multiple of 16 and cols a multiple of 32");
  if (src == dst) return fail(DG_ERR_SHAPE, "src and dst must not alias");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  DG_LAUNCH(PC_COPY, hs, dg::launch_pack(src, dst, rows, cols, hs));
  return DG_OK;
}

dg_status dg_copy_bytes(void* dst, const void* src, size_t n, void* stream) {
  if (!dst || !src) return fail(DG_ERR_NULL, "NULL pointer");
  if (n % 16) return fail(DG_ERR_SHAPE, "n must be a multiple of 16");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  DG_LAUNCH(PC_COPY, hs, dg::launch_copy(dst, src, n, hs));
  return DG_OK;
}

dg_status dg_bench_read_stream(const void* src, size_t n, uint32_t* xor_out, void* stream) {
  if (!src || !xor_out) return fail(DG_ERR_NULL, "NULL pointer");
  if (n % 16) return fail(DG_ERR_SHAPE, "n must be a multiple of 16");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  DG_LAUNCH(PC_COPY, hs, dg::launch_read_stream(src, n, xor_out, hs));
  return DG_OK;
}

int32_t dg_bench_mfma_loop_blocks(void) { return dg::mfma_loop_blocks(); }

dg_status dg_bench_mfma_loop(int32_t iters, float* out, void* stream) {
  if (!out) return fail(DG_ERR_NULL, "NULL pointer");
  if (iters < 1) return fail(DG_ERR_SHAPE, "iters must be >= 1");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  DG_LAUNCH(PC_COPY, hs, dg::launch_mfma_loop(iters, out, hs));
  return DG_OK;
}

int32_t dg_prof_num_classes(void) { return PC_COUNT; }

const char* dg_prof_class_name(int32_t cls) {
  return (cls >= 0 && cls < PC_COUNT) ? kProfNames[cls] : "";
}

dg_status dg_prof_enable(uint32_t mask) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.mask = mask;
  return DG_OK;
}

dg_status dg_prof_read(int32_t cls, double* total_ms, int64_t* launches) {
  if (cls < 0 || cls >= PC_COUNT) return fail(DG_ERR_SHAPE, "bad class");
  if (!total_ms || !launches) return fail(DG_ERR_NULL, "NULL output");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  dg_status s = prof_harvest();
  if (s != DG_OK) return s;
  *total_ms = g_prof.total_ms[cls];
  *launches = g_prof.count[cls];
  return DG_OK;
}

dg_status dg_prof_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  dg_status s = prof_harvest();
  if (s != DG_OK) return s;
  for (int i = 0; i < PC_COUNT; ++i) {
    g_prof.total_ms[i] = 0.0;
    g_prof.count[i] = 0;
  }
  return DG_OK;
}

}  // extern "C"

// ---- decoder: workspace layout and kernel sequence ------------------------------------------

namespace {

constexpr int kRouterSplit = 8;   // k-splits of the router projection (summed by topk)
constexpr int kOProjSplit = 4;    // most k-splits of the attention output projection

// k-splits of the output projection for calls of `tokens` rows: enough (up to 4) for units of
// 128 tokens x 128 output rows to cover every compute unit once (calls of >= 1,024 tokens run
// two such units per 8-wave workgroup).  Large calls (a batch of canvases, a long prefill
// chunk) take fewer fp32 partial planes, which both the projection writes and the residual
// kernel reads.  A compacted step passes the whole batch's token count, so its rounding matches
// the full step's.
int o_proj_split(int tokens, int d_model) {
  const int tiles = (tokens + 127) / 128, nblk = (d_model + 127) / 128;
  return std::max(1, std::min(kOProjSplit, (256 + tiles * nblk - 1) / (tiles * nblk)));
}

struct DecWs {
  float* h;           // [T][d] residual stream (fp32)
  uint16_t* u;        // [T][d] normed activations (bf16)
  uint16_t* qkv;      // [T][(Hq + 2 Hkv) dh]
  uint16_t* attn;     // [T][Hq dh]
  uint16_t* o_part;   // attention split partials (bf16)
  float* ml_part;
  int max_split;
  float* proj_part;   // [kOProjSplit][T][d] output-projection partials
  float* router_part; // [kRouterSplit][T][E]
  int32_t* topk;      // [T][k]
  float* gates;       // [T][k]
  int32_t* perm;      // [T k + T]
  int32_t* inv;       // [T k]
  int32_t* chunks;    // [max_chunks][3]
  int32_t* n_chunks;  // [1]
  int max_chunks;
  uint16_t* act;      // [T k + T][max(F, Fs)]
  uint16_t* y;        // [T k + T][d]
  EbWs eb;            // LM-head statistics partials and the sampler's scratch
  // fp8 configuration only (NULL otherwise)
  uint8_t* u8;        // [T][d] e4m3 codes of the FFN / LM-head input
  float* u8s;         // [T] their row scales
  float* act32;       // [T k + T][max(F, Fs)] fp32 SwiGLU output
  uint8_t* act8;      // its e4m3 codes
  float* act8s;       // [T k + T] row scales
  uint8_t* hot;       // 1 KiB read by the streaming kernels' past-the-end loads (never used)
  uint8_t* kq;        // [T][Hkv][dh] e4m3 canvas keys (fp8 KV cache)
  uint8_t* vq;        // values
  float* kqs;         // [T][Hkv] their row scales
  float* vqs;
};

int attn_base_blocks(const dg_dims& d, int B, int C) {
  const int R = (d.n_q_heads / d.n_kv_heads) * C;
  return B * d.n_kv_heads * ((R + 63) / 64);
}

// C: tokens per canvas in the call (the canvas length, or an append's token count)
DecWs carve_dec(Carver& c, const dg_dims& d, int B, int C) {
  DecWs w;
  const size_t T = static_cast<size_t>(B) * C;
  const int dq = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
  const int fmax = std::max(d.ffn_inner, d.shared_inner);
  const size_t rows = T * d.top_k + T;
  w.h = c.take<float>(T * d.d_model);
  w.u = c.take<uint16_t>(T * d.d_model);
  w.qkv = c.take<uint16_t>(T * dq);
  w.attn = c.take<uint16_t>(T * d.n_q_heads * d.head_dim);
  w.max_split = std::max(1, 1024 / attn_base_blocks(d, B, C));
  // split partial rows: max_split * prow <= max(prow, 65,536), because prow <= 64 * base blocks;
  // sized by that bound, the workspace grows monotonically with C
  const size_t prow = static_cast<size_t>(B) * d.n_q_heads * C;
  const size_t part_rows = std::max<size_t>(prow, 65536);
  w.o_part = c.take<uint16_t>(part_rows * d.head_dim);
  w.ml_part = c.take<float>(part_rows * 2);
  w.proj_part = c.take<float>(static_cast<size_t>(kOProjSplit) * T * d.d_model);
  w.router_part = c.take<float>(static_cast<size_t>(kRouterSplit) * T * d.n_experts);
  w.topk = c.take<int32_t>(T * d.top_k);
  w.gates = c.take<float>(T * d.top_k);
  w.perm = c.take<int32_t>(rows);
  w.inv = c.take<int32_t>(T * d.top_k);
  const int tr = dg::moe_tile_rows_min();   // the most tiles any tile size produces
  w.max_chunks = d.n_experts + static_cast<int>((T * d.top_k + tr - 1) / tr) +
                 static_cast<int>((T + tr - 1) / tr);
  w.chunks = c.take<int32_t>(static_cast<size_t>(w.max_chunks) * 3);
  w.n_chunks = c.take<int32_t>(1);
  w.act = c.take<uint16_t>(rows * fmax);
  w.y = c.take<uint16_t>(rows * d.d_model);
  w.eb = carve_eb(c, static_cast<int>(T), d.vocab / dg::gemm_lmhead_rows_per_block(), d.vocab);
  w.hot = c.take<uint8_t>(1024);
  // e4m3 canvas key and value rows (used with an fp8 KV cache; small, so always carved)
  const size_t kvrows = T * d.n_kv_heads;
  w.kq = c.take<uint8_t>(kvrows * d.head_dim);
  w.vq = c.take<uint8_t>(kvrows * d.head_dim);
  w.kqs = c.take<float>(kvrows);
  w.vqs = c.take<float>(kvrows);
  w.u8 = nullptr; w.u8s = nullptr; w.act32 = nullptr; w.act8 = nullptr; w.act8s = nullptr;
  if (d.wdtype == DG_FP8_E4M3) {
    w.u8 = c.take<uint8_t>(T * d.d_model);
    w.u8s = c.take<float>(T);
    w.act32 = c.take<float>(rows * fmax);
    w.act8 = c.take<uint8_t>(rows * fmax);
    w.act8s = c.take<float>(rows);
  }
  return w;
}

bool layer_global(const dg_dims& d, int l) {
  return d.window == 0 || (l + 1) % d.global_every == 0;
}

size_t kv_layer_elems(const dg_dims& d, const dg_kv* kv) {
  return static_cast<size_t>(kv->batch) * d.n_kv_heads * kv->cap * d.head_dim;
}

// need_room: the call appends C tokens per canvas
dg_status check_kv(const dg_model* m, const dg_kv* kv, bool need_room, int C = 0) {
  if (!kv || !kv->k || !kv->v || !kv->len) return fail(DG_ERR_NULL, "kv or a kv pointer is NULL");
  if (kv->dtype != DG_BF16 && kv->dtype != DG_FP8_E4M3)
    return fail(DG_ERR_SHAPE, "kv dtype %d is neither DG_BF16 nor DG_FP8_E4M3", kv->dtype);
  if (kv->dtype == DG_FP8_E4M3) {
    if (!kv->k_scale || !kv->v_scale) return fail(DG_ERR_NULL, "fp8 kv scale pointer is NULL");
    if (m->dims.head_dim != 128 && m->dims.head_dim != 256)
      return fail(DG_ERR_SHAPE, "an fp8 kv cache needs head_dim 128 or 256 (got %d)",
                  m->dims.head_dim);
  }
  if (kv->batch < 1 || kv->batch > 64) return fail(DG_ERR_SHAPE, "kv batch must be in [1, 64]");
  if (kv->cap < 1) return fail(DG_ERR_SHAPE, "kv capacity must be >= 1");
  for (int b = 0; b < kv->batch; ++b) {
    if (kv->len[b] < 0 || kv->len[b] > kv->cap)
      return fail(DG_ERR_CAPACITY, "kv len[%d] = %d outside [0, cap = %d]", b, kv->len[b], kv->cap);
    if (need_room && kv->len[b] + C > kv->cap)
      return fail(DG_ERR_CAPACITY, "kv len[%d] + %d appended tokens = %d exceeds cap %d", b, C,
                  kv->len[b] + C, kv->cap);
  }
  return DG_OK;
}

dg_status run_ffn(const dg_model* m, int l, int T, DecWs& w, const uint16_t* next_gain,
                  bool next_q8, float* trace_logits, int32_t* trace_idx, float* trace_gates,
                  hipStream_t s);

// One transformer layer on ws.h (the attention norm of this layer must already be in ws.u), over
// C tokens per canvas (the canvas, or the tokens an encoder pass appends).  causal: encoder pass
// (causal among the C tokens, writes their K/V into the cache); next_gain: the norm of the
// following consumer applied to the new h (NULL: none), with its e4m3 codes when next_q8.
// Optional router traces.
// A compacted decoder step runs only the canvases idx[0 .. n) of the batch (n == 0: all of them,
// in order); their cache rows, state rows and output rows are reached through idx.
struct BatchMap {
  int n = 0;
  int idx[64];
};

dg_status run_layer(const dg_model* m, const dg_kv* kv, int l, int C, bool causal, DecWs& w,
                    const uint16_t* next_gain, bool next_q8, bool skip_ffn, float* trace_logits,
                    int32_t* trace_idx, float* trace_gates, hipStream_t s,
                    const BatchMap* bm = nullptr) {
  const dg_dims& d = m->dims;
  const dg_layer_w& lw = m->layers[l];
  const bool mapped = bm && bm->n > 0;
  const int B = mapped ? bm->n : kv->batch, T = B * C;
  const int dq = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
  const size_t kvl = kv_layer_elems(d, kv);
  const bool f8 = kv->dtype == DG_FP8_E4M3;
  const size_t esz = f8 ? 1 : 2;      // bytes per cached element
  uint8_t* kc = static_cast<uint8_t*>(kv->k) + kvl * esz * l;
  uint8_t* vc = static_cast<uint8_t*>(kv->v) + kvl * esz * l;
  const size_t kvr = kvl / d.head_dim;  // rows (one scale each) per layer
  float* ksc = f8 ? kv->k_scale + kvr * l : nullptr;
  float* vsc = f8 ? kv->v_scale + kvr * l : nullptr;

  dg::WGemmArgs g;
  memset(&g, 0, sizeof(g));
  g.hot = w.hot;
  // QKV projection
  g.X = w.u; g.ldx = d.d_model; g.W = static_cast<const uint16_t*>(lw.w_qkv);
  g.K = g.K_sh = d.d_model; g.N = g.N_sh = dq; g.ntok = T; g.out = w.qkv; g.ldo = dq; g.ksplit = 1;
  DG_LAUNCH(PC_GEMM_QKV, s, dg::launch_dense_packed_bf16(g, s));

  // attention over [visible cache ; canvas]
  dg::AttnArgs at;
  memset(&at, 0, sizeof(at));
  at.qkv = w.qkv; at.cap = kv->cap;
  at.kc = reinterpret_cast<const uint16_t*>(kc);
  at.vc = reinterpret_cast<const uint16_t*>(vc);
  at.B = B; at.C = C; at.Hq = d.n_q_heads; at.Hkv = d.n_kv_heads; at.dh = d.head_dim;
  at.window = layer_global(d, l) ? 0 : d.window;
  at.causal = causal ? 1 : 0;
  for (int b = 0; b < B; ++b) {
    at.kvb[b] = mapped ? bm->idx[b] : b;
    at.len[b] = kv->len[at.kvb[b]];
  }
  // the key split is chosen for the whole batch, so a compacted step splits (and rounds) every
  // canvas's attention exactly as the full step does
  int max_keys = 0;
  for (int b = 0; b < kv->batch; ++b) {
    const int lo = at.window > 0 ? std::max(0, kv->len[b] - at.window + 1) : 0;
    max_keys = std::max(max_keys, kv->len[b] - lo + C);
  }
  at.scale_log2e = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(d.head_dim)));
  at.n_split = std::min(w.max_split, dg::attention_pick_split(kv->batch, C, d.n_q_heads,
                                                              d.n_kv_heads, max_keys));
  at.o_part = w.o_part; at.ml_part = w.ml_part; at.out = w.attn;
  if (f8) {
    // e4m3 rows of the canvas keys and values (an encoder pass also stores them in the cache at
    // len + i: rows the attention does not read from the cache)
    at.f8 = 1;
    at.ksc = ksc; at.vsc = vsc;
    at.kq = w.kq; at.vq = w.vq; at.kqs = w.kqs; at.vqs = w.vqs;
    DG_LAUNCH(PC_QUANT, s, dg::launch_kv_quant(at, w.kq, w.vq, w.kqs, w.vqs,
                                                  causal ? kc : nullptr, causal ? vc : nullptr,
                                                  causal ? ksc : nullptr, causal ? vsc : nullptr,
                                                  s));
  }
  DG_LAUNCH(PC_ATTENTION, s, dg::launch_attention(at, s));
  if (causal && !f8) {
    DG_LAUNCH(PC_KV_WRITE, s, dg::launch_kv_write(w.qkv, reinterpret_cast<uint16_t*>(kc),
                                                  reinterpret_cast<uint16_t*>(vc), B, C,
                                                  d.n_q_heads, d.n_kv_heads, d.head_dim,
                                                  kv->cap, kv->len, s));
  }
  if (skip_ffn) return DG_OK;

  // output projection (k-split partials) + residual + pre-FFN norm
  memset(&g, 0, sizeof(g));
  g.hot = w.hot;
  g.X = w.attn; g.ldx = d.n_q_heads * d.head_dim; g.W = static_cast<const uint16_t*>(lw.w_o);
  g.K = g.K_sh = d.n_q_heads * d.head_dim; g.N = g.N_sh = d.d_model; g.ntok = T;
  const int o_split = o_proj_split(kv->batch * C, d.d_model);
  g.out = w.proj_part; g.ldo = d.d_model; g.ksplit = o_split;
  g.split_stride = static_cast<long long>(T) * d.d_model;
  DG_LAUNCH(PC_GEMM_O, s, dg::launch_dense_packed_f32(g, s));
  DG_LAUNCH(PC_RMSNORM, s, dg::launch_resid_norm(w.h, w.proj_part, o_split, T, d.d_model,
                                                 static_cast<const uint16_t*>(lw.ffn_norm), w.u,
                                                 d.norm_eps, w.u8, w.u8s, s));
  return run_ffn(m, l, T, w, next_gain, next_q8, trace_logits, trace_idx, trace_gates, s);
}

// The FFN half of a layer on ws.h, whose pre-FFN norm (and, for fp8, its e4m3 codes) is in ws.u:
// router, top-k, permutation, routed + shared SwiGLU experts, combine (+ the next norm).
dg_status run_ffn(const dg_model* m, int l, int T, DecWs& w, const uint16_t* next_gain,
                  bool next_q8, float* trace_logits, int32_t* trace_idx, float* trace_gates,
                  hipStream_t s) {
  const dg_dims& d = m->dims;
  const dg_layer_w& lw = m->layers[l];
  const bool fp8 = m->fp8();
  dg::WGemmArgs g;
  // router
  memset(&g, 0, sizeof(g));
  g.hot = w.hot;
  g.X = w.u; g.ldx = d.d_model; g.W = static_cast<const uint16_t*>(lw.w_router);
  g.K = g.K_sh = d.d_model; g.N = g.N_sh = d.n_experts; g.ntok = T;
  g.out = w.router_part; g.ldo = d.n_experts; g.ksplit = kRouterSplit;
  g.split_stride = static_cast<long long>(T) * d.n_experts;
  DG_LAUNCH(PC_GEMM_ROUTER, s, dg::launch_gemm_dense_f32(g, s));
  int32_t* idx = trace_idx ? trace_idx : w.topk;
  float* gates = trace_gates ? trace_gates : w.gates;
  DG_LAUNCH(PC_TOPK, s, dg::launch_topk(w.router_part, kRouterSplit, T, d.n_experts, d.top_k, idx,
                                        gates, trace_logits, s));
  // expert tiles: wide ones for long prefill chunks and large batches (bf16 and e4m3 weights)
  const int tile_rows = dg::moe_tile_rows(T);
  DG_LAUNCH(PC_PERMUTE, s, dg::launch_permute(idx, T, d.top_k, d.n_experts,
                                              tile_rows, w.perm, w.inv, w.chunks,
                                              w.n_chunks, w.max_chunks, s));
  // routed + shared experts: gate/up with SwiGLU, then down
  const int fmax = std::max(d.ffn_inner, d.shared_inner);
  memset(&g, 0, sizeof(g));
  g.hot = w.hot;
  g.X = w.u; g.ldx = d.d_model; g.x_rows = w.perm;
  g.W = static_cast<const uint16_t*>(lw.w_gate_up);
  g.w_estride = 2LL * d.ffn_inner * d.d_model;
  g.W_sh = static_cast<const uint16_t*>(lw.ws_gate_up);
  g.K = g.K_sh = d.d_model; g.N = d.ffn_inner; g.N_sh = d.shared_inner;
  g.n_experts = d.n_experts; g.chunks = w.chunks; g.n_chunks = w.n_chunks;
  g.grid_tiles = w.max_chunks; g.out = w.act; g.ldo = fmax; g.ksplit = 1;
  g.sh_tiles = (T + tile_rows - 1) / tile_rows;
  const long long rows = static_cast<long long>(T) * d.top_k + T;
  if (fp8) {
    // e4m3 codes of u (gathered through the permutation), fp32 SwiGLU output, then its codes
    g.X = reinterpret_cast<const uint16_t*>(w.u8); g.x_scale = w.u8s;
    g.w_scale = lw.s_gate_up; g.wsc_estride = 2LL * d.ffn_inner; g.w_scale_sh = lw.ss_gate_up;
    g.out = w.act32;
    DG_LAUNCH(PC_MOE_GATEUP, s, dg::launch_moe_gateup_fp8(g, tile_rows, s));
    DG_LAUNCH(PC_QUANT, s, dg::launch_quant_rows(w.act32, true, fmax, w.act8, fmax, w.act8s, rows,
                                                 static_cast<long long>(T) * d.top_k,
                                                 d.ffn_inner, d.shared_inner, s));
  } else {
    DG_LAUNCH(PC_MOE_GATEUP, s, dg::launch_moe_gateup(g, tile_rows, s));
  }
  memset(&g, 0, sizeof(g));
  g.hot = w.hot;
  g.X = w.act; g.ldx = fmax; g.W = static_cast<const uint16_t*>(lw.w_down);
  g.w_estride = static_cast<long long>(d.d_model) * d.ffn_inner;
  g.W_sh = static_cast<const uint16_t*>(lw.ws_down);
  g.K = d.ffn_inner; g.K_sh = d.shared_inner; g.N = g.N_sh = d.d_model;
  g.n_experts = d.n_experts; g.chunks = w.chunks; g.n_chunks = w.n_chunks;
  g.grid_tiles = w.max_chunks; g.out = w.y; g.ldo = d.d_model; g.ksplit = 1;
  g.sh_tiles = (T + tile_rows - 1) / tile_rows;
  if (fp8) {
    g.X = reinterpret_cast<const uint16_t*>(w.act8); g.x_scale = w.act8s;
    g.w_scale = lw.s_down; g.wsc_estride = d.d_model; g.w_scale_sh = lw.ss_down;
    DG_LAUNCH(PC_MOE_DOWN, s, dg::launch_moe_down_fp8(g, tile_rows, s));
  } else {
    DG_LAUNCH(PC_MOE_DOWN, s, dg::launch_moe_down(g, tile_rows, s));
  }
  DG_LAUNCH(PC_COMBINE, s, dg::launch_combine(w.h, w.y, w.inv, gates, T, d.top_k, d.d_model,
                                              next_gain, w.u, d.norm_eps,
                                              next_q8 ? w.u8 : nullptr,
                                              next_q8 ? w.u8s : nullptr, s));
  return DG_OK;
}

dg_status check_model(const dg_model* m) {
  if (!m) return fail(DG_ERR_NULL, "model is NULL");
  return DG_OK;
}

// LM head over the final norm in ws.u (fp8: its e4m3 codes in ws.u8) with the tempered
// statistics epilogue; logits [T][V] bf16
dg_status run_lm_head(const dg_model* m, int T, DecWs& w, uint16_t* logits, float inv_t_log2e,
                      hipStream_t s, const BatchMap* bm = nullptr) {
  const dg_dims& d = m->dims;
  dg::WGemmArgs g;
  memset(&g, 0, sizeof(g));
  if (bm && bm->n > 0) {
    g.omap_C = d.canvas_len;
    for (int b = 0; b < bm->n; ++b) g.omap[b] = bm->idx[b];
  }
  g.hot = w.hot;
  g.X = w.u; g.ldx = d.d_model; g.W = static_cast<const uint16_t*>(m->w_lm);
  g.K = g.K_sh = d.d_model; g.N = g.N_sh = d.vocab; g.ntok = T; g.out = logits;
  g.ldo = d.vocab; g.ksplit = 1; g.inv_t_log2e = inv_t_log2e; g.part = w.eb.part;
  if (m->fp8()) {
    g.X = reinterpret_cast<const uint16_t*>(w.u8); g.x_scale = w.u8s; g.w_scale = m->s_lm;
    DG_LAUNCH(PC_LMHEAD, s, dg::launch_lmhead_packed_fp8(g, s));
  } else {
    DG_LAUNCH(PC_LMHEAD, s, dg::launch_lmhead_packed(g, s));
  }
  return DG_OK;
}

}  // namespace

extern "C" {

size_t dg_workspace_bytes(const dg_model* m, int32_t batch) {
  if (!m || batch < 1 || batch > 64) return 0;
  Carver c(nullptr);
  carve_dec(c, m->dims, batch, m->dims.canvas_len);
  return c.off + 256;
}

size_t dg_append_workspace_bytes(const dg_model* m, int32_t batch, int32_t max_tokens) {
  if (!m || batch < 1 || batch > 64 || max_tokens < 1 || max_tokens > DG_MAX_APPEND_TOKENS ||
      static_cast<long long>(batch) * max_tokens > 65536)
    return 0;
  Carver c(nullptr);
  carve_dec(c, m->dims, batch, max_tokens);
  return c.off + 256;
}

// The decoder step over the canvases of `bm` (all of them when bm is NULL), checked by the caller
static dg_status decoder_step_rows(const dg_model* m, const dg_kv* kv, int32_t step,
                                   const dg_sched_params* p, dg_eb_state* st, dg_step_out* out,
                                   void* ws, hipStream_t hs, const BatchMap* bm) {
  const dg_dims& d = m->dims;
  const bool mapped = bm && bm->n > 0;
  const int B = mapped ? bm->n : kv->batch, C = d.canvas_len, T = B * C;
  Carver c(ws);
  DecWs w = carve_dec(c, d, kv->batch, C);
  dg_status s;
  DG_LAUNCH(PC_EMBED, hs, dg::launch_embed(st->canvas, m->embed, w.h, T, d.d_model, d.vocab, hs,
                                           C, mapped ? bm->n : 0, mapped ? bm->idx : nullptr));
  DG_LAUNCH(PC_RMSNORM, hs, dg::launch_rmsnorm(w.h, static_cast<const uint16_t*>(m->layers[0].attn_norm),
                                               w.u, T, d.d_model, d.norm_eps, nullptr, nullptr, hs));
  for (int l = 0; l < d.n_layers; ++l) {
    const bool last = l + 1 == d.n_layers;
    const uint16_t* next = !last ? static_cast<const uint16_t*>(m->layers[l + 1].attn_norm)
                                 : m->final_norm;
    if ((s = run_layer(m, kv, l, C, false, w, next, last && m->fp8(), false, nullptr, nullptr,
                       nullptr, hs, bm)) != DG_OK)
      return s;
  }
  // LM head with the tempered statistics, then the sampler
  dg::EbArgs a = eb_args(p, B, C, d.vocab, step, st, out, out->logits, w.eb);
  if (mapped) {
    a.mapped = 1;
    for (int b = 0; b < bm->n; ++b) a.bmap[b] = bm->idx[b];
  }
  if ((s = run_lm_head(m, T, w, out->logits, a.inv_t_log2e, hs, bm)) != DG_OK) return s;
  return run_sampler_tail(a, hs);
}

dg_status dg_decoder_step_sched(const dg_model* m, const dg_kv* kv, int32_t step,
                                const dg_sched_params* p, dg_eb_state* st, dg_step_out* out,
                                void* ws, size_t ws_bytes, void* stream) {
  dg_status s = check_model(m);
  if (s != DG_OK) return s;
  if ((s = check_kv(m, kv, false)) != DG_OK) return s;
  if ((s = check_sched(p, step)) != DG_OK) return s;
  if ((s = check_state(st)) != DG_OK) return s;
  if ((s = check_out(out, true)) != DG_OK) return s;
  if (!ws) return fail(DG_ERR_NULL, "workspace is NULL");
  const size_t need = dg_workspace_bytes(m, kv->batch);
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  return decoder_step_rows(m, kv, step, p, st, out, ws, static_cast<hipStream_t>(stream),
                           nullptr);
}

dg_status dg_decoder_step_live(const dg_model* m, const dg_kv* kv, int32_t step,
                               const dg_sched_params* p, dg_eb_state* st, dg_step_out* out,
                               int32_t n_live, const int32_t* live, void* ws, size_t ws_bytes,
                               void* stream) {
  dg_status s = check_model(m);
  if (s != DG_OK) return s;
  if ((s = check_kv(m, kv, false)) != DG_OK) return s;
  if ((s = check_sched(p, step)) != DG_OK) return s;
  if ((s = check_state(st)) != DG_OK) return s;
  if ((s = check_out(out, true)) != DG_OK) return s;
  if (!ws || !live) return fail(DG_ERR_NULL, "workspace or live is NULL");
  if (n_live < 1 || n_live > kv->batch)
    return fail(DG_ERR_SHAPE, "n_live = %d outside [1, %d]", n_live, kv->batch);
  BatchMap bm;
  bm.n = n_live;
  bool seen[64] = {};
  for (int j = 0; j < n_live; ++j) {
    if (live[j] < 0 || live[j] >= kv->batch || seen[live[j]])
      return fail(DG_ERR_SHAPE, "live[%d] = %d is out of range or repeated", j, live[j]);
    seen[live[j]] = true;
    bm.idx[j] = live[j];
  }
  const size_t need = dg_workspace_bytes(m, kv->batch);
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  return decoder_step_rows(m, kv, step, p, st, out, ws, static_cast<hipStream_t>(stream), &bm);
}

dg_status dg_decoder_step(const dg_model* m, const dg_kv* kv, int32_t step, const dg_eb_params* p,
                          dg_eb_state* st, dg_step_out* out, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!p) return fail(DG_ERR_NULL, "params is NULL");
  const dg_sched_params q = sched_from_eb(p);
  return dg_decoder_step_sched(m, kv, step, &q, st, out, ws, ws_bytes, stream);
}

// The encoder pass over C new tokens per canvas (checked by the caller): causal among them,
// each layer writing their keys and values at [len, len + C); then len += C
static dg_status encoder_append(const dg_model* m, dg_kv* kv, const int32_t* tokens, int C,
                                void* ws, size_t ws_bytes, hipStream_t hs) {
  const dg_dims& d = m->dims;
  const int B = kv->batch, T = B * C;
  Carver sz(nullptr);
  carve_dec(sz, d, B, C);
  if (ws_bytes < sz.off + 256)
    return fail(DG_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, sz.off + 256);
  Carver c(ws);
  DecWs w = carve_dec(c, d, B, C);
  dg_status s;
  DG_LAUNCH(PC_EMBED, hs, dg::launch_embed(tokens, m->embed, w.h, T, d.d_model, d.vocab, hs));
  DG_LAUNCH(PC_RMSNORM, hs, dg::launch_rmsnorm(w.h, static_cast<const uint16_t*>(m->layers[0].attn_norm),
                                               w.u, T, d.d_model, d.norm_eps, nullptr, nullptr, hs));
  for (int l = 0; l < d.n_layers; ++l) {
    const bool last = l + 1 == d.n_layers;  // its keys/values are all the last layer adds
    const uint16_t* next = last ? nullptr : static_cast<const uint16_t*>(m->layers[l + 1].attn_norm);
    if ((s = run_layer(m, kv, l, C, true, w, next, false, last, nullptr, nullptr, nullptr, hs)) !=
        DG_OK)
      return s;
  }
  for (int b = 0; b < B; ++b) kv->len[b] += C;
  return DG_OK;
}

dg_status dg_kv_append_canvas(const dg_model* m, dg_kv* kv, const int32_t* tokens, void* ws,
                              size_t ws_bytes, void* stream) {
  dg_status s = check_model(m);
  if (s != DG_OK) return s;
  if ((s = check_kv(m, kv, true, m->dims.canvas_len)) != DG_OK) return s;
  if (!tokens || !ws) return fail(DG_ERR_NULL, "tokens or workspace is NULL");
  return encoder_append(m, kv, tokens, m->dims.canvas_len, ws, ws_bytes,
                        static_cast<hipStream_t>(stream));
}

dg_status dg_kv_append_tokens(const dg_model* m, dg_kv* kv, const int32_t* tokens,
                              int32_t n_tokens, void* ws, size_t ws_bytes, void* stream) {
  dg_status s = check_model(m);
  if (s != DG_OK) return s;
  if (!tokens || !ws) return fail(DG_ERR_NULL, "tokens or workspace is NULL");
  if (n_tokens < 1 || n_tokens > DG_MAX_APPEND_TOKENS)
    return fail(DG_ERR_SHAPE, "n_tokens = %d outside [1, %d]", n_tokens, DG_MAX_APPEND_TOKENS);
  if (m->dims.window > 0 && n_tokens > m->dims.window)
    return fail(DG_ERR_SHAPE, "n_tokens = %d exceeds the sliding window %d", n_tokens,
                m->dims.window);
  if ((s = check_kv(m, kv, true, n_tokens)) != DG_OK) return s;
  if (static_cast<long long>(kv->batch) * n_tokens > 65536)
    return fail(DG_ERR_SHAPE, "batch * n_tokens = %lld exceeds 65,536",
                static_cast<long long>(kv->batch) * n_tokens);
  return encoder_append(m, kv, tokens, n_tokens, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

size_t dg_generate_workspace_bytes(const dg_model* m, int32_t batch) {
  const size_t base = dg_workspace_bytes(m, batch);
  return base ? base + 512 : 0;   // + the canvas ids of the current canvas, 256-byte aligned
}

dg_status dg_generate_sched(const dg_model* m, dg_kv* kv, const dg_gen_params* gen,
                            const dg_sched_params* p, dg_eb_state* state, dg_step_out* out,
                            int32_t* tokens, int32_t* canvases, int32_t* steps, void* ws,
                            size_t ws_bytes, void* stream) {
  dg_status s = check_model(m);
  if (s != DG_OK) return s;
  if (!gen || !tokens || !canvases || !ws) return fail(DG_ERR_NULL, "gen, tokens, canvases or ws is NULL");
  const int C = m->dims.canvas_len;
  if (gen->gen_length < 1) return fail(DG_ERR_SHAPE, "gen_length must be >= 1");
  const long long total_ll = (static_cast<long long>(gen->gen_length) + C - 1) / C;
  if ((s = check_sched(p, 0)) != DG_OK) return s;
  if ((s = check_state(state)) != DG_OK) return s;
  if ((s = check_out(out, true)) != DG_OK) return s;
  if ((s = check_kv(m, kv, false)) != DG_OK) return s;
  for (int b = 0; b < kv->batch; ++b)
    if (kv->len[b] + total_ll * C > kv->cap)
      return fail(DG_ERR_CAPACITY, "kv len[%d] + %lld generated tokens exceeds cap %d", b,
                  total_ll * C, kv->cap);
  const int B = kv->batch, total = static_cast<int>(total_ll);
  if (static_cast<long long>(total) * B > (1ll << 31))
    return fail(DG_ERR_SHAPE, "too many canvases for 31-bit canvas ids");
  const size_t need = dg_generate_workspace_bytes(m, B);
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const size_t step_ws = dg_workspace_bytes(m, B);
  uint32_t* ids = reinterpret_cast<uint32_t*>(
      (reinterpret_cast<uintptr_t>(ws) + step_ws + 255) & ~static_cast<uintptr_t>(255));
  dg_eb_state st = *state;
  st.canvas_id = ids;
  std::vector<uint32_t> hid(B);
  std::vector<int32_t> hdone(B), hcanvas(static_cast<size_t>(B) * C), live;
  std::vector<char> has_eos(B, 0);
  *canvases = 0;
  for (int c = 0; c < total; ++c) {
    // canvas c of sequence b draws its noise with canvas id c * B + b
    for (int b = 0; b < B; ++b) hid[b] = static_cast<uint32_t>(c * B + b);
    DG_HIP(hipMemcpyAsync(ids, hid.data(), sizeof(uint32_t) * B, hipMemcpyHostToDevice, hs));
    DG_LAUNCH(PC_EB_COMMIT, hs, dg::launch_canvas_init(p->seed, st, B, C, m->dims.vocab, hs));
    live.resize(B);
    for (int b = 0; b < B; ++b) live[b] = b;
    int n = 0;
    for (int step = 0; step < p->max_steps; ++step) {
      // with compaction, a step runs only the samples not yet frozen
      if (gen->compact_frozen && static_cast<int>(live.size()) < B)
        s = dg_decoder_step_live(m, kv, step, p, &st, out, static_cast<int32_t>(live.size()),
                                 live.data(), ws, step_ws, stream);
      else
        s = dg_decoder_step_sched(m, kv, step, p, &st, out, ws, step_ws, stream);
      if (s != DG_OK) return s;
      ++n;
      // adaptive stop: the canvas's loop ends once every sample is frozen
      DG_HIP(hipMemcpyAsync(hdone.data(), st.done, sizeof(int32_t) * B, hipMemcpyDeviceToHost, hs));
      DG_HIP(hipStreamSynchronize(hs));
      live.clear();
      for (int b = 0; b < B; ++b)
        if (!hdone[b]) live.push_back(b);
      if (live.empty()) break;
    }
    DG_HIP(hipMemcpy2DAsync(tokens + static_cast<size_t>(c) * C, sizeof(int32_t) * total * C,
                            st.canvas, sizeof(int32_t) * C, sizeof(int32_t) * C, B,
                            hipMemcpyDeviceToDevice, hs));
    if ((s = dg_kv_append_canvas(m, kv, st.canvas, ws, step_ws, stream)) != DG_OK) return s;
    if (steps) steps[c] = n;
    *canvases = c + 1;
    if (gen->eos_token_id >= 0) {
      DG_HIP(hipMemcpyAsync(hcanvas.data(), st.canvas, sizeof(int32_t) * B * C,
                            hipMemcpyDeviceToHost, hs));
      DG_HIP(hipStreamSynchronize(hs));
      bool all = true;
      for (int b = 0; b < B; ++b) {
        for (int i = 0; i < C && !has_eos[b]; ++i) has_eos[b] = hcanvas[b * C + i] == gen->eos_token_id;
        all = all && has_eos[b];
      }
      if (gen->eos_early_stop && all) break;
    }
  }
  return DG_OK;
}

dg_status dg_generate(const dg_model* m, dg_kv* kv, const dg_gen_params* gen,
                      const dg_eb_params* p, dg_eb_state* state, dg_step_out* out,
                      int32_t* tokens, int32_t* canvases, int32_t* steps, void* ws,
                      size_t ws_bytes, void* stream) {
  if (!p) return fail(DG_ERR_NULL, "params is NULL");
  const dg_sched_params q = sched_from_eb(p);
  return dg_generate_sched(m, kv, gen, &q, state, out, tokens, canvases, steps, ws, ws_bytes,
                           stream);
}

// One layer over C tokens per canvas (the canvas, or an encoder call's token count) on the
// caller's residual stream; ws is carved for C tokens per canvas
static dg_status layer_forward_n(const dg_model* m, const dg_kv* kv, int layer, bool causal,
                                 int C, float* h, float* router_logits, int32_t* topk_idx,
                                 float* gates, void* ws, size_t ws_bytes, hipStream_t hs) {
  const dg_dims& d = m->dims;
  Carver sz(nullptr);
  carve_dec(sz, d, kv->batch, C);
  if (ws_bytes < sz.off + 256)
    return fail(DG_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, sz.off + 256);
  const int T = kv->batch * C;
  Carver c(ws);
  DecWs w = carve_dec(c, d, kv->batch, C);
  dg_status s;
  DG_HIP(hipMemcpyAsync(w.h, h, sizeof(float) * T * d.d_model, hipMemcpyDeviceToDevice, hs));
  DG_LAUNCH(PC_RMSNORM, hs, dg::launch_rmsnorm(w.h, static_cast<const uint16_t*>(m->layers[layer].attn_norm),
                                               w.u, T, d.d_model, d.norm_eps, nullptr, nullptr, hs));
  if ((s = run_layer(m, kv, layer, C, causal, w, nullptr, false, false, router_logits, topk_idx,
                     gates, hs)) != DG_OK)
    return s;
  DG_HIP(hipMemcpyAsync(h, w.h, sizeof(float) * T * d.d_model, hipMemcpyDeviceToDevice, hs));
  return DG_OK;
}

dg_status dg_layer_forward(const dg_model* m, const dg_kv* kv, int32_t layer, int32_t causal,
                           float* h, float* router_logits, int32_t* topk_idx, float* gates,
                           void* ws, size_t ws_bytes, void* stream) {
  dg_status s = check_model(m);
  if (s != DG_OK) return s;
  if ((s = check_kv(m, kv, causal != 0, m->dims.canvas_len)) != DG_OK) return s;
  if (!h || !ws) return fail(DG_ERR_NULL, "h or workspace is NULL");
  if (layer < 0 || layer >= m->dims.n_layers) return fail(DG_ERR_SHAPE, "layer out of range");
  const size_t need = dg_workspace_bytes(m, kv->batch);
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  return layer_forward_n(m, kv, layer, causal != 0, m->dims.canvas_len, h, router_logits,
                         topk_idx, gates, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

dg_status dg_layer_forward_tokens(const dg_model* m, const dg_kv* kv, int32_t layer,
                                  int32_t n_tokens, float* h, float* router_logits,
                                  int32_t* topk_idx, float* gates, void* ws, size_t ws_bytes,
                                  void* stream) {
  dg_status s = check_model(m);
  if (s != DG_OK) return s;
  if (!h || !ws) return fail(DG_ERR_NULL, "h or workspace is NULL");
  if (layer < 0 || layer >= m->dims.n_layers) return fail(DG_ERR_SHAPE, "layer out of range");
  if (n_tokens < 1 || n_tokens > DG_MAX_APPEND_TOKENS)
    return fail(DG_ERR_SHAPE, "n_tokens = %d outside [1, %d]", n_tokens, DG_MAX_APPEND_TOKENS);
  if (m->dims.window > 0 && n_tokens > m->dims.window)
    return fail(DG_ERR_SHAPE, "n_tokens = %d exceeds the sliding window %d", n_tokens,
                m->dims.window);
  if ((s = check_kv(m, kv, true, n_tokens)) != DG_OK) return s;
  if (static_cast<long long>(kv->batch) * n_tokens > 65536)
    return fail(DG_ERR_SHAPE, "batch * n_tokens exceeds 65,536");
  return layer_forward_n(m, kv, layer, true, n_tokens, h, router_logits, topk_idx, gates, ws,
                         ws_bytes, static_cast<hipStream_t>(stream));
}

dg_status dg_ffn_forward(const dg_model* m, int32_t layer, int32_t batch, float* h,
                         float* router_logits, int32_t* topk_idx, float* gates, void* ws,
                         size_t ws_bytes, void* stream) {
  dg_status s = check_model(m);
  if (s != DG_OK) return s;
  if (!h || !ws) return fail(DG_ERR_NULL, "h or workspace is NULL");
  if (layer < 0 || layer >= m->dims.n_layers) return fail(DG_ERR_SHAPE, "layer out of range");
  if (batch < 1 || batch > 64) return fail(DG_ERR_SHAPE, "batch must be in [1, 64]");
  const size_t need = dg_workspace_bytes(m, batch);
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  const dg_dims& d = m->dims;
  const int T = batch * d.canvas_len;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  Carver c(ws);
  DecWs w = carve_dec(c, d, batch, d.canvas_len);
  DG_HIP(hipMemcpyAsync(w.h, h, sizeof(float) * T * d.d_model, hipMemcpyDeviceToDevice, hs));
  DG_LAUNCH(PC_RMSNORM, hs, dg::launch_rmsnorm(w.h, static_cast<const uint16_t*>(m->layers[layer].ffn_norm),
                                               w.u, T, d.d_model, d.norm_eps, w.u8, w.u8s, hs));
  if ((s = run_ffn(m, layer, T, w, nullptr, false, router_logits, topk_idx, gates, hs)) != DG_OK)
    return s;
  DG_HIP(hipMemcpyAsync(h, w.h, sizeof(float) * T * d.d_model, hipMemcpyDeviceToDevice, hs));
  return DG_OK;
}

dg_status dg_lm_head_forward(const dg_model* m, int32_t batch, const float* h, int32_t step,
                             const dg_eb_params* p, dg_step_out* out, void* ws, size_t ws_bytes,
                             void* stream) {
  dg_status s = check_model(m);
  if (s != DG_OK) return s;
  if (!h || !ws) return fail(DG_ERR_NULL, "h or workspace is NULL");
  if ((s = check_params(p, step)) != DG_OK) return s;
  if (!out || !out->entropy || !out->argmax || !out->logits)
    return fail(DG_ERR_NULL, "out, out->entropy, out->argmax or out->logits is NULL");
  if (batch < 1 || batch > 64) return fail(DG_ERR_SHAPE, "batch must be in [1, 64]");
  const size_t need = dg_workspace_bytes(m, batch);
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  const dg_dims& d = m->dims;
  const int T = batch * d.canvas_len;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  Carver c(ws);
  DecWs w = carve_dec(c, d, batch, d.canvas_len);
  DG_LAUNCH(PC_RMSNORM, hs, dg::launch_rmsnorm(h, m->final_norm, w.u, T, d.d_model, d.norm_eps,
                                               w.u8, w.u8s, hs));
  dg_eb_state none;
  memset(&none, 0, sizeof(none));
  const dg_sched_params q = sched_from_eb(p);
  dg::EbArgs a = eb_args(&q, batch, d.canvas_len, d.vocab, step, &none, out, out->logits, w.eb);
  if ((s = run_lm_head(m, T, w, out->logits, a.inv_t_log2e, hs)) != DG_OK) return s;
  DG_LAUNCH(PC_STATS_MERGE, hs, dg::launch_stats_merge(a, hs));
  return DG_OK;
}

dg_status dg_quantize_rows_fp8(const void* src, int32_t src_is_f32, uint8_t* codes, float* scales,
                               int64_t rows, int64_t cols, void* stream) {
  if (!src || !codes || !scales) return fail(DG_ERR_NULL, "NULL pointer");
  if (rows < 1 || cols < 4 || cols % 4 || rows > 0x7fffffffLL)
    return fail(DG_ERR_SHAPE, "need rows >= 1 and cols a positive multiple of 4");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  DG_LAUNCH(PC_QUANT, hs, dg::launch_quant_rows(src, src_is_f32 != 0, cols, codes, cols, scales,
                                                rows, rows, static_cast<int>(cols),
                                                static_cast<int>(cols), hs));
  return DG_OK;
}

dg_status dg_pack_weight_fp8(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t cols,
                             void* stream) {
  if (!src || !dst) return fail(DG_ERR_NULL, "NULL pointer");
  if (rows < 16 || cols < 64 || rows % 16 || cols % 64)
    return fail(DG_ERR_SHAPE, "rows must be a multiple of 16 and cols a multiple of 64");
  if (src == dst) return fail(DG_ERR_SHAPE, "src and dst must not alias");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  DG_LAUNCH(PC_COPY, hs, dg::launch_pack_fp8(src, dst, rows, cols, hs));
  return DG_OK;
}

}  // extern "C"
