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
  const uint16_t* w_lm;
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
  PC_EB_COMMIT, PC_CANDIDATES, PC_CAND_APPLY, PC_KV_WRITE, PC_COPY, PC_COUNT
};
const char* kProfNames[PC_COUNT] = {
    "embed", "rmsnorm", "gemm_qkv", "attention", "gemm_o", "gemm_router", "topk",
    "permute", "moe_gateup", "moe_down", "combine", "lmhead", "logit_stats", "stats_merge",
    "eb_commit", "candidates", "cand_apply", "kv_write", "copy"};

struct Prof {
  std::mutex mu;
  bool on = false;
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
  if (g_prof.on) {
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
};

// The sampler's scratch, carved the same way for dg_eb_sample and dg_decoder_step.
EbWs carve_eb(Carver& c, int rows, int n_part, int vocab) {
  EbWs w;
  w.n_part = n_part;
  w.part = c.take<dg::SoftStats>(static_cast<size_t>(rows) * n_part);
  w.need = c.take<uint8_t>(rows);
  w.n_cand = dg::cand_chunks(vocab);
  w.cand_score = c.take<double>(static_cast<size_t>(rows) * w.n_cand);
  w.cand_idx = c.take<int32_t>(static_cast<size_t>(rows) * w.n_cand);
  return w;
}

dg_status check_params(const dg_eb_params* p, int32_t step) {
  if (!p) return fail(DG_ERR_NULL, "params is NULL");
  if (p->max_steps < 1) return fail(DG_ERR_STATE, "max_steps must be >= 1");
  if (step < 0 || step >= p->max_steps)
    return fail(DG_ERR_STATE, "step %d outside [0, %d)", step, p->max_steps);
  if (!(p->t_max > 0.0) || !(p->t_min > 0.0)) return fail(DG_ERR_STATE, "temperatures must be > 0");
  if (!(p->entropy_bound >= 0.0)) return fail(DG_ERR_STATE, "entropy_bound must be >= 0");
  if (p->stability < 0) return fail(DG_ERR_STATE, "stability must be >= 0");
  return DG_OK;
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

// T_s = t_max + (t_min - t_max) s / (S - 1) in fp64; the kernels use fp32(1 / T_s)
void temperature(const dg_eb_params* p, int step, float* inv_t, float* inv_t_log2e) {
  double t = p->t_max;
  if (p->max_steps > 1)
    t = p->t_max + (p->t_min - p->t_max) * static_cast<double>(step) /
                       static_cast<double>(p->max_steps - 1);
  *inv_t = static_cast<float>(1.0 / t);
  *inv_t_log2e = static_cast<float>(static_cast<double>(*inv_t) * 1.4426950408889634);
}

dg::EbArgs eb_args(const dg_eb_params* p, int B, int C, int V, int step, const dg_eb_state* st,
                   const dg_step_out* out, const uint16_t* logits, const EbWs& w) {
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
  return a;
}

// stats partials are ready: merge, commit, candidates
dg_status run_sampler_tail(const dg::EbArgs& a, hipStream_t s) {
  DG_LAUNCH(PC_STATS_MERGE, s, dg::launch_stats_merge(a, s));
  DG_LAUNCH(PC_EB_COMMIT, s, dg::launch_eb_commit(a, s));
  DG_LAUNCH(PC_CANDIDATES, s, dg::launch_candidates(a, s));
  DG_LAUNCH(PC_CAND_APPLY, s, dg::launch_cand_apply(a, s));
  return DG_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------------

extern "C" {

const char* dg_last_error(void) { return g_err; }

dg_status dg_model_create(const dg_dims* d, const dg_layer_w* layers, const void* embed,
                          const void* final_norm, const void* w_lm, dg_model** out) {
  if (!d || !layers || !embed || !final_norm || !w_lm || !out)
    return fail(DG_ERR_NULL, "dg_model_create: NULL argument");
  *out = nullptr;
  if (d->wdtype != DG_BF16) return fail(DG_ERR_DTYPE, "only DG_BF16 weights are supported");
  if (d->n_layers < 1 || d->d_model < 32 || d->n_q_heads < 1 || d->n_kv_heads < 1 ||
      d->head_dim < 16)
    return fail(DG_ERR_SHAPE, "non-positive or too small dimension");
  if (d->d_model % 32 || d->ffn_inner % 32 || d->shared_inner % 32)
    return fail(DG_ERR_SHAPE, "d_model, ffn_inner and shared_inner must be multiples of 32");
  if (d->head_dim % 16 || d->head_dim > 256)
    return fail(DG_ERR_SHAPE, "head_dim must be a multiple of 16 and <= 256");
  if (d->n_q_heads % d->n_kv_heads) return fail(DG_ERR_SHAPE, "n_q_heads %% n_kv_heads != 0");
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
  }
  dg_model* m = new (std::nothrow) dg_model;
  if (!m) return fail(DG_ERR_HIP, "host allocation failed");
  m->dims = *d;
  m->layers.assign(layers, layers + d->n_layers);
  m->embed = static_cast<const uint16_t*>(embed);
  m->final_norm = static_cast<const uint16_t*>(final_norm);
  m->w_lm = static_cast<const uint16_t*>(w_lm);
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

dg_status dg_eb_sample(const uint16_t* logits, int32_t B, int32_t C, int32_t V, int32_t step,
                       const dg_eb_params* p, dg_eb_state* st, dg_step_out* out, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!logits || !ws) return fail(DG_ERR_NULL, "logits or workspace is NULL");
  dg_status s = check_params(p, step);
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

dg_status dg_copy_bytes(void* dst, const void* src, size_t n, void* stream) {
  if (!dst || !src) return fail(DG_ERR_NULL, "NULL pointer");
  if (n % 16) return fail(DG_ERR_SHAPE, "n must be a multiple of 16");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  DG_LAUNCH(PC_COPY, hs, dg::launch_copy(dst, src, n, hs));
  return DG_OK;
}

int32_t dg_prof_num_classes(void) { return PC_COUNT; }

const char* dg_prof_class_name(int32_t cls) {
  return (cls >= 0 && cls < PC_COUNT) ? kProfNames[cls] : "";
}

dg_status dg_prof_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = on != 0;
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

// ---- decoder entry points (filled in with the decoder kernels) ----------------------------
extern "C" {
size_t dg_workspace_bytes(const dg_model* m, int32_t batch) { (void)m; (void)batch; return 0; }
dg_status dg_decoder_step(const dg_model*, const dg_kv*, int32_t, const dg_eb_params*,
                          dg_eb_state*, dg_step_out*, void*, size_t, void*) {
  return fail(DG_ERR_UNSUPPORTED, "dg_decoder_step not built yet");
}
dg_status dg_kv_append_canvas(const dg_model*, dg_kv*, const int32_t*, void*, size_t, void*) {
  return fail(DG_ERR_UNSUPPORTED, "dg_kv_append_canvas not built yet");
}
dg_status dg_layer_forward(const dg_model*, const dg_kv*, int32_t, int32_t, float*, float*,
                           int32_t*, float*, void*, size_t, void*) {
  return fail(DG_ERR_UNSUPPORTED, "dg_layer_forward not built yet");
}
}
