/*
 * dg.h - C ABI of libdg.so: one denoising step of a block-diffusion decoder over a token canvas,
 * fused with the entropy-bound (EB) sampler, and the append of a finished canvas to the KV cache.
 *
 * What the calls compute comes from these passages:
 *   - DiffusionGemma model card, "Model overview": an encoder prefills the prompt into a KV cache;
 *     a decoder denoises a block ("canvas") of tokens with bidirectional attention over the canvas
 *     and cross-attention to the cached context; a finished canvas is processed by the encoder
 *     and appended to the KV cache before the next canvas starts.  Dimension table: 30 layers,
 *     8 of 128 experts active plus 1 shared, canvas 256, vocabulary ~262K, sliding window 1,024.
 *   - DiffusionGemma model card, Best Practices section 1 (diffusion sampling settings): at most
 *     48 steps; temperature decaying linearly 0.8 -> 0.4 for logit shaping; each step selects the
 *     lowest-entropy tokens while their bound stays under the entropy bound 0.1; unselected tokens
 *     are fully renoised; early stop only when the mean canvas entropy is below 0.005 and the
 *     most likely tokens are unchanged over two consecutive steps.
 *   - diffusers DiffusionGemmaPipeline docs: "Schedulers" (EntropyBoundScheduler, t_max/t_min,
 *     entropy_bound), "Static cache and compilation" (fixed-shape cache, graph replay),
 *     "Adaptive stopping" (per-sample freeze, stability_threshold, confidence_threshold=None
 *     disables), the class text (uniform corruption, no mask token; logits [batch, canvas, vocab]).
 *
 * Conventions for every call:
 *   - Every tensor pointer is DEVICE memory owned by the caller, unless marked "host".  The
 *     library borrows pointers and never frees them; it never allocates device memory.
 *   - bf16 tensors are passed as uint16_t bit patterns (or const void*), row-major, with the
 *     layouts stated below.  Weight matrices are [out_features, in_features].
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are asynchronous on it:
 *     DG_OK means "validated and enqueued".  No call allocates device memory, and no call but
 *     dg_generate (which reads the done flags on the host) synchronises the host, so a decoder
 *     step can be captured in a HIP graph.
 *   - Validation is synchronous and happens before anything is enqueued: on a non-OK status
 *     nothing was enqueued and dg_last_error() describes the problem.  No C++ exception crosses
 *     the ABI.
 *   - A model is immutable after dg_model_create.  Calls with distinct state, workspace and
 *     stream may run concurrently; calls sharing a workspace must be ordered by the caller.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_ERR_NULL = 1,         /* a required pointer is NULL                                     */
  DG_ERR_SHAPE = 2,        /* inconsistent or unsupported dimensions                          */
  DG_ERR_DTYPE = 3,        /* unsupported weight dtype                                        */
  DG_ERR_CAPACITY = 4,     /* len[b] + canvas_len > KV capacity                               */
  DG_ERR_WORKSPACE = 5,    /* workspace smaller than the size query returned                  */
  DG_ERR_STATE = 6,        /* step index outside [0, max_steps) or bad sampler parameters     */
  DG_ERR_UNSUPPORTED = 7,  /* valid request the library does not implement                   */
  DG_ERR_HIP = 8,          /* a HIP runtime call failed                                        */
  DG_ERR_NONFINITE = 9     /* written to *dev_status when a logit row is not finite           */
} dg_status;

/* Weight dtypes.  DG_FP8_E4M3 is the fp8 configuration: the model card quotes its speed on H100
 * in FP8 without a scheme, so this library reads it as OCP e4m3 (bias 7, max 448, no infinities)
 * for the routed and shared expert matrices and the LM head, each row (output channel) with an
 * fp32 scale amax / 448, and their inputs quantised the same way per token row at run time
 * (nearest even, saturating, decided in binary32); fp32 accumulation; output = accumulator *
 * input scale * weight scale.  Attention, router, norms and embedding stay bf16. */
enum { DG_BF16 = 0, DG_FP8_E4M3 = 1 };

/* Model dimensions.  d_model, ffn_inner, shared_inner, (Hq + 2 Hkv) head_dim and Hq head_dim must
 * be multiples of 32 (d_model, ffn_inner, shared_inner multiples of 64 with DG_FP8_E4M3);
 * d_model <= 8192 (a token row is held in the registers of one workgroup);
 * head_dim one of 16, 32, 64, 128, 256;
 * n_q_heads a multiple of n_kv_heads; 1 <= top_k <= n_experts <= 256; vocab a multiple of 256;
 * 1 <= canvas_len <= 1024; window == 0 (every layer global) or window >= canvas_len. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, ffn_inner, shared_inner, vocab, canvas_len;
  int32_t window;        /* sliding window in tokens; 0 = every layer global                  */
  int32_t global_every;  /* layer l is global iff window == 0 || (l + 1) % global_every == 0   */
  int32_t wdtype;        /* DG_BF16 or DG_FP8_E4M3 (expert and LM-head matrices)              */
  float norm_eps;        /* RMSNorm epsilon (1e-6)                                            */
} dg_dims;

/* One layer's weights (device).  Shapes with d = d_model, Hq, Hkv, dh, E, F, Fs:
 *   attn_norm, ffn_norm [d]            RMSNorm gains
 *   w_qkv   [(Hq + 2 Hkv) dh, d]       rows: queries, keys, values; head-major     (PACKED)
 *   w_o     [d, Hq dh]                                                           (PACKED)
 *   w_router[E, d]
 *   w_gate_up [E][2F][d]               per expert: F gate rows, then F up rows      (PACKED)
 *   w_down    [E][d][F]                                                             (PACKED)
 *   ws_gate_up[2Fs][d], ws_down [d][Fs]  the shared expert                          (PACKED)
 * PACKED matrices are stored fragment-major, as dg_pack_weight writes them: they are streamed
 * from HBM once per step, and this layout makes every wave load one contiguous KiB.
 * All other matrices are plain row-major [out, in], bf16.
 * With DG_FP8_E4M3 the four expert matrices hold e4m3 codes packed by dg_pack_weight_fp8, and
 * s_gate_up [E][2F], s_down [E][d], ss_gate_up [2Fs], ss_down [d] are their fp32 row scales
 * (dg_quantize_rows_fp8); with DG_BF16 the scale pointers are ignored. */
typedef struct {
  const void *attn_norm, *w_qkv, *w_o, *ffn_norm, *w_router;
  const void *w_gate_up, *w_down, *ws_gate_up, *ws_down;
  const float *s_gate_up, *s_down, *ss_gate_up, *ss_down;
} dg_layer_w;

typedef struct dg_model dg_model;

/* Build a model handle that BORROWS every pointer until dg_model_destroy.  The encoder and the
 * decoder share these weights (diffusers docs, "PEFT adapters": base weights are tied).
 * layers: host array [n_layers]; embed [V, d] row-major bf16; final_norm [d]; w_lm [V, d] PACKED
 * (so w_lm cannot alias embed): bf16, or e4m3 codes with row scales s_lm [V] for DG_FP8_E4M3
 * (s_lm is ignored for DG_BF16). */
dg_status dg_model_create(const dg_dims* dims, const dg_layer_w* layers, const void* embed,
                          const void* final_norm, const void* w_lm, const float* s_lm,
                          dg_model** out);
void dg_model_destroy(dg_model* model);

/* Static KV cache (diffusers docs, "Static cache and compilation").
 * k, v: [n_layers][batch][Hkv][cap][dh] device rows; len: HOST array [batch] of valid lengths.
 * dtype DG_BF16 (0, the default of a zero-filled struct): k, v hold bf16 and the scale pointers
 * are ignored.  dtype DG_FP8_E4M3 (the FP8 configuration the model card quotes its speed in,
 * read here for the cache too; head_dim 128 or 256 only): k, v hold one e4m3 code (byte) per
 * element and k_scale, v_scale [n_layers][batch][Hkv][cap] the fp32 scale of each row (one
 * token, one KV head), so a row reads as codes * scale.  Every canvas query, key and value row
 * is quantised the same way (scale amax / 448, codes nearest-even with saturation, decided in
 * binary32) before the attention, and an encoder pass stores its quantised key and value rows.
 * All pointers are borrowed; the library never allocates or frees them. */
typedef struct {
  void *k, *v;
  int32_t batch, cap;
  int32_t* len;
  int32_t dtype;            /* DG_BF16 or DG_FP8_E4M3                                         */
  float *k_scale, *v_scale; /* DG_FP8_E4M3: row scales (device); ignored for DG_BF16          */
} dg_kv;

/* Sampler constants; defaults are the model card's (Best Practices section 1). */
typedef struct {
  int32_t max_steps;      /* 48                                                               */
  double t_max, t_min;    /* 0.8 -> 0.4, linear over steps 0 .. max_steps-1                   */
  double entropy_bound;   /* 0.1: summed entropy of the positions committed in one step       */
  double stop_entropy;    /* 0.005: stop when mean entropy < this; negative disables the stop */
  int32_t stability;      /* 1: argmax unchanged over two consecutive steps                   */
  uint64_t seed;          /* Philox4x32-10 key                                                */
} dg_eb_params;

/* Per-canvas sampler state (device, caller-owned, carried across calls).  Shapes [B, C] or [B]. */
typedef struct {
  int32_t* canvas;        /* [B, C] token ids, in/out                                         */
  uint8_t* committed;     /* [B, C] 1 = committed (kept)                                      */
  int32_t* prev_argmax;   /* [B, C] argmax of the previous step                               */
  int32_t* stable_count;  /* [B] consecutive steps with an unchanged argmax                    */
  int32_t* done;          /* [B] 1 = frozen; later calls never modify this canvas              */
  const uint32_t* canvas_id; /* [B] Philox stream id of each canvas (< 2^31)                  */
  int32_t* dev_status;    /* [1] sticky; set to DG_ERR_NONFINITE on a non-finite logit row    */
} dg_eb_state;

/* The pipeline's interchangeable samplers (diffusers DiffusionGemmaPipeline docs, "Schedulers"
 * and "Predictor-corrector sampling"): only the commit / renoise rule changes; the statistics,
 * the adaptive stop (stop_entropy, stability) and the Philox streams are shared.
 *   DG_SCHED_ENTROPY_BOUND: the model card's sampler (t_max, t_min, entropy_bound), as
 *     dg_eb_params describes it.
 *   DG_SCHED_BLOCK_REFINEMENT: at the fixed `temperature` (0 = greedy: the candidate is the
 *     argmax; else a Gumbel-max draw from softmax(logits / temperature)), confidence =
 *     p(candidate) under softmax(logits / T_eff) (T_eff = temperature, or 1 when greedy); each
 *     step commits, among the uncommitted positions, every one with confidence > threshold plus
 *     the step's even share of the canvas, floor((s+1) C / S) - floor(s C / S), of the most
 *     confident others (lower position first on ties); the last step commits everything left;
 *     editing_threshold >= 0 lets a committed position take a different candidate whose
 *     confidence is above it; the rest is renoised uniformly.  top_k (a vocabulary filter of the
 *     draw) must be 0: the filter is not built.
 *   DG_SCHED_DISCRETE_DDIM: uniform (D3PM) corruption with alpha(t) = 1 - t; with
 *     P = max_steps - corrector_steps, call step s < P - 1 draws every position from the exact
 *     posterior sum_m p(m) q(x_{t_{s+1}} | x_{t_s}, x_0 = m), t_s = 1 - s / P; call steps
 *     P - 1 .. max_steps - 2 are leave-one-out corrector sweeps at t = 1 / P, each redrawing the
 *     corrector_k positions of lowest p(current token) from alpha p_loo + (1 - alpha) / V with
 *     p_loo proportional to p(m) / q(current | m); the last call step sets every position to its
 *     argmax and commits the canvas.  Nothing is committed before that.
 * Every scheduler finalises a canvas (uncommitted positions take the argmax) when the adaptive
 * stop holds: argmax unchanged over stability + 1 consecutive steps and mean entropy of
 * softmax(logits / T) below stop_entropy (T = T_s for the entropy bound, T_eff otherwise). */
enum { DG_SCHED_ENTROPY_BOUND = 0, DG_SCHED_BLOCK_REFINEMENT = 1, DG_SCHED_DISCRETE_DDIM = 2 };

typedef struct {
  int32_t kind;               /* DG_SCHED_*                                                    */
  int32_t max_steps;          /* num_inference_steps (48)                                      */
  double t_max, t_min;        /* entropy bound: 0.8 -> 0.4                                     */
  double entropy_bound;       /* entropy bound: 0.1                                            */
  double temperature;         /* block refinement, DDIM: >= 0, 0 = greedy                      */
  double threshold;           /* block refinement: 0.9                                         */
  double editing_threshold;   /* block refinement: < 0 disables editing                        */
  int32_t top_k;              /* block refinement: 0                                           */
  int32_t corrector_steps;    /* DDIM: 0 <= corrector_steps <= max_steps - 1                   */
  int32_t corrector_k;        /* DDIM: positions per corrector sweep, >= 0                     */
  double stop_entropy;        /* 0.005; negative disables the adaptive stop                    */
  int32_t stability;          /* 1                                                             */
  uint64_t seed;              /* Philox4x32-10 key                                             */
} dg_sched_params;

/* Per-step outputs (device, caller-owned). */
typedef struct {
  float* entropy;         /* [B, C] entropy (nats) of softmax(logits / T_s)                   */
  int32_t* argmax;        /* [B, C] argmax of the logits, lowest index on ties                */
  uint8_t* commit_now;    /* [B, C] positions committed by this step (incl. finalised ones)   */
  uint16_t* logits;       /* [B, C, V] bf16 logits (dg_decoder_step writes them)              */
} dg_step_out;

/* Workspace sizes in bytes (0 on invalid arguments). */
size_t dg_workspace_bytes(const dg_model* model, int32_t batch);
size_t dg_eb_workspace_bytes(int32_t batch, int32_t canvas_len, int32_t vocab);

/* Initial canvases (diffusers DiffusionGemmaPipeline docs, class text: the corruption is uniform
 * over the vocabulary and there is no mask token): every position a Philox4x32-10 draw uniform
 * over [0, vocab) from params->seed and the canvas's id, committed = 0, prev_argmax = 0,
 * stable_count = 0, done = 0, dev_status = 0.  batch >= 1, 1 <= canvas_len <= 1024, vocab >= 1.
 * Errors: DG_ERR_NULL (params, state or one of its pointers), DG_ERR_SHAPE (a size out of
 * range). */
dg_status dg_canvas_init(const dg_eb_params* params, dg_eb_state* state, int32_t batch,
                         int32_t canvas_len, int32_t vocab, void* stream);

/* One denoising step at step index `step` (0 <= step < max_steps).  The decoder forward over the
 * canvases (DiffusionGemma model card, "Model overview": bidirectional attention over the canvas
 * joined with cross-attention to the cached context in kv, routed + shared MoE, the LM head),
 * then the entropy-bound sampler update of `state` (model card, Best Practices section 1: the
 * temperature schedule, the lowest-entropy selection under the bound, renoising of the rest and
 * the adaptive stop; diffusers docs, "Schedulers" and "Adaptive stopping").  Writes
 * out->logits/entropy/argmax/commit_now for every canvas that is not frozen; a frozen canvas
 * (state->done) keeps its state.  kv is read only; kv->len[b] + canvas_len <= kv->cap is not
 * required here.  Errors: DG_ERR_NULL, DG_ERR_SHAPE (kv batch outside [1, 64], an fp8 kv at an
 * unsupported head_dim), DG_ERR_CAPACITY (kv->len[b] outside [0, cap]), DG_ERR_STATE (step or
 * params out of range), DG_ERR_WORKSPACE (ws_bytes < dg_workspace_bytes(model, kv->batch)). */
dg_status dg_decoder_step(const dg_model* model, const dg_kv* kv, int32_t step,
                          const dg_eb_params* params, dg_eb_state* state, dg_step_out* out,
                          void* ws, size_t ws_bytes, void* stream);

/* The entropy-bound sampler alone (DiffusionGemma model card, Best Practices section 1;
 * diffusers docs, "Schedulers" (EntropyBoundScheduler) and "Adaptive stopping") on given bf16
 * logits [B, C, V] row-major, which the decoder returns (diffusers docs, class text).  The same
 * update as in dg_decoder_step; out->logits is ignored.  vocab a multiple of 256, canvas_len
 * <= 1024.  Errors: DG_ERR_NULL, DG_ERR_SHAPE, DG_ERR_STATE (step or params out of range),
 * DG_ERR_WORKSPACE (ws_bytes < dg_eb_workspace_bytes(batch, canvas_len, vocab)). */
dg_status dg_eb_sample(const uint16_t* logits, int32_t batch, int32_t canvas_len, int32_t vocab,
                       int32_t step, const dg_eb_params* params, dg_eb_state* state,
                       dg_step_out* out, void* ws, size_t ws_bytes, void* stream);

/* dg_eb_sample for callers that cannot allocate or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and results,
 * with the scratch in a fixed device array of dg_eb_sample_noalloc_max_bytes() bytes (8 MiB) that
 * the library holds on each GPU it runs on until the process ends.  The device address of that
 * array is looked up once per device on the first call there (with that device current); the call
 * itself allocates nothing.  Errors: those of dg_eb_sample, and DG_ERR_WORKSPACE when
 * dg_eb_workspace_bytes(B, C, V) exceeds the array (at V = 262,144 that is about 4,600 positions
 * in all, e.g. B = 16 canvases of 256).  Every call on one GPU shares that GPU's array: calls
 * that may overlap on one GPU (different streams, or host threads) race and must be ordered by
 * the caller.  No entry needs clearing between calls: every scratch entry a kernel reads is
 * written earlier in the same call. */
size_t dg_eb_sample_noalloc_max_bytes(void);
dg_status dg_eb_sample_noalloc(const uint16_t* logits, int32_t batch, int32_t canvas_len,
                               int32_t vocab, int32_t step, const dg_eb_params* params,
                               dg_eb_state* state, dg_step_out* out, void* stream);

/* dg_decoder_step and dg_eb_sample with any of the pipeline's schedulers (dg_sched_params).
 * Same layouts, workspaces and errors; DG_ERR_STATE also for an unknown kind, a negative
 * temperature or a corrector_steps outside [0, max_steps - 1], DG_ERR_UNSUPPORTED for
 * top_k != 0.  The state carries the same fields across calls. */
dg_status dg_decoder_step_sched(const dg_model* model, const dg_kv* kv, int32_t step,
                                const dg_sched_params* params, dg_eb_state* state,
                                dg_step_out* out, void* ws, size_t ws_bytes, void* stream);
/* Frozen-canvas compaction (diffusers docs, "Adaptive stopping": each sample of a batch freezes
 * on its own).  dg_decoder_step_sched over only the canvases live[0 .. n_live) of the batch
 * (host array of distinct indices in [0, kv->batch)): their cache rows, state rows and output
 * rows are read and written in place; the other canvases' state and outputs are not touched, and
 * the step does no work for them.  Every live canvas's results are bit-identical to the full
 * step's (the attention key split is chosen for the whole batch).  Workspace as for the full
 * step.  Errors: those of dg_decoder_step_sched; DG_ERR_SHAPE for n_live outside [1, batch] or
 * a repeated or out-of-range index. */
dg_status dg_decoder_step_live(const dg_model* model, const dg_kv* kv, int32_t step,
                               const dg_sched_params* params, dg_eb_state* state,
                               dg_step_out* out, int32_t n_live, const int32_t* live, void* ws,
                               size_t ws_bytes, void* stream);
dg_status dg_sample(const uint16_t* logits, int32_t batch, int32_t canvas_len, int32_t vocab,
                    int32_t step, const dg_sched_params* params, dg_eb_state* state,
                    dg_step_out* out, void* ws, size_t ws_bytes, void* stream);

/* Append of finished canvases (DiffusionGemma model card, "Model overview": a finished canvas is
 * processed by the encoder and appended to the KV cache before the next canvas starts; the
 * encoder and decoder share their weights, diffusers docs, "PEFT adapters").  Encoder pass over
 * tokens [B, C] int32 (causal inside the canvas, sees the cache); every layer writes its
 * keys/values (an fp8 kv: their e4m3 rows and scales) at [len[b], len[b] + C).  On DG_OK the
 * HOST array kv->len is advanced by C immediately (the device writes are enqueued).  Errors:
 * DG_ERR_NULL, DG_ERR_SHAPE, DG_ERR_CAPACITY (len[b] + C > cap), DG_ERR_WORKSPACE
 * (ws_bytes < dg_workspace_bytes(model, kv->batch)). */
dg_status dg_kv_append_canvas(const dg_model* model, dg_kv* kv, const int32_t* tokens,
                              void* ws, size_t ws_bytes, void* stream);

/* Largest token count per canvas of one dg_kv_append_tokens call. */
#define DG_MAX_APPEND_TOKENS 8192

/* Workspace for dg_kv_append_tokens calls of up to max_tokens tokens per canvas
 * (1 <= max_tokens <= DG_MAX_APPEND_TOKENS and batch * max_tokens <= 65,536; else 0).  The size
 * grows with max_tokens, so it also covers every smaller call. */
size_t dg_append_workspace_bytes(const dg_model* model, int32_t batch, int32_t max_tokens);

/* Chunked prefill (DiffusionGemma model card, "Model overview": the encoder works as the prefill
 * stage, processing the prompt autoregressively into the KV cache).  Encoder pass over n_tokens
 * new tokens per canvas, tokens [B, n_tokens] int32 row-major: the same layers as
 * dg_kv_append_canvas, causal among the new tokens, every cached key visible (sliding-window
 * layers: cache position j is visible to new token i iff (len[b] + i) - j < window).  Every layer
 * writes the new tokens' keys/values at [len[b], len[b] + n_tokens).  A prompt split into
 * consecutive calls is encoded as in one causal pass (up to rounding), for any split.
 * Errors: DG_ERR_NULL (model, kv, tokens or ws), DG_ERR_SHAPE (n_tokens outside
 * [1, DG_MAX_APPEND_TOKENS]; n_tokens > window on a windowed model, where the window would also
 * have to cut inside the new tokens; batch * n_tokens > 65,536), DG_ERR_CAPACITY
 * (len[b] + n_tokens > cap), DG_ERR_WORKSPACE (ws_bytes below the size for n_tokens).  On DG_OK
 * the HOST array kv->len advances by n_tokens immediately (the device writes are enqueued). */
dg_status dg_kv_append_tokens(const dg_model* model, dg_kv* kv, const int32_t* tokens,
                              int32_t n_tokens, void* ws, size_t ws_bytes, void* stream);

/* The outer generation loop (diffusers DiffusionGemmaPipeline docs, the __call__ parameters
 * gen_length, num_inference_steps, eos_early_stop, eos_token_id, and "Adaptive stopping";
 * DiffusionGemma model card, "Model overview": a finished canvas is encoded and appended before
 * the next one starts). */
typedef struct {
  int32_t gen_length;       /* tokens per sequence, rounded up to whole canvases (>= 1)       */
  int32_t eos_token_id;     /* < 0: no EOS check                                              */
  int32_t eos_early_stop;   /* nonzero: start no further canvas once every sequence has
                               produced eos_token_id (at any position of a finished canvas)   */
  int32_t compact_frozen;   /* nonzero: once a sample of the batch is frozen (adaptive stop),
                               the canvas's later steps run only the samples still live
                               (dg_decoder_step_live): same tokens, less work               */
} dg_gen_params;

/* Workspace of dg_generate: dg_workspace_bytes(model, batch) + 512 (0 on invalid arguments). */
size_t dg_generate_workspace_bytes(const dg_model* model, int32_t batch);

/* Generates up to n = ceil(gen_length / canvas_len) canvases per sequence on a cache that holds
 * the prompt (see dg_kv_append_tokens).  For canvas c: the initial canvas with canvas ids
 * c * B + b (state->canvas_id is not read), then dg_decoder_step for steps 0, 1, ... until every
 * sample is frozen or max_steps steps ran, then the canvas is copied to
 * tokens[b, c*C : (c+1)*C] and appended with dg_kv_append_canvas.  The EOS check follows each
 * canvas.  tokens: device int32 [B, n * C]; *canvases (host): canvases generated; steps (host,
 * optional, [n]): decoder steps run per canvas.  state and out hold the last canvas's state and
 * step outputs (out->logits is required).  Unlike the step calls, this call synchronises the
 * stream after every step (to read the done flags) and after every canvas with an EOS check;
 * it returns with the last canvas's copy and append enqueued.  kv->len advances by C per
 * canvas.  Errors: those of the calls it makes, checked first where possible: DG_ERR_NULL,
 * DG_ERR_SHAPE (gen_length < 1), DG_ERR_CAPACITY (len + n * C > cap), DG_ERR_WORKSPACE,
 * DG_ERR_STATE, DG_ERR_HIP. */
dg_status dg_generate(const dg_model* model, dg_kv* kv, const dg_gen_params* gen,
                      const dg_eb_params* params, dg_eb_state* state, dg_step_out* out,
                      int32_t* tokens, int32_t* canvases, int32_t* steps, void* ws,
                      size_t ws_bytes, void* stream);

/* dg_generate with any of the pipeline's schedulers (dg_sched_params); dg_generate is this call
 * with the entropy-bound scheduler. */
dg_status dg_generate_sched(const dg_model* model, dg_kv* kv, const dg_gen_params* gen,
                            const dg_sched_params* params, dg_eb_state* state, dg_step_out* out,
                            int32_t* tokens, int32_t* canvases, int32_t* steps, void* ws,
                            size_t ws_bytes, void* stream);

/* Thread-local description of the last non-OK status returned on this thread. */
const char* dg_last_error(void);

/* ---- stage entry points used by the parity tests and the benchmark ------------------------ */

/* One decoder (causal = 0) or encoder (causal = 1) layer on a residual stream h [B*C, d] fp32,
 * updated in place.  Optional trace outputs (NULL to skip): router logits fp32 [B*C, E],
 * top-k ids int32 [B*C, k] (descending logit), gates fp32 [B*C, k]. */
dg_status dg_layer_forward(const dg_model* model, const dg_kv* kv, int32_t layer, int32_t causal,
                           float* h, float* router_logits, int32_t* topk_idx, float* gates,
                           void* ws, size_t ws_bytes, void* stream);

/* One encoder layer over n_tokens new tokens per canvas, exactly as dg_kv_append_tokens runs it
 * (same kernels and launch shapes for the same n_tokens): h [B * n_tokens, d] fp32 is the layer's
 * input residual stream, updated in place; the layer writes the new tokens' keys/values at
 * [len[b], len[b] + n_tokens) of its cache slice (kv->len is not advanced).  Trace outputs as for
 * dg_layer_forward.  ws: at least dg_append_workspace_bytes(model, B, n_tokens).  Errors as for
 * dg_kv_append_tokens, plus DG_ERR_SHAPE for a layer out of range. */
dg_status dg_layer_forward_tokens(const dg_model* model, const dg_kv* kv, int32_t layer,
                                  int32_t n_tokens, float* h, float* router_logits,
                                  int32_t* topk_idx, float* gates, void* ws, size_t ws_bytes,
                                  void* stream);

/* Packs a row-major bf16 matrix [rows][cols] (rows % 16 == 0, cols % 32 == 0; an [E][N][K]
 * expert tensor is passed as rows = E N) into the fragment-major layout the expert kernels
 * read: element (n, k) moves to ((n/16 * cols/32 + k/32) * 64 + (k%32)/8 * 16 + n%16) * 8 + k%8.
 * src and dst are distinct device buffers of rows * cols bf16; asynchronous on `stream`. */
dg_status dg_pack_weight(const void* src, void* dst, int64_t rows, int64_t cols, void* stream);

/* One FFN half-layer (pre-FFN norm, router, routed + shared experts, residual) on h [B*C, d]
 * fp32, updated in place; batch = B.  Trace outputs as for dg_layer_forward. */
dg_status dg_ffn_forward(const dg_model* model, int32_t layer, int32_t batch, float* h,
                         float* router_logits, int32_t* topk_idx, float* gates, void* ws,
                         size_t ws_bytes, void* stream);

/* Final norm and LM head on h [B*C, d] fp32 (read only): writes out->logits (bf16 [B, C, V]),
 * out->entropy (of softmax(logits / T_step), the schedule of params) and out->argmax, exactly as
 * dg_decoder_step computes them; no sampler state is read or written. */
dg_status dg_lm_head_forward(const dg_model* model, int32_t batch, const float* h, int32_t step,
                             const dg_eb_params* params, dg_step_out* out, void* ws,
                             size_t ws_bytes, void* stream);

/* Per-row e4m3 quantisation of a row-major matrix src [rows][cols] (bf16, or fp32 when
 * src_is_f32): scales[r] = max_c |src[r][c]| / 448 in fp32 (1 for an all-zero row) and
 * codes[r][c] = e4m3(src[r][c] / scales[r]), binary32 division, nearest even, saturating.
 * cols % 4 == 0; codes [rows][cols] uint8 and scales [rows] fp32 are device buffers. */
dg_status dg_quantize_rows_fp8(const void* src, int32_t src_is_f32, uint8_t* codes, float* scales,
                               int64_t rows, int64_t cols, void* stream);

/* Packs e4m3 codes [rows][cols] (rows % 16 == 0, cols % 64 == 0) into the fragment-major layout
 * the fp8 expert and LM-head kernels read: element (n, k) moves to
 * ((n/16 * cols/64 + k/64) * 64 + (k%64)/16 * 16 + n%16) * 16 + k%16.  Distinct buffers. */
dg_status dg_pack_weight_fp8(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t cols,
                             void* stream);

/* Plain device copy of n bytes (bandwidth / counter calibration). */
dg_status dg_copy_bytes(void* dst, const void* src, size_t n, void* stream);

/* Measured ceilings for the benchmark's roofline lines (measurement only, not part of the
 * decoding path).
 * dg_bench_read_stream: reads the n bytes at device `src` (n a multiple of 16) and writes the XOR
 *   of all its 32-bit words to the device word `xor_out`; the read rate of a plain stream.  The
 *   per-block XORs pass through a library-owned device array, so calls on one GPU that overlap
 *   in time race (the benchmark issues them on one stream).
 * dg_bench_mfma_loop: dg_bench_mfma_loop_blocks() workgroups of 4 waves, each wave `iters` rounds
 *   of 8 independent 16x16x32 bf16 MFMAs (2 * 16 * 16 * 32 flops each), one float per thread
 *   written to device `out` (blocks * 256 floats); the matrix-core rate the chip sustains.
 * Errors: DG_ERR_NULL for a NULL pointer, DG_ERR_SHAPE for n % 16 != 0 or iters < 1. */
dg_status dg_bench_read_stream(const void* src, size_t n, uint32_t* xor_out, void* stream);
int32_t dg_bench_mfma_loop_blocks(void);
dg_status dg_bench_mfma_loop(int32_t iters, float* out, void* stream);

/* Kernel timing: the library records HIP events around every launch of the kernel classes set
 * in `mask` (bit i = class i; 0 = off) on the call's stream and accumulates their durations.
 * Classes are listed by dg_prof_class_name(i) for i in [0, dg_prof_num_classes()). */
int32_t dg_prof_num_classes(void);
const char* dg_prof_class_name(int32_t cls);
dg_status dg_prof_enable(uint32_t mask);
/* Synchronises the recorded events and returns the total milliseconds and launch count. */
dg_status dg_prof_read(int32_t cls, double* total_ms, int64_t* launches);
dg_status dg_prof_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
