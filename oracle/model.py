"""Decoder step and encoder append of the block-diffusion model, written plainly in fp64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix:
  * an encoder-decoder whose encoder and decoder share one set of weights (diffusers
    DiffusionGemmaPipeline docs, "PEFT adapters" and the ``model`` parameter);
  * a causal encoder prefills the prompt into a KV cache and later reads every finished canvas,
    whose keys and values are appended to that cache; the decoder denoises the canvas with
    bidirectional attention over the canvas and cross-attention to the cached context
    (DiffusionGemma model card, "Model overview"; diffusers docs, introduction);
  * 30 layers, a sparse MoE with 8 of 128 experts active plus 1 shared expert, a ~262K
    vocabulary, a 256-token canvas and a 1,024-token sliding window (model card dimension table);
  * the model returns logits [batch, canvas_length, vocab_size] (diffusers docs, class text).

Readings (the pages give no layer internals, so each of these is a reading):
  * pre-norm RMSNorm before attention, before the FFN and before the LM head, with a gain
    vector and eps = 1e-6; the embedding is a row gather with no scale;
  * attention: one joint softmax per query over the visible cache keys and the canvas keys,
    scale 1/sqrt(head_dim), no positional encoding, no soft-cap; query head h reads KV head
    floor(h * Hkv / Hq); the decoder sees every canvas key, the encoder canvas key j <= i;
    a sliding-window layer lets canvas query i (absolute position len + i) see cache position j
    only if (len + i) - j < window;  layer l is global iff window == 0 or
    (l + 1) % global_every == 0;
  * MoE: router logits r = u W_r^T, softmax over the experts, the top-k by logit (lowest index
    on ties, listed in descending order), gates = softmax weights renormalised over the top-k;
    the shared expert is added with weight 1; every FFN is SwiGLU:
    (silu(u W_gate^T) * (u W_up^T)) W_down^T, where the gate rows come first in W_gate_up;
  * the QKV projection is one [(Hq + 2 Hkv) * dh, d] matrix: queries, then keys, then values,
    head-major inside each part;
  * the appended keys and values are those each layer computes from its normed input for the
    canvas positions; they are stored in bf16, the cache's storage type.

Weights arrive as float64 arrays holding the bf16 (storage) values; activations are not rounded,
except the logits (rounded to bf16 before the sampler reads them) and the stored cache entries.
"""
import numpy as np

from .numerics import quantize_rows_e4m3, round_bf16


def rms_norm(x, gain, eps):
    """x / sqrt(mean(x^2) + eps) * gain along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gain


def silu(x):
    return x / (1.0 + np.exp(-x))


def softmax(x, axis=-1):
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def layer_is_global(layer, dims):
    return dims["window"] == 0 or (layer + 1) % dims["global_every"] == 0


def visible_cache_mask(cache_len, canvas_len, window):
    """[C, cache_len] bool: may canvas query i see cache position j (sliding-window rule)."""
    i = np.arange(canvas_len)[:, None]
    j = np.arange(cache_len)[None, :]
    if window <= 0:
        return np.ones((canvas_len, cache_len), dtype=bool)
    return (cache_len + i) - j < window


def attention(q, k_cache, v_cache, k_new, v_new, cache_mask, causal, q_pos=None):
    """Joint softmax attention for one canvas.

    q [R, Hq, dh] for the canvas positions q_pos (default: all C positions, R = C);
    k_cache, v_cache [Hkv, L, dh]; k_new, v_new [C, Hkv, dh]; cache_mask [R, L] bool;
    causal: canvas query i sees canvas key j only if j <= i.  Returns [R, Hq, dh].
    """
    rows, hq, dh = q.shape
    clen = k_new.shape[0]
    hkv = k_new.shape[1]
    q_pos = np.arange(clen) if q_pos is None else np.asarray(q_pos)
    out = np.zeros_like(q)
    j = np.arange(clen)[None, :]
    canvas_mask = (j <= q_pos[:, None]) if causal else np.ones((rows, clen), dtype=bool)
    mask = np.concatenate([cache_mask, canvas_mask], axis=1)          # [R, L + C]
    for h in range(hq):
        g = (h * hkv) // hq
        keys = np.concatenate([k_cache[g], k_new[:, g, :]], axis=0)   # [L + C, dh]
        vals = np.concatenate([v_cache[g], v_new[:, g, :]], axis=0)
        s = q[:, h, :] @ keys.T / np.sqrt(dh)
        s = np.where(mask, s, -np.inf)
        out[:, h, :] = softmax(s, axis=-1) @ vals
    return out


def fp8_linear(x, w_q, s_w):
    """x W^T with e4m3 weights (fp8 configuration): each row of x is quantised to e4m3 with its
    own scale (numerics.quantize_rows_e4m3); the e4m3 products and their sums are exact in fp64;
    the sum is multiplied by the row's input scale and the output channel's weight scale.
    w_q [N, K] e4m3 values (float64), s_w [N]."""
    q, s = quantize_rows_e4m3(x)
    return (q @ w_q.T) * s[..., None] * np.asarray(s_w, dtype=np.float64)


def linear(x, w, s_w=None):
    """x W^T; with a weight scale vector the weights are e4m3 and the product is fp8_linear."""
    return x @ w.T if s_w is None else fp8_linear(x, w, s_w)


def swiglu_ffn(u, w_gate_up, w_down, s_gate_up=None, s_down=None):
    """(silu(u Wg^T) * (u Wu^T)) Wd^T with Wg = first half of the rows of w_gate_up (with scales:
    both products in fp8, the SwiGLU output quantised per row before the down product)."""
    f = w_gate_up.shape[0] // 2
    gu = linear(u, w_gate_up, s_gate_up)
    return linear(silu(gu[..., :f]) * gu[..., f:], w_down, s_down)


def route(u, w_router, top_k, force_idx=None):
    """Router: logits, top-k expert ids (descending logit, lowest id on ties) and gates.

    force_idx [T, k]: use these expert ids instead of the top-k (gates are still the softmax
    weights renormalised over the chosen experts).  The parity tests pass the GPU's choice here
    for rows whose k-th and (k+1)-th logits are a near-tie, where either choice is correct."""
    r = u @ w_router.T                                                # [T, E]
    pi = softmax(r, axis=-1)
    ntok, n_exp = r.shape
    idx = np.zeros((ntok, top_k), dtype=np.int64)
    for t in range(ntok):
        order = sorted(range(n_exp), key=lambda e: (-r[t, e], e))
        idx[t] = order[:top_k]
    if force_idx is not None:
        idx = np.asarray(force_idx, dtype=np.int64).reshape(ntok, top_k).copy()
    sel = np.take_along_axis(pi, idx, axis=1)
    gates = sel / sel.sum(axis=1, keepdims=True)
    return r, idx, gates


def moe(u, lw, top_k, force_idx=None):
    """Sparse MoE FFN: sum over the top-k experts of gate * FFN_e(u), plus the shared expert
    (force_idx: see ``route``)."""
    r, idx, gates = route(u, lw["w_router"], top_k, force_idx)
    ntok, d = u.shape
    n_exp = lw["w_router"].shape[0]
    y = np.zeros((ntok, top_k, d))
    fp8 = "s_gate_up" in lw
    for e in range(n_exp):
        t_list, j_list = np.nonzero(idx == e)
        if t_list.size:
            y[t_list, j_list] = swiglu_ffn(u[t_list], lw["w_gate_up"][e], lw["w_down"][e],
                                           lw["s_gate_up"][e] if fp8 else None,
                                           lw["s_down"][e] if fp8 else None)
    out = swiglu_ffn(u, lw["ws_gate_up"], lw["ws_down"], lw.get("ss_gate_up"), lw.get("ss_down"))
    for j in range(top_k):
        out = out + gates[:, j:j + 1] * y[:, j]
    return out, dict(router_logits=r, topk_idx=idx, gates=gates)


def split_qkv(qkv, dims):
    hq, hkv, dh = dims["hq"], dims["hkv"], dims["dh"]
    q = qkv[..., :hq * dh].reshape(qkv.shape[:-1] + (hq, dh))
    k = qkv[..., hq * dh:(hq + hkv) * dh].reshape(qkv.shape[:-1] + (hkv, dh))
    v = qkv[..., (hq + hkv) * dh:].reshape(qkv.shape[:-1] + (hkv, dh))
    return q, k, v


def kv_fp8(dims):
    """Is the KV cache of this model stored in e4m3 (the fp8 KV configuration)?"""
    return dims.get("kv_dtype", "bf16") in ("e4m3", "fp8")


def quantize_dequantize_rows(x):
    """x as its per-row e4m3 codes times the row scale (numerics.quantize_rows_e4m3 along the
    last axis), as float64: the value an e4m3 row with an fp32 scale represents."""
    q, s = quantize_rows_e4m3(x)
    return q * s[..., None]


def attention_block(h, lw, dims, layer, k_cache, v_cache, cache_len, causal, rows=None):
    """First half of a layer: h + O-projection of the joint attention over RMSNorm(h).

    h [B, C, d]; k_cache, v_cache [B, Hkv, cap, dh] (this layer); cache_len [B].
    Returns (h after attention, k [B, C, Hkv, dh], v) -- k, v are the canvas keys/values.
    rows: only these canvas positions' outputs (h after attention is then [B, len(rows), d]);
    every position still makes its key and value, and a query's output depends on its own row
    and the keys and values only.

    fp8 KV configuration (reading; the pages only quote FP8 speed): the normed input and the QKV
    product are taken in their bf16 storage forms, and every query, key and value row of dh
    values (one token, one head) is replaced by its per-row e4m3 quantisation (codes times fp32
    scale) before the attention; the cache holds such rows.  The returned k, v are the quantised
    canvas rows."""
    eps = dims["eps"]
    bsz, clen, d = h.shape
    u = rms_norm(h, lw["attn_norm"], eps)
    if kv_fp8(dims):
        u = round_bf16(u)
    qkv = u @ lw["w_qkv"].T
    if kv_fp8(dims):
        qkv = round_bf16(qkv)
    q, k, v = split_qkv(qkv, dims)
    if kv_fp8(dims):
        q, k, v = (quantize_dequantize_rows(x) for x in (q, k, v))
    window = 0 if layer_is_global(layer, dims) else dims["window"]
    rows = np.arange(clen) if rows is None else np.asarray(rows)
    o = np.zeros((bsz, rows.shape[0]) + q.shape[2:])
    for b in range(bsz):
        n = int(cache_len[b])
        mask = visible_cache_mask(n, clen, window)[rows]
        o[b] = attention(q[b, rows], k_cache[b, :, :n], v_cache[b, :, :n], k[b], v[b], mask,
                         causal, q_pos=rows)
    return h[:, rows] + o.reshape(bsz, rows.shape[0], -1) @ lw["w_o"].T, k, v


def ffn_block(h, lw, dims, force_idx=None):
    """Second half of a layer: h + MoE(RMSNorm(h)).  Returns (new h, routing info).
    force_idx [B, C, k] or None (see ``route``)."""
    bsz, clen, d = h.shape
    u = rms_norm(h, lw["ffn_norm"], dims["eps"])
    f, info = moe(u.reshape(bsz * clen, d), lw, dims["top_k"], force_idx)
    return h + f.reshape(bsz, clen, d), info


def layer_forward(h, lw, dims, layer, k_cache, v_cache, cache_len, causal, force_idx=None):
    """One transformer layer over a batch of canvases.

    h [B, C, d] residual stream; k_cache, v_cache [B, Hkv, cap, dh] (this layer);
    cache_len [B]; force_idx [B, C, k] or None (see ``route``).
    Returns (new h, k [B, C, Hkv, dh], v, routing info).
    """
    h, k, v = attention_block(h, lw, dims, layer, k_cache, v_cache, cache_len, causal)
    h, info = ffn_block(h, lw, dims, force_idx)
    return h, k, v, info


def decoder_forward(canvas, model, cache, force_idx=None):
    """Decoder pass over canvases [B, C] -> logits [B, C, V] (bf16-rounded, as float64).

    cache: dict(k, v: lists over layers of [B, Hkv, cap, dh], len [B]).
    force_idx: None, or a list over layers of [B, C, k] expert ids (see ``route``).
    Also returns the fp64 logits before rounding and per-layer routing info.
    """
    dims = model["dims"]
    h = model["embed"][np.asarray(canvas)]
    infos = []
    for layer, lw in enumerate(model["layers"]):
        fi = None if force_idx is None else force_idx[layer]
        h, _, _, info = layer_forward(h, lw, dims, layer, cache["k"][layer], cache["v"][layer],
                                      cache["len"], causal=False, force_idx=fi)
        infos.append(info)
    z = linear(rms_norm(h, model["final_norm"], dims["eps"]), model["w_lm"], model.get("s_lm"))
    return round_bf16(z), z, infos


def encoder_append(tokens, model, cache, round_stored=True, force_idx=None):
    """Encoder pass over finished canvases [B, C]: causal inside the canvas, sees the cache.

    Each layer stores its keys and values at [len, len + C), rounded to bf16 (the cache's storage
    type) unless ``round_stored`` is False; len += C.  The cache dict is updated in place.
    force_idx: None, or a list over layers of [B, C, k] expert ids (see ``route``).
    """
    dims = model["dims"]
    tokens = np.asarray(tokens)
    bsz, clen = tokens.shape
    h = model["embed"][tokens]
    for layer, lw in enumerate(model["layers"]):
        kc, vc = cache["k"][layer], cache["v"][layer]
        if np.any(cache["len"] + clen > kc.shape[2]):
            raise ValueError("cache capacity exceeded")
        fi = None if force_idx is None else force_idx[layer]
        h, k, v, _ = layer_forward(h, lw, dims, layer, kc, vc, cache["len"], causal=True,
                                   force_idx=fi)
        for b in range(bsz):
            n = int(cache["len"][b])
            # the layer's k, v are already e4m3 rows in the fp8 KV configuration (exact)
            store = round_bf16 if round_stored and not kv_fp8(dims) else np.asarray
            kc[b, :, n:n + clen] = store(k[b].transpose(1, 0, 2))
            vc[b, :, n:n + clen] = store(v[b].transpose(1, 0, 2))
    cache["len"] = cache["len"] + clen
    return cache


def quantize_model_e4m3(model):
    """The fp8 configuration of a model: the routed and shared expert matrices and the LM head
    are quantised per output channel (row) with numerics.quantize_rows_e4m3, keeping their scales
    (s_gate_up [E, 2F], s_down [E, d], ss_gate_up [2Fs], ss_down [d], s_lm [V]); attention, router,
    norms and embedding stay in bf16.  Returns a new model dict (float64 arrays)."""
    out = dict(dims=dict(model["dims"], wdtype="e4m3"), layers=[])
    for lw in model["layers"]:
        out["layers"].append(quantize_layer_e4m3(lw))
    for key in ("embed", "final_norm"):
        out[key] = model[key]
    out["w_lm"], out["s_lm"] = quantize_rows_e4m3(model["w_lm"])
    return out


def quantize_layer_e4m3(lw):
    """One layer of the fp8 configuration (see quantize_model_e4m3)."""
    q = dict(lw)
    for key, skey in (("w_gate_up", "s_gate_up"), ("w_down", "s_down"),
                      ("ws_gate_up", "ss_gate_up"), ("ws_down", "ss_down")):
        q[key], q[skey] = quantize_rows_e4m3(lw[key])
    return q
