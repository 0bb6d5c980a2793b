"""Thin Python driver over the C ABI: torch owns device memory and streams, libdg.so computes.

Names follow include/dg.h.  Nothing here computes any part of the path; it allocates caller-owned
buffers, fills the C structs and checks statuses.
"""
import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import check, ptr, stream_ptr


def eb_params(max_steps=48, t_max=0.8, t_min=0.4, entropy_bound=0.1, stop_entropy=0.005,
              stability=1, seed=2):
    """Sampler constants; the defaults are the model card's (Best Practices section 1)."""
    return _lib.dg_eb_params(int(max_steps), float(t_max), float(t_min), float(entropy_bound),
                             float(stop_entropy), int(stability), int(seed))


def eb_params_from_dict(p, seed):
    return eb_params(p["max_steps"], p["t_max"], p["t_min"], p["entropy_bound"],
                     p["stop_entropy"], p["stability"], seed)


class SamplerState:
    """Per-canvas sampler state (device tensors), see dg_eb_state."""

    def __init__(self, batch, canvas_len, device="cuda", canvas_ids=None):
        self.B, self.C = batch, canvas_len
        self.canvas = torch.zeros((batch, canvas_len), dtype=torch.int32, device=device)
        self.committed = torch.zeros((batch, canvas_len), dtype=torch.uint8, device=device)
        self.prev_argmax = torch.zeros((batch, canvas_len), dtype=torch.int32, device=device)
        self.stable_count = torch.zeros(batch, dtype=torch.int32, device=device)
        self.done = torch.zeros(batch, dtype=torch.int32, device=device)
        ids = np.arange(batch, dtype=np.int64) if canvas_ids is None else np.asarray(canvas_ids)
        self.canvas_id = torch.tensor(ids.astype(np.int32), dtype=torch.int32, device=device)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=device)

    def struct(self):
        return _lib.dg_eb_state(*(ptr(t) for t in (self.canvas, self.committed, self.prev_argmax,
                                                   self.stable_count, self.done, self.canvas_id,
                                                   self.dev_status)))

    def host(self):
        return dict(canvas=self.canvas.cpu().numpy().astype(np.int64),
                    committed=self.committed.cpu().numpy().astype(bool),
                    prev_argmax=self.prev_argmax.cpu().numpy().astype(np.int64),
                    stable_count=self.stable_count.cpu().numpy().astype(np.int64),
                    done=self.done.cpu().numpy().astype(bool))

    def load_host(self, st):
        self.canvas.copy_(torch.from_numpy(np.asarray(st["canvas"], dtype=np.int32)))
        self.committed.copy_(torch.from_numpy(np.asarray(st["committed"], dtype=np.uint8)))
        self.prev_argmax.copy_(torch.from_numpy(np.asarray(st["prev_argmax"], dtype=np.int32)))
        self.stable_count.copy_(torch.from_numpy(np.asarray(st["stable_count"], dtype=np.int32)))
        self.done.copy_(torch.from_numpy(np.asarray(st["done"], dtype=np.int32)))


class StepOut:
    """Per-step outputs, see dg_step_out."""

    def __init__(self, batch, canvas_len, vocab, device="cuda", with_logits=True):
        self.entropy = torch.zeros((batch, canvas_len), dtype=torch.float32, device=device)
        self.argmax = torch.zeros((batch, canvas_len), dtype=torch.int32, device=device)
        self.commit_now = torch.zeros((batch, canvas_len), dtype=torch.uint8, device=device)
        self.logits = (torch.zeros((batch, canvas_len, vocab), dtype=torch.bfloat16,
                                   device=device) if with_logits else None)

    def struct(self):
        return _lib.dg_step_out(ptr(self.entropy), ptr(self.argmax), ptr(self.commit_now),
                                ptr(self.logits))


def workspace(nbytes, device="cuda"):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def canvas_init(params, state, vocab, stream=None):
    lib = _lib.load()
    st = state.struct()
    check(lib.dg_canvas_init(ctypes.byref(params), ctypes.byref(st), state.B, state.C, vocab,
                             stream_ptr(stream)), "dg_canvas_init")


def eb_sample(logits, step, params, state, out, ws=None, stream=None):
    """Standalone EB sampler on bf16 logits [B, C, V] (device)."""
    lib = _lib.load()
    b, c, v = logits.shape
    need = lib.dg_eb_workspace_bytes(b, c, v)
    if ws is None:
        ws = workspace(need, logits.device)
    st, o = state.struct(), out.struct()
    check(lib.dg_eb_sample(ptr(logits), b, c, v, step, ctypes.byref(params), ctypes.byref(st),
                           ctypes.byref(o), ptr(ws), ws.numel(), stream_ptr(stream)),
          "dg_eb_sample")
    return ws


SCHED_KINDS = {"entropy_bound": _lib.DG_SCHED_ENTROPY_BOUND,
               "block_refinement": _lib.DG_SCHED_BLOCK_REFINEMENT,
               "discrete_ddim": _lib.DG_SCHED_DISCRETE_DDIM}


def sched_params(kind, max_steps=48, seed=2, temperature=0.0, threshold=0.9,
                 editing_threshold=-1.0, top_k=0, corrector_steps=0, corrector_k=0,
                 stop_entropy=0.005, stability=1, t_max=0.8, t_min=0.4, entropy_bound=0.1):
    """Parameters of one of the pipeline's schedulers (dg_sched_params)."""
    return _lib.dg_sched_params(SCHED_KINDS[kind], max_steps, t_max, t_min, entropy_bound,
                                temperature, threshold, editing_threshold, top_k,
                                corrector_steps, corrector_k, stop_entropy, stability, seed)


def sched_params_from_dict(p, seed):
    """dg_sched_params from an oracle-style parameter dict (oracle.schedulers.default_params)."""
    keys = ("max_steps", "temperature", "threshold", "editing_threshold", "corrector_steps",
            "corrector_k", "stop_entropy", "stability")
    return sched_params(p["kind"], seed=seed, **{k: p[k] for k in keys if k in p})


def sample(logits, step, params, state, out, ws=None, stream=None):
    """Any scheduler's step on given bf16 logits [B, C, V] (dg_sample)."""
    lib = _lib.load()
    b, c, v = logits.shape
    need = lib.dg_eb_workspace_bytes(b, c, v)
    if ws is None:
        ws = workspace(need, logits.device)
    st, o = state.struct(), out.struct()
    check(lib.dg_sample(ptr(logits), b, c, v, step, ctypes.byref(params), ctypes.byref(st),
                        ctypes.byref(o), ptr(ws), ws.numel(), stream_ptr(stream)), "dg_sample")
    return ws


def decoder_step_sched(model, kv, step, params, state, out, ws, stream=None):
    lib = _lib.load()
    kvs, st, o = kv.struct(), state.struct(), out.struct()
    check(lib.dg_decoder_step_sched(model.handle, ctypes.byref(kvs), step, ctypes.byref(params),
                                    ctypes.byref(st), ctypes.byref(o), ptr(ws), ws.numel(),
                                    stream_ptr(stream)), "dg_decoder_step_sched")


def eb_sample_noalloc(logits, step, params, state, out, stream=None):
    """The standalone EB sampler with the library's built-in scratch (dg_eb_sample_noalloc)."""
    lib = _lib.load()
    b, c, v = logits.shape
    st, o = state.struct(), out.struct()
    check(lib.dg_eb_sample_noalloc(ptr(logits), b, c, v, step, ctypes.byref(params),
                                   ctypes.byref(st), ctypes.byref(o), stream_ptr(stream)),
          "dg_eb_sample_noalloc")


def dims_struct(d):
    wd = _lib.DG_FP8_E4M3 if d.get("wdtype", "bf16") in ("e4m3", "fp8") else _lib.DG_BF16
    return _lib.dg_dims(d["n_layers"], d["d"], d["hq"], d["hkv"], d["dh"], d["E"], d["top_k"],
                        d["F"], d["Fs"], d["V"], d["C"], d["window"], d["global_every"],
                        wd, d["eps"])


class Model:
    """A dg_model handle over device weights (dict from synth.model_to_device or
    synth.make_model_device).  Keeps the tensors alive for the handle's lifetime."""

    LAYER_KEYS = ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_router", "w_gate_up", "w_down",
                  "ws_gate_up", "ws_down")
    PACKED_KEYS = ("w_qkv", "w_o", "w_gate_up", "w_down", "ws_gate_up", "ws_down")
    FP8_KEYS = ("w_gate_up", "w_down", "ws_gate_up", "ws_down")
    SCALE_KEYS = ("s_gate_up", "s_down", "ss_gate_up", "ss_down")

    def __init__(self, weights, packed=False, wdtype="bf16"):
        """weights: row-major bf16 device tensors; unless ``packed``, the streamed matrices
        are repacked in place into the fragment-major layout.  wdtype "e4m3": the expert and
        LM-head matrices are first quantised per row to e4m3 codes (the bf16 masters are
        released) and their fp32 row scales are kept as s_* entries."""
        lib = _lib.load()
        self.weights = weights
        self.dims = dict(weights["dims"], wdtype=wdtype)
        fp8 = wdtype in ("e4m3", "fp8")
        if weights["w_lm"].data_ptr() == weights["embed"].data_ptr():
            weights["w_lm"] = weights["w_lm"].clone()
        if not packed:
            for lw in weights["layers"]:
                for k in self.PACKED_KEYS:
                    if fp8 and k in self.FP8_KEYS:
                        lw[k], lw[self.SCALE_KEYS[self.FP8_KEYS.index(k)]] = quantize_pack_fp8(lw[k])
                    else:
                        pack_weight_(lw[k])
            if fp8:
                weights["w_lm"], weights["s_lm"] = quantize_pack_fp8(weights["w_lm"])
            else:
                pack_weight_(weights["w_lm"])
        n = self.dims["n_layers"]
        layers = (_lib.dg_layer_w * n)()
        for i, lw in enumerate(weights["layers"]):
            for k in self.LAYER_KEYS:
                want = torch.uint8 if fp8 and k in self.FP8_KEYS else torch.bfloat16
                assert lw[k].dtype == want and lw[k].is_contiguous(), k
                setattr(layers[i], k, lw[k].data_ptr())
            if fp8:
                for k in self.SCALE_KEYS:
                    assert lw[k].dtype == torch.float32 and lw[k].is_contiguous(), k
                    setattr(layers[i], k, lw[k].data_ptr())
        self._dims = dims_struct(self.dims)
        h = ctypes.c_void_p()
        check(lib.dg_model_create(ctypes.byref(self._dims), layers, ptr(weights["embed"]),
                                  ptr(weights["final_norm"]), ptr(weights["w_lm"]),
                                  ptr(weights.get("s_lm")) if fp8 else None,
                                  ctypes.byref(h)), "dg_model_create")
        self.handle = h

    def workspace_bytes(self, batch):
        return _lib.load().dg_workspace_bytes(self.handle, batch)

    def append_workspace_bytes(self, batch, max_tokens):
        return _lib.load().dg_append_workspace_bytes(self.handle, batch, max_tokens)

    def close(self):
        if self.handle:
            _lib.load().dg_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def kv_is_fp8(dims):
    return dims.get("kv_dtype", "bf16") in ("e4m3", "fp8")


class KVCache:
    """Static KV cache [n_layers][B][Hkv][cap][dh] K and V with host lengths: bf16, or (dims
    kv_dtype "e4m3") e4m3 codes (uint8) with fp32 row scales [n_layers][B][Hkv][cap]."""

    def __init__(self, dims, batch, cap, device="cuda", k=None, v=None, lengths=None,
                 k_scale=None, v_scale=None):
        shape = (dims["n_layers"], batch, dims["hkv"], cap, dims["dh"])
        self.fp8 = kv_is_fp8(dims)
        dt = torch.uint8 if self.fp8 else torch.bfloat16
        self.k = k if k is not None else torch.zeros(shape, dtype=dt, device=device)
        self.v = v if v is not None else torch.zeros(shape, dtype=dt, device=device)
        assert tuple(self.k.shape) == shape and tuple(self.v.shape) == shape
        assert self.k.dtype == dt and self.v.dtype == dt
        if self.fp8:
            sshape = shape[:-1]
            self.k_scale = (k_scale if k_scale is not None else
                            torch.ones(sshape, dtype=torch.float32, device=device))
            self.v_scale = (v_scale if v_scale is not None else
                            torch.ones(sshape, dtype=torch.float32, device=device))
            assert tuple(self.k_scale.shape) == sshape and tuple(self.v_scale.shape) == sshape
            assert self.k_scale.dtype == torch.float32 and self.v_scale.dtype == torch.float32
        else:
            self.k_scale = self.v_scale = None
        self.batch, self.cap = batch, cap
        self.len = (ctypes.c_int32 * batch)(*([0] * batch if lengths is None else
                                              [int(x) for x in lengths]))

    @classmethod
    def from_host(cls, dims, cache, cap, device="cuda"):
        if kv_is_fp8(dims):
            k, v = (torch.from_numpy(np.stack(cache[n])).to(device) for n in ("k", "v"))
            ks, vs = (torch.from_numpy(np.stack(cache[n]).astype(np.float32)).to(device)
                      for n in ("k_scale", "v_scale"))
            return cls(dims, k.shape[1], cap, device, k, v, cache["len"], ks, vs)
        k = torch.from_numpy(np.stack(cache["k"])).to(device=device, dtype=torch.bfloat16)
        v = torch.from_numpy(np.stack(cache["v"])).to(device=device, dtype=torch.bfloat16)
        return cls(dims, k.shape[1], cap, device, k, v, cache["len"])

    def struct(self):
        if self.fp8:
            return _lib.dg_kv(ptr(self.k), ptr(self.v), self.batch, self.cap, self.len,
                              _lib.DG_FP8_E4M3, ptr(self.k_scale), ptr(self.v_scale))
        return _lib.dg_kv(ptr(self.k), ptr(self.v), self.batch, self.cap, self.len,
                          _lib.DG_BF16, None, None)

    def lengths(self):
        return [self.len[i] for i in range(self.batch)]


def decoder_step(model, kv, step, params, state, out, ws, stream=None):
    lib = _lib.load()
    kvs, st, o = kv.struct(), state.struct(), out.struct()
    check(lib.dg_decoder_step(model.handle, ctypes.byref(kvs), step, ctypes.byref(params),
                              ctypes.byref(st), ctypes.byref(o), ptr(ws), ws.numel(),
                              stream_ptr(stream)), "dg_decoder_step")


def kv_append_canvas(model, kv, tokens, ws, stream=None):
    lib = _lib.load()
    kvs = kv.struct()
    check(lib.dg_kv_append_canvas(model.handle, ctypes.byref(kvs), ptr(tokens), ptr(ws),
                                  ws.numel(), stream_ptr(stream)), "dg_kv_append_canvas")


def kv_append_tokens(model, kv, tokens, ws, stream=None):
    """Chunked prefill: encoder pass over tokens [B, n] (int32 device), appended to the cache."""
    lib = _lib.load()
    kvs = kv.struct()
    n = int(tokens.shape[1])
    check(lib.dg_kv_append_tokens(model.handle, ctypes.byref(kvs), ptr(tokens), n, ptr(ws),
                                  ws.numel(), stream_ptr(stream)), "dg_kv_append_tokens")


def generate(model, kv, params, state, out, gen_length, eos_token_id=-1, eos_early_stop=True,
             ws=None, stream=None, compact_frozen=False):
    """The canvas loop on a cache that holds the prompt: returns (tokens [B, n*C] int32 device,
    canvases generated, decoder steps per canvas).  params: dg_eb_params (the entropy bound) or
    dg_sched_params (any scheduler, dg_generate_sched)."""
    lib = _lib.load()
    c = state.C
    n = -(-int(gen_length) // c)
    tokens = torch.zeros((state.B, n * c), dtype=torch.int32, device=state.canvas.device)
    if ws is None:
        ws = workspace(lib.dg_generate_workspace_bytes(model.handle, state.B),
                       state.canvas.device)
    gen = _lib.dg_gen_params(int(gen_length), int(eos_token_id), 1 if eos_early_stop else 0,
                             1 if compact_frozen else 0)
    kvs, st, o = kv.struct(), state.struct(), out.struct()
    done = ctypes.c_int32(0)
    steps = (ctypes.c_int32 * n)()
    fn = lib.dg_generate_sched if isinstance(params, _lib.dg_sched_params) else lib.dg_generate
    check(fn(model.handle, ctypes.byref(kvs), ctypes.byref(gen), ctypes.byref(params),
             ctypes.byref(st), ctypes.byref(o), ptr(tokens), ctypes.byref(done),
             ctypes.cast(steps, ctypes.c_void_p), ptr(ws), ws.numel(), stream_ptr(stream)),
          "dg_generate")
    k = done.value
    return tokens[:, :k * c], k, [steps[i] for i in range(k)]


def decoder_step_live(model, kv, step, params, state, out, live, ws, stream=None):
    """dg_decoder_step_live: the step over the canvases in `live` only (dg_sched_params)."""
    lib = _lib.load()
    kvs, st, o = kv.struct(), state.struct(), out.struct()
    arr = (ctypes.c_int32 * len(live))(*[int(x) for x in live])
    check(lib.dg_decoder_step_live(model.handle, ctypes.byref(kvs), step, ctypes.byref(params),
                                   ctypes.byref(st), ctypes.byref(o), len(live), arr, ptr(ws),
                                   ws.numel(), stream_ptr(stream)), "dg_decoder_step_live")


def layer_forward(model, kv, layer, causal, h, ws, router_logits=None, topk_idx=None,
                  gates=None, stream=None):
    lib = _lib.load()
    kvs = kv.struct()
    check(lib.dg_layer_forward(model.handle, ctypes.byref(kvs), layer, int(causal), ptr(h),
                               ptr(router_logits), ptr(topk_idx), ptr(gates), ptr(ws),
                               ws.numel(), stream_ptr(stream)), "dg_layer_forward")


def layer_forward_tokens(model, kv, layer, h, ws, router_logits=None, topk_idx=None, gates=None,
                         stream=None):
    """One encoder layer over n = h.shape[0] / B new tokens per canvas (dg_layer_forward_tokens)."""
    lib = _lib.load()
    kvs = kv.struct()
    n = h.shape[0] // kv.batch
    check(lib.dg_layer_forward_tokens(model.handle, ctypes.byref(kvs), layer, n, ptr(h),
                                      ptr(router_logits), ptr(topk_idx), ptr(gates), ptr(ws),
                                      ws.numel(), stream_ptr(stream)), "dg_layer_forward_tokens")


def pack_weight(src, dst, stream=None):
    """dst <- fragment-major layout of the bf16 matrix src ([..., N, K] viewed as [rows, K])."""
    cols = src.shape[-1]
    rows = src.numel() // cols
    check(_lib.load().dg_pack_weight(ptr(src), ptr(dst), rows, cols, stream_ptr(stream)),
          "dg_pack_weight")


def pack_weight_(w, stream=None):
    """In-place repack of a bf16 device matrix into the fragment-major layout."""
    tmp = torch.empty_like(w)
    pack_weight(w, tmp, stream)
    w.copy_(tmp)


def ffn_forward(model, layer, batch, h, ws, router_logits=None, topk_idx=None, gates=None,
                stream=None):
    check(_lib.load().dg_ffn_forward(model.handle, layer, batch, ptr(h), ptr(router_logits),
                                     ptr(topk_idx), ptr(gates), ptr(ws), ws.numel(),
                                     stream_ptr(stream)), "dg_ffn_forward")


def lm_head_forward(model, batch, h, step, params, out, ws, stream=None):
    o = out.struct()
    check(_lib.load().dg_lm_head_forward(model.handle, batch, ptr(h), step, ctypes.byref(params),
                                         ctypes.byref(o), ptr(ws), ws.numel(), stream_ptr(stream)),
          "dg_lm_head_forward")


def quantize_rows_fp8(src, codes, scales, stream=None):
    """e4m3 codes [rows, cols] (uint8) and fp32 row scales of a bf16 or fp32 matrix."""
    cols = src.shape[-1]
    rows = src.numel() // cols
    assert src.dtype in (torch.bfloat16, torch.float32) and src.is_contiguous()
    check(_lib.load().dg_quantize_rows_fp8(ptr(src), int(src.dtype == torch.float32), ptr(codes),
                                           ptr(scales), rows, cols, stream_ptr(stream)),
          "dg_quantize_rows_fp8")


def pack_weight_fp8(src, dst, stream=None):
    cols = src.shape[-1]
    rows = src.numel() // cols
    check(_lib.load().dg_pack_weight_fp8(ptr(src), ptr(dst), rows, cols, stream_ptr(stream)),
          "dg_pack_weight_fp8")


def quantize_pack_fp8(w, stream=None):
    """(packed e4m3 codes with w's shape, fp32 row scales) of a bf16 matrix [..., N, K]."""
    cols = w.shape[-1]
    rows = w.numel() // cols
    codes = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    scales = torch.empty(rows, dtype=torch.float32, device=w.device)
    quantize_rows_fp8(w, codes, scales, stream)
    packed = torch.empty_like(codes)
    pack_weight_fp8(codes, packed, stream)
    del codes
    return packed, scales


def copy_bytes(dst, src, nbytes, stream=None):
    check(_lib.load().dg_copy_bytes(ptr(dst), ptr(src), nbytes, stream_ptr(stream)),
          "dg_copy_bytes")


def read_stream(src, nbytes, xor_out, stream=None):
    """XOR of the 32-bit words of the first nbytes of src into the one-word tensor xor_out."""
    check(_lib.load().dg_bench_read_stream(ptr(src), nbytes, ptr(xor_out), stream_ptr(stream)),
          "dg_bench_read_stream")


def mfma_loop_blocks():
    return _lib.load().dg_bench_mfma_loop_blocks()


def mfma_loop(iters, out, stream=None):
    """The bf16 MFMA loop: out holds mfma_loop_blocks() * 256 floats."""
    check(_lib.load().dg_bench_mfma_loop(iters, ptr(out), stream_ptr(stream)),
          "dg_bench_mfma_loop")


class KernelTimer:
    """HIP-event timing of library kernel classes (dg_prof_*)."""

    def __init__(self):
        self.lib = _lib.load()
        n = self.lib.dg_prof_num_classes()
        self.names = [self.lib.dg_prof_class_name(i).decode() for i in range(n)]

    def enable(self, names=None):
        """Time the named kernel classes (all when None; [] turns timing off)."""
        names = self.names if names is None else names
        mask = 0
        for n in names:
            mask |= 1 << self.names.index(n)
        check(self.lib.dg_prof_enable(mask), "dg_prof_enable")

    def reset(self):
        check(self.lib.dg_prof_reset(), "dg_prof_reset")

    def read(self, name):
        ms = ctypes.c_double()
        cnt = ctypes.c_int64()
        check(self.lib.dg_prof_read(self.names.index(name), ctypes.byref(ms), ctypes.byref(cnt)),
              "dg_prof_read")
        return ms.value, cnt.value
