"""ctypes binding of libdg.so (include/dg.h): argument marshalling only.

Every compute step runs in the library's HIP kernels; this module only mirrors the C structs,
declares the entry points with the same names, and turns torch tensors into raw pointers.
Loading fails loudly when the library has not been built.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdg.so")

DG_OK = 0
STATUS_NAMES = ["DG_OK", "DG_ERR_NULL", "DG_ERR_SHAPE", "DG_ERR_DTYPE", "DG_ERR_CAPACITY",
                "DG_ERR_WORKSPACE", "DG_ERR_STATE", "DG_ERR_UNSUPPORTED", "DG_ERR_HIP",
                "DG_ERR_NONFINITE"]
DG_BF16 = 0
DG_FP8_E4M3 = 1

c_void_p = ctypes.c_void_p
i32 = ctypes.c_int32


class dg_dims(ctypes.Structure):
    _fields_ = [("n_layers", i32), ("d_model", i32), ("n_q_heads", i32), ("n_kv_heads", i32),
                ("head_dim", i32), ("n_experts", i32), ("top_k", i32), ("ffn_inner", i32),
                ("shared_inner", i32), ("vocab", i32), ("canvas_len", i32), ("window", i32),
                ("global_every", i32), ("wdtype", i32), ("norm_eps", ctypes.c_float)]


class dg_layer_w(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_router",
                                        "w_gate_up", "w_down", "ws_gate_up", "ws_down",
                                        "s_gate_up", "s_down", "ss_gate_up", "ss_down")]


class dg_kv(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("batch", i32), ("cap", i32),
                ("len", ctypes.POINTER(i32)), ("dtype", i32), ("k_scale", c_void_p),
                ("v_scale", c_void_p)]


class dg_eb_params(ctypes.Structure):
    _fields_ = [("max_steps", i32), ("t_max", ctypes.c_double), ("t_min", ctypes.c_double),
                ("entropy_bound", ctypes.c_double), ("stop_entropy", ctypes.c_double),
                ("stability", i32), ("seed", ctypes.c_uint64)]


DG_SCHED_ENTROPY_BOUND = 0
DG_SCHED_BLOCK_REFINEMENT = 1
DG_SCHED_DISCRETE_DDIM = 2


class dg_sched_params(ctypes.Structure):
    _fields_ = [("kind", i32), ("max_steps", i32), ("t_max", ctypes.c_double),
                ("t_min", ctypes.c_double), ("entropy_bound", ctypes.c_double),
                ("temperature", ctypes.c_double), ("threshold", ctypes.c_double),
                ("editing_threshold", ctypes.c_double), ("top_k", i32),
                ("corrector_steps", i32), ("corrector_k", i32),
                ("stop_entropy", ctypes.c_double), ("stability", i32),
                ("seed", ctypes.c_uint64)]


class dg_eb_state(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("canvas", "committed", "prev_argmax", "stable_count",
                                        "done", "canvas_id", "dev_status")]


class dg_step_out(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("entropy", "argmax", "commit_now", "logits")]


class dg_gen_params(ctypes.Structure):
    _fields_ = [("gen_length", i32), ("eos_token_id", i32), ("eos_early_stop", i32),
                ("compact_frozen", i32)]


P = ctypes.POINTER
_SIGS = {
    "dg_last_error": (ctypes.c_char_p, []),
    "dg_model_create": (i32, [P(dg_dims), P(dg_layer_w), c_void_p, c_void_p, c_void_p,
                              c_void_p, P(c_void_p)]),
    "dg_model_destroy": (None, [c_void_p]),
    "dg_workspace_bytes": (ctypes.c_size_t, [c_void_p, i32]),
    "dg_eb_workspace_bytes": (ctypes.c_size_t, [i32, i32, i32]),
    "dg_canvas_init": (i32, [P(dg_eb_params), P(dg_eb_state), i32, i32, i32, c_void_p]),
    "dg_decoder_step": (i32, [c_void_p, P(dg_kv), i32, P(dg_eb_params), P(dg_eb_state),
                              P(dg_step_out), c_void_p, ctypes.c_size_t, c_void_p]),
    "dg_eb_sample": (i32, [c_void_p, i32, i32, i32, i32, P(dg_eb_params), P(dg_eb_state),
                           P(dg_step_out), c_void_p, ctypes.c_size_t, c_void_p]),
    "dg_sample": (i32, [c_void_p, i32, i32, i32, i32, P(dg_sched_params), P(dg_eb_state),
                        P(dg_step_out), c_void_p, ctypes.c_size_t, c_void_p]),
    "dg_decoder_step_sched": (i32, [c_void_p, P(dg_kv), i32, P(dg_sched_params), P(dg_eb_state),
                                    P(dg_step_out), c_void_p, ctypes.c_size_t, c_void_p]),
    "dg_decoder_step_live": (i32, [c_void_p, P(dg_kv), i32, P(dg_sched_params), P(dg_eb_state),
                                   P(dg_step_out), i32, P(i32), c_void_p, ctypes.c_size_t,
                                   c_void_p]),
    "dg_generate_sched": (i32, [c_void_p, P(dg_kv), P(dg_gen_params), P(dg_sched_params),
                                P(dg_eb_state), P(dg_step_out), c_void_p, P(i32), c_void_p,
                                c_void_p, ctypes.c_size_t, c_void_p]),
    "dg_eb_sample_noalloc_max_bytes": (ctypes.c_size_t, []),
    "dg_eb_sample_noalloc": (i32, [c_void_p, i32, i32, i32, i32, P(dg_eb_params), P(dg_eb_state),
                                   P(dg_step_out), c_void_p]),
    "dg_kv_append_canvas": (i32, [c_void_p, P(dg_kv), c_void_p, c_void_p, ctypes.c_size_t,
                                  c_void_p]),
    "dg_append_workspace_bytes": (ctypes.c_size_t, [c_void_p, i32, i32]),
    "dg_generate_workspace_bytes": (ctypes.c_size_t, [c_void_p, i32]),
    "dg_generate": (i32, [c_void_p, P(dg_kv), P(dg_gen_params), P(dg_eb_params), P(dg_eb_state),
                          P(dg_step_out), c_void_p, P(i32), c_void_p, c_void_p, ctypes.c_size_t,
                          c_void_p]),
    "dg_kv_append_tokens": (i32, [c_void_p, P(dg_kv), c_void_p, i32, c_void_p, ctypes.c_size_t,
                                  c_void_p]),
    "dg_layer_forward": (i32, [c_void_p, P(dg_kv), i32, i32, c_void_p, c_void_p, c_void_p,
                               c_void_p, c_void_p, ctypes.c_size_t, c_void_p]),
    "dg_layer_forward_tokens": (i32, [c_void_p, P(dg_kv), i32, i32, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, ctypes.c_size_t, c_void_p]),
    "dg_ffn_forward": (i32, [c_void_p, i32, i32, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p, ctypes.c_size_t, c_void_p]),
    "dg_lm_head_forward": (i32, [c_void_p, i32, c_void_p, i32, P(dg_eb_params), P(dg_step_out),
                                 c_void_p, ctypes.c_size_t, c_void_p]),
    "dg_quantize_rows_fp8": (i32, [c_void_p, i32, c_void_p, c_void_p, ctypes.c_int64,
                                   ctypes.c_int64, c_void_p]),
    "dg_pack_weight_fp8": (i32, [c_void_p, c_void_p, ctypes.c_int64, ctypes.c_int64, c_void_p]),
    "dg_copy_bytes": (i32, [c_void_p, c_void_p, ctypes.c_size_t, c_void_p]),
    "dg_bench_read_stream": (i32, [c_void_p, ctypes.c_size_t, c_void_p, c_void_p]),
    "dg_bench_mfma_loop_blocks": (i32, []),
    "dg_bench_mfma_loop": (i32, [i32, c_void_p, c_void_p]),
    "dg_pack_weight": (i32, [c_void_p, c_void_p, ctypes.c_int64, ctypes.c_int64, c_void_p]),
    "dg_prof_num_classes": (i32, []),
    "dg_prof_class_name": (ctypes.c_char_p, [i32]),
    "dg_prof_enable": (i32, [ctypes.c_uint32]),
    "dg_prof_read": (i32, [i32, P(ctypes.c_double), P(ctypes.c_int64)]),
    "dg_prof_reset": (i32, []),
}
EXPORTED = sorted(_SIGS)

_lib = None


class DgError(RuntimeError):
    pass


def load(path=LIB_PATH):
    """Load libdg.so (raises if it has not been built) and declare its entry points."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise DgError(f"{path} is missing: build it with "
                      f"`python -m block_diffusion_decoding_canvas_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status, what=""):
    if status != DG_OK:
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        msg = load().dg_last_error().decode(errors="replace")
        raise DgError(f"{what}: {name}: {msg}")


def ptr(t):
    """Raw device pointer of a torch tensor (None -> NULL)."""
    return None if t is None else c_void_p(t.data_ptr())


def stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return c_void_p(s.cuda_stream)
