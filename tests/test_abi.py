"""CPU checks of the C ABI library: it loads without a GPU, exports every declared symbol, and
host-side validation rejects bad calls before anything is enqueued (no compute call is made)."""
import ctypes
import os
import re

import pytest

from block_diffusion_decoding_canvas_amd import _lib, driver

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "dg.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(dg_[a-z_0-9]+)\s*\(", src)
    return sorted(set(names))


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_functions()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(_lib.EXPORTED)


def _tiny_dims(**kw):
    d = dict(n_layers=2, d=64, hq=4, hkv=4, dh=16, E=8, top_k=2, F=128, Fs=128, V=512, C=16,
             window=0, global_every=1, eps=1e-6)
    d.update(kw)
    return driver.dims_struct(d)


def _create(dims, null_layer=False, scales=True, s_lm=True):
    lib = _lib.load()
    n = dims.n_layers
    layers = (_lib.dg_layer_w * n)()
    fake = 0x1000
    for i in range(n):
        for k in driver.Model.LAYER_KEYS:
            setattr(layers[i], k, fake)
        if scales:
            for k in driver.Model.SCALE_KEYS:
                setattr(layers[i], k, fake)
    if null_layer:
        layers[n - 1].w_down = None
    h = ctypes.c_void_p()
    st = lib.dg_model_create(ctypes.byref(dims), layers, ctypes.c_void_p(fake),
                             ctypes.c_void_p(fake), ctypes.c_void_p(fake),
                             ctypes.c_void_p(fake) if s_lm else None, ctypes.byref(h))
    return st, h


def test_model_create_validation():
    lib = _lib.load()
    st, h = _create(_tiny_dims())
    assert st == 0 and h.value
    assert lib.dg_workspace_bytes(h, 1) > 0
    lib.dg_model_destroy(h)
    bad = [dict(hq=6, hkv=4), dict(top_k=9), dict(d=48), dict(F=100), dict(V=500),
           dict(C=0), dict(C=2000), dict(window=8), dict(dh=8), dict(d=8224)]
    for kw in bad:
        st, _ = _create(_tiny_dims(**kw))
        assert st == 2, kw                       # DG_ERR_SHAPE
        assert lib.dg_last_error()
    st, h = _create(_tiny_dims(d=8192))            # the largest row a workgroup holds
    assert st == 0
    lib.dg_model_destroy(h)
    st, _ = _create(_tiny_dims(), null_layer=True)
    assert st == 1                               # DG_ERR_NULL
    d = _tiny_dims()
    d.wdtype = 7
    st, _ = _create(d)
    assert st == 3                               # DG_ERR_DTYPE
    # the bf16 configuration ignores the scale pointers
    st, h = _create(_tiny_dims(), scales=False, s_lm=False)
    assert st == 0
    lib.dg_model_destroy(h)


def test_fp8_model_create_validation():
    lib = _lib.load()
    fp8 = dict(wdtype="e4m3")
    st, h = _create(_tiny_dims(**fp8))
    assert st == 0
    # the fp8 workspace holds the e4m3 activation buffers on top of the bf16 one
    st2, hb = _create(_tiny_dims())
    assert lib.dg_workspace_bytes(h, 1) > lib.dg_workspace_bytes(hb, 1)
    lib.dg_model_destroy(h)
    lib.dg_model_destroy(hb)
    assert _create(_tiny_dims(d=96, **fp8))[0] == 2        # d_model % 64
    assert _create(_tiny_dims(F=96, **fp8))[0] == 2        # ffn_inner % 64
    assert _create(_tiny_dims(**fp8), scales=False)[0] == 1
    assert _create(_tiny_dims(**fp8), s_lm=False)[0] == 1


def test_quantize_and_pack_fp8_validation():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    assert lib.dg_quantize_rows_fp8(fake, 0, fake, fake, 4, 6, None) == 2
    assert lib.dg_quantize_rows_fp8(fake, 0, fake, fake, 0, 8, None) == 2
    assert lib.dg_quantize_rows_fp8(None, 0, fake, fake, 4, 8, None) == 1
    assert lib.dg_pack_weight_fp8(fake, ctypes.c_void_p(0x2000), 16, 32, None) == 2
    assert lib.dg_pack_weight_fp8(fake, ctypes.c_void_p(0x2000), 8, 64, None) == 2
    assert lib.dg_pack_weight_fp8(fake, fake, 16, 64, None) == 2   # aliasing
    assert lib.dg_pack_weight_fp8(None, fake, 16, 64, None) == 1


def test_stage_calls_validate():
    lib = _lib.load()
    st, h = _create(_tiny_dims())
    ws = lib.dg_workspace_bytes(h, 2)
    fake = ctypes.c_void_p(0x1000)
    assert lib.dg_ffn_forward(h, 2, 1, fake, None, None, None, fake, ws, None) == 2   # layer
    assert lib.dg_ffn_forward(h, 0, 2, fake, None, None, None, fake, ws - 1, None) == 5
    assert lib.dg_ffn_forward(h, 0, 0, fake, None, None, None, fake, ws, None) == 2
    p = driver.eb_params(max_steps=8)
    out = _lib.dg_step_out(0x1000, 0x1000, 0x1000, 0x1000)
    assert lib.dg_lm_head_forward(h, 2, fake, 8, ctypes.byref(p), ctypes.byref(out), fake, ws,
                                  None) == 6
    out.logits = None
    assert lib.dg_lm_head_forward(h, 2, fake, 0, ctypes.byref(p), ctypes.byref(out), fake, ws,
                                  None) == 1
    lib.dg_model_destroy(h)


def test_eb_sample_validation_before_launch():
    lib = _lib.load()
    p = driver.eb_params()
    fake = ctypes.c_void_p(0x1000)
    state = _lib.dg_eb_state(*([0x1000] * 7))
    out = _lib.dg_step_out(0x1000, 0x1000, 0x1000, 0)
    need = lib.dg_eb_workspace_bytes(1, 256, 262144)
    assert need > 0

    def call(step=0, b=1, c=256, v=262144, ws=need, params=p, st=state, o=out, logits=fake):
        return lib.dg_eb_sample(logits, b, c, v, step, ctypes.byref(params),
                                ctypes.byref(st) if st is not None else None,
                                ctypes.byref(o), fake, ws, None)

    assert call(step=48) == 6                    # DG_ERR_STATE
    assert call(step=-1) == 6
    assert call(ws=need - 1) == 5                # DG_ERR_WORKSPACE
    assert call(v=1000) == 2                     # DG_ERR_SHAPE
    assert call(c=2048) == 2
    assert call(logits=None) == 1                # DG_ERR_NULL
    st2 = _lib.dg_eb_state(*([0x1000] * 7))
    st2.done = None
    assert call(st=st2) == 1
    bad = driver.eb_params(t_min=0.0)
    assert call(params=bad) == 6


def test_eb_sample_noalloc_validation_before_launch():
    """The allocation-free sampler validates like dg_eb_sample and rejects inputs whose scratch
    exceeds its fixed array, before any HIP call."""
    lib = _lib.load()
    cap = lib.dg_eb_sample_noalloc_max_bytes()
    assert cap == 8 << 20
    p = driver.eb_params()
    fake = ctypes.c_void_p(0x1000)
    state = _lib.dg_eb_state(*([0x1000] * 7))
    out = _lib.dg_step_out(0x1000, 0x1000, 0x1000, 0)

    def call(b=1, c=256, v=262144, logits=fake, step=0):
        return lib.dg_eb_sample_noalloc(logits, b, c, v, step, ctypes.byref(p),
                                        ctypes.byref(state), ctypes.byref(out), None)

    assert call(logits=None) == 1                # DG_ERR_NULL
    assert call(v=1000) == 2                     # DG_ERR_SHAPE
    assert call(c=2048) == 2
    assert lib.dg_eb_workspace_bytes(16, 256, 262144) <= cap
    assert lib.dg_eb_workspace_bytes(32, 256, 262144) > cap
    assert call(b=32) == 5                       # DG_ERR_WORKSPACE: beyond the fixed scratch
    assert b"scratch" in lib.dg_last_error()


def test_layer_forward_tokens_validate():
    lib = _lib.load()
    st, h = _create(_tiny_dims())
    lens = (ctypes.c_int32 * 1)(60)
    kv = _lib.dg_kv(0x1000, 0x1000, 1, 64, lens)
    fake = ctypes.c_void_p(0x1000)
    ws = lib.dg_append_workspace_bytes(h, 1, 4)

    def call(layer=0, n=4, w=ws):
        return lib.dg_layer_forward_tokens(h, ctypes.byref(kv), layer, n, fake, None, None, None,
                                           fake, w, None)

    assert call(layer=2) == 2                    # layer out of range
    assert call(n=0) == 2
    assert call(n=5, w=1 << 40) == 4             # 60 + 5 > cap 64
    assert call(w=ws - 1) == 5                   # workspace sized below 4 tokens
    assert lens[0] == 60
    lib.dg_model_destroy(h)


def test_decoder_calls_validate_kv_and_step():
    lib = _lib.load()
    st, h = _create(_tiny_dims())
    assert st == 0
    lens = (ctypes.c_int32 * 1)(60)
    kv = _lib.dg_kv(0x1000, 0x1000, 1, 64, lens)
    p = driver.eb_params(max_steps=8)
    state = _lib.dg_eb_state(*([0x1000] * 7))
    out = _lib.dg_step_out(0x1000, 0x1000, 0x1000, 0x1000)
    ws = lib.dg_workspace_bytes(h, 1)
    fake = ctypes.c_void_p(0x1000)
    # append past capacity: 60 + 16 > 64
    assert lib.dg_kv_append_canvas(h, ctypes.byref(kv), fake, fake, ws, None) == 4
    assert lens[0] == 60
    assert lib.dg_decoder_step(h, ctypes.byref(kv), 8, ctypes.byref(p), ctypes.byref(state),
                               ctypes.byref(out), fake, ws, None) == 6
    assert lib.dg_decoder_step(h, ctypes.byref(kv), 0, ctypes.byref(p), ctypes.byref(state),
                               ctypes.byref(out), fake, ws - 1, None) == 5
    out.logits = None
    assert lib.dg_decoder_step(h, ctypes.byref(kv), 0, ctypes.byref(p), ctypes.byref(state),
                               ctypes.byref(out), fake, ws, None) == 1
    lib.dg_model_destroy(h)


def test_append_tokens_validate():
    lib = _lib.load()
    st, h = _create(_tiny_dims())
    assert st == 0
    lens = (ctypes.c_int32 * 1)(60)
    kv = _lib.dg_kv(0x1000, 0x1000, 1, 64, lens)
    fake = ctypes.c_void_p(0x1000)
    sizes = [lib.dg_append_workspace_bytes(h, 1, n) for n in (1, 4, 15, 16, 17, 100, 1000, 8192)]
    assert all(s > 0 for s in sizes) and sizes == sorted(sizes)
    assert lib.dg_append_workspace_bytes(h, 1, 16) == lib.dg_workspace_bytes(h, 1)
    assert lib.dg_append_workspace_bytes(h, 1, 0) == 0
    assert lib.dg_append_workspace_bytes(h, 1, 8193) == 0
    assert lib.dg_append_workspace_bytes(h, 16, 8192) == 0      # batch * tokens > 65,536
    ws4 = lib.dg_append_workspace_bytes(h, 1, 4)

    def call(n, ws=ws4, tokens=fake):
        return lib.dg_kv_append_tokens(h, ctypes.byref(kv), tokens, n, fake, ws, None)

    assert call(0) == 2                          # DG_ERR_SHAPE
    assert call(8193, ws=1 << 40) == 2
    assert call(5, ws=1 << 40) == 4              # 60 + 5 > cap 64: DG_ERR_CAPACITY
    assert call(4, ws=ws4 - 1) == 5              # DG_ERR_WORKSPACE
    assert call(4, tokens=None) == 1             # DG_ERR_NULL
    assert lens[0] == 60                         # nothing appended
    lib.dg_model_destroy(h)
    # a windowed model takes at most `window` tokens per call
    st, h = _create(_tiny_dims(window=32, global_every=2))
    assert st == 0
    lens[0] = 0
    assert lib.dg_kv_append_tokens(h, ctypes.byref(kv), fake, 33, fake, 1 << 40, None) == 2
    lib.dg_model_destroy(h)


def test_generate_validates():
    lib = _lib.load()
    st, h = _create(_tiny_dims())
    assert st == 0
    lens = (ctypes.c_int32 * 1)(60)
    kv = _lib.dg_kv(0x1000, 0x1000, 1, 64, lens)
    p = driver.eb_params(max_steps=8)
    state = _lib.dg_eb_state(*([0x1000] * 7))
    out = _lib.dg_step_out(0x1000, 0x1000, 0x1000, 0x1000)
    need = lib.dg_generate_workspace_bytes(h, 1)
    assert need == lib.dg_workspace_bytes(h, 1) + 512
    fake = ctypes.c_void_p(0x1000)
    done = ctypes.c_int32(-7)

    def call(g, ws=need, tokens=fake, o=out):
        gen = _lib.dg_gen_params(g, -1, 1)
        return lib.dg_generate(h, ctypes.byref(kv), ctypes.byref(gen), ctypes.byref(p),
                               ctypes.byref(state), ctypes.byref(o), tokens, ctypes.byref(done),
                               None, fake, ws, None)

    assert call(4) == 4                  # 60 + one 16-token canvas > cap 64: DG_ERR_CAPACITY
    lens[0] = 0
    assert call(0) == 2                  # gen_length < 1: DG_ERR_SHAPE
    assert call(65) == 4                 # 5 canvases = 80 tokens > 64
    assert call(64, ws=need - 1) == 5    # DG_ERR_WORKSPACE
    assert call(64, tokens=None) == 1    # DG_ERR_NULL
    out2 = _lib.dg_step_out(0x1000, 0x1000, 0x1000, 0)
    assert call(64, o=out2) == 1         # logits are required
    assert lens[0] == 0 and done.value == -7
    lib.dg_model_destroy(h)


def test_prof_classes_named():
    t = driver.KernelTimer()
    assert "moe_gateup" in t.names and "lmhead" in t.names and "attention" in t.names


def test_fp8_kv_validation_before_launch():
    """An e4m3 cache needs both scale arrays and head_dim 128 or 256; an unknown dtype is an
    error; all before any HIP call."""
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    lens = (ctypes.c_int32 * 1)(60)
    p = driver.eb_params(max_steps=8)
    state = _lib.dg_eb_state(*([0x1000] * 7))
    out = _lib.dg_step_out(0x1000, 0x1000, 0x1000, 0x1000)

    def step(h, kv, ws):
        return lib.dg_decoder_step(h, ctypes.byref(kv), 8, ctypes.byref(p), ctypes.byref(state),
                                   ctypes.byref(out), fake, ws, None)

    st, h = _create(_tiny_dims())                  # head_dim 16
    assert st == 0
    ws = lib.dg_workspace_bytes(h, 1)
    kv = _lib.dg_kv(0x1000, 0x1000, 1, 64, lens, _lib.DG_FP8_E4M3, 0x2000, 0x3000)
    assert step(h, kv, ws) == 2                    # DG_ERR_SHAPE: fp8 cache at head_dim 16
    assert b"head_dim" in lib.dg_last_error()
    lib.dg_model_destroy(h)
    st, h = _create(_tiny_dims(hq=2, hkv=1, dh=128))
    assert st == 0
    ws = lib.dg_workspace_bytes(h, 1)
    kv = _lib.dg_kv(0x1000, 0x1000, 1, 64, lens, _lib.DG_FP8_E4M3, 0x2000, None)
    assert step(h, kv, ws) == 1                    # DG_ERR_NULL: missing value scales
    kv = _lib.dg_kv(0x1000, 0x1000, 1, 64, lens, 7, 0x2000, 0x3000)
    assert step(h, kv, ws) == 2                    # unknown dtype
    kv = _lib.dg_kv(0x1000, 0x1000, 1, 64, lens, _lib.DG_FP8_E4M3, 0x2000, 0x3000)
    assert step(h, kv, ws) == 6                    # valid cache: the step index (8 of 8) fails
    lib.dg_model_destroy(h)
