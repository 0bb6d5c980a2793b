"""The step entry points under HIP graph capture.

dg_decoder_step and dg_eb_sample enqueue kernels only (no allocation, no host synchronisation,
no memset nodes), so a caller may capture a step once and replay it.  Each case captures one call
with torch.cuda.graph, replays it three times from the same starting state, with eager GPU work
and synchronisations between the replays, and requires every replay to reproduce the eager call
bit for bit: outputs (entropy, argmax, commit flags, logits) and the sampler state it updates.

Workloads: the 2-layer toy decoder with a sharp LM head (commits happen mid-run, so the candidate
draw and renoise paths are captured too), 8 steps each captured separately; two full-width layers
(d 2816, 16/8 heads of 256, 128 experts top-8 + shared, V 262,144) over a 2,048-entry cache at
steps 0 and 47 (the last step finalises the canvas); the standalone sampler on the 256-row
262,144-vocabulary logits at step 36, where most peaked rows commit.
"""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from oracle import sampler as osamp

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _state_tensors(state):
    return [state.canvas, state.committed, state.prev_argmax, state.stable_count, state.done,
            state.dev_status]


def _out_tensors(out):
    return [t for t in (out.entropy, out.argmax, out.commit_now, out.logits) if t is not None]


def _snapshot(ts):
    return [t.clone() for t in ts]


def _restore(ts, snap):
    for t, s in zip(ts, snap):
        t.copy_(s)


def _check_replays(call, state, out, what, replays=3):
    """Eager call, then capture + `replays` replays from the same state; bit-exact comparison."""
    st = _state_tensors(state)
    start = _snapshot(st)
    call()
    torch.cuda.synchronize()
    want_out, want_st = _snapshot(_out_tensors(out)), _snapshot(st)
    _restore(st, start)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    junk = torch.randn(512, 512, device=DEV)
    for r in range(replays):
        _restore(st, start)
        for t in _out_tensors(out):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        junk = junk @ junk.T / 512.0        # eager work between the replays
        torch.cuda.synchronize()
        for name, a, b in zip(("entropy", "argmax", "commit_now", "logits"),
                              _out_tensors(out), want_out):
            assert torch.equal(a, b), f"{what}: replay {r}: {name} differs from the eager call"
        for name, a, b in zip(("canvas", "committed", "prev_argmax", "stable_count", "done",
                               "dev_status"), st, want_st):
            assert torch.equal(a, b), f"{what}: replay {r}: state {name} differs"
    del g
    return want_out, want_st


def test_decoder_step_graph_tiny_hot():
    dims = synth.dims_tiny()
    mdev = synth.model_to_device(synth.make_model(dims, seed=0, norm_gain_std=0.1, lm_std=1.0),
                                 DEV)
    model = driver.Model(mdev)
    kv = driver.KVCache(dims, 1, 64, DEV)
    ws = driver.workspace(model.workspace_bytes(1))
    prompt = synth.prompt_ids(32, dims["V"])
    for c0 in range(0, 32, dims["C"]):
        driver.kv_append_canvas(model, kv, torch.tensor(prompt[None, c0:c0 + dims["C"]],
                                                        dtype=torch.int32, device=DEV), ws)
    torch.cuda.synchronize()
    p = driver.eb_params_from_dict(dict(osamp.default_params(), max_steps=8), 2)
    state = driver.SamplerState(1, dims["C"], DEV)
    driver.canvas_init(p, state, dims["V"])
    out = driver.StepOut(1, dims["C"], dims["V"], DEV)
    commits = 0
    for s in range(8):
        print(f"graph case tiny step {s}", flush=True)
        want_out, _ = _check_replays(lambda: driver.decoder_step(model, kv, s, p, state, out, ws),
                                     state, out, f"tiny step {s}")
        commits += int(want_out[2].sum())
        if bool(state.done.all()):
            break
    assert commits > 0, "no commits happened: the candidate path was not captured"


@pytest.mark.parametrize("step", [0, 47])
def test_decoder_step_graph_full_width(step):
    dims = synth.dims_full(n_layers=2)
    weights = synth.make_model_device(dims, DEV, seed=0)
    model = driver.Model(weights)
    cap, length = 2048 + dims["C"], 2048
    kc, vc = synth.make_cache_device(dims, 1, cap, length, DEV, seed=1)
    kv = driver.KVCache(dims, 1, cap, DEV, kc, vc, [length])
    ws = driver.workspace(model.workspace_bytes(1))
    p = driver.eb_params()
    state = driver.SamplerState(1, dims["C"], DEV)
    driver.canvas_init(p, state, dims["V"])
    out = driver.StepOut(1, dims["C"], dims["V"], DEV)
    print(f"graph case full width step {step}", flush=True)
    _, want_st = _check_replays(lambda: driver.decoder_step(model, kv, step, p, state, out, ws),
                                state, out, f"full width step {step}")
    if step == 47:
        assert bool(want_st[4].all()), "the last step must finalise the canvas"
        assert bool(want_st[1].all())


def test_eb_sample_graph():
    z, _ = synth.sampler_logits(256, 262144, seed=1)
    logits = synth.to_device_bf16(z.reshape(1, 256, 262144), DEV)
    p = driver.eb_params(stop_entropy=-1.0)
    state = driver.SamplerState(1, 256, DEV)
    driver.canvas_init(p, state, 262144)
    out = driver.StepOut(1, 256, 262144, DEV, with_logits=False)
    ws = driver.workspace(_ws_bytes(1, 256, 262144))
    print("graph case eb_sample step 36", flush=True)
    want_out, _ = _check_replays(lambda: driver.eb_sample(logits, 36, p, state, out, ws),
                                 state, out, "eb_sample step 36")
    assert int(want_out[2].sum()) > 0


def _ws_bytes(b, c, v):
    from block_diffusion_decoding_canvas_amd import _lib
    return _lib.load().dg_eb_workspace_bytes(b, c, v)
