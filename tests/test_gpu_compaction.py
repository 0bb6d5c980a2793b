"""Frozen-canvas compaction (dg_decoder_step_live, dg_generate's compact_frozen): a step over only
the live canvases of a batch gives their state, outputs and cache rows bit for bit as the full
step does, and leaves the frozen canvases alone.

Workloads: the toy decoder with a sharp LM head (commits mid-run, so the canvases of a batch of 3
freeze at different steps), run step by step with and without compaction and through the
generation loop; the same toy decoder over 64 canvases, whose live steps drop from the long-call
kernel shapes to the decoder-step ones as canvases freeze; and two full-width layers with the 262,144-entry vocabulary, a batch of 4
canvases (1,024 tokens: the wide tile configurations) against 2 live ones (512 tokens).
"""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _toy(B=3):
    dims = synth.dims_tiny()
    mnp = synth.make_model(dims, seed=0, norm_gain_std=0.1, lm_std=1.0)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    cache = synth.make_cache(dims, B, 96, 32, seed=1)
    cache["len"] = np.array([32, 20, 27][:B])
    return dims, model, cache


def _state_equal(a, b, live=None):
    ha, hb = a.host(), b.host()
    for k in ha:
        assert np.array_equal(ha[k], hb[k]), k


@pytest.mark.parametrize("kind", ["entropy_bound", "block_refinement"])
def test_compacted_steps_bit_identical_with_staggered_freezes(kind):
    dims, model, cache = _toy()
    B, C, V = 3, dims["C"], dims["V"]
    kv = driver.KVCache.from_host(dims, cache, 96, DEV)
    ws = driver.workspace(model.workspace_bytes(B))
    p = driver.sched_params(kind, max_steps=12, seed=4, temperature=0.6, threshold=0.95)
    full, comp = (driver.SamplerState(B, C, DEV, canvas_ids=[5, 1, 9]) for _ in range(2))
    driver.canvas_init(driver.eb_params(seed=4), full, V)
    driver.canvas_init(driver.eb_params(seed=4), comp, V)
    of, oc = driver.StepOut(B, C, V, DEV), driver.StepOut(B, C, V, DEV)
    staggered = False
    for s in range(12):
        live = [b for b in range(B) if not bool(comp.done[b])]
        if not live:
            break
        staggered |= 0 < len(live) < B
        print(f"{kind} step {s}: live canvases {live}", flush=True)
        driver.decoder_step_sched(model, kv, s, p, full, of, ws)
        driver.decoder_step_live(model, kv, s, p, comp, oc, live, ws)
        torch.cuda.synchronize()
        _state_equal(full, comp)
        for b in live:      # the outputs of live canvases; frozen rows keep their last values
            assert torch.equal(of.logits[b], oc.logits[b])
            assert torch.equal(of.entropy[b], oc.entropy[b])
            assert torch.equal(of.argmax[b], oc.argmax[b])
            assert torch.equal(of.commit_now[b], oc.commit_now[b])
    assert staggered, "the canvases froze together: the workload does not stagger"
    assert bool(full.done.all())


def test_generate_compacted_matches_uncompacted():
    dims, model, cache = _toy()
    B, C, V = 3, dims["C"], dims["V"]
    p = driver.sched_params("entropy_bound", max_steps=10, seed=6)
    results = []
    for compact in (False, True):
        kv = driver.KVCache.from_host(dims, cache, 96, DEV)
        st = driver.SamplerState(B, C, DEV)
        out = driver.StepOut(B, C, V, DEV)
        tokens, n, steps = driver.generate(model, kv, p, st, out, 2 * C, compact_frozen=compact)
        torch.cuda.synchronize()
        results.append((tokens.cpu().numpy(), n, steps, kv.k.clone(), kv.v.clone(),
                        kv.lengths()))
    a, b = results
    assert np.array_equal(a[0], b[0]) and a[1] == b[1] and a[2] == b[2]
    assert torch.equal(a[3], b[3]) and torch.equal(a[4], b[4]) and a[5] == b[5]
    print(f"generate: {a[1]} canvases, steps {a[2]}")


def test_compacted_full_width_bit_identical():
    """Per-row arithmetic of every product does not depend on which rows share a tile: a step
    over 2 of 4 canvases (512 tokens, narrow tiles) equals the full step (1,024 tokens, wide
    expert tiles) on those canvases, bit for bit."""
    dims = synth.dims_full(n_layers=2)
    B, C, V = 4, dims["C"], dims["V"]
    w = synth.make_model_device(dims, DEV, seed=3)
    model = driver.Model(w)
    cap = 2048 + C
    k, v = synth.make_cache_device(dims, B, cap, 2048, DEV, seed=4)
    kv = driver.KVCache(dims, B, cap, DEV, k, v, [2048, 1500, 2048, 999])
    ws = driver.workspace(model.workspace_bytes(B))
    p = driver.sched_params("entropy_bound", seed=7, stop_entropy=-1.0)
    full, comp = (driver.SamplerState(B, C, DEV) for _ in range(2))
    driver.canvas_init(driver.eb_params(seed=7), full, V)
    driver.canvas_init(driver.eb_params(seed=7), comp, V)
    of, oc = driver.StepOut(B, C, V, DEV), driver.StepOut(B, C, V, DEV)
    live = [3, 1]
    for s in (0, 1):
        driver.decoder_step_sched(model, kv, s, p, full, of, ws)
        driver.decoder_step_live(model, kv, s, p, comp, oc, live, ws)
        torch.cuda.synchronize()
        for b in live:
            assert torch.equal(of.logits[b], oc.logits[b]), f"logits canvas {b} step {s}"
            assert torch.equal(of.entropy[b], oc.entropy[b])
        hf, hc = full.host(), comp.host()
        for key in hf:
            assert np.array_equal(hf[key][live], hc[key][live]), key
        for b in (0, 2):                      # not live: untouched by the compacted step
            assert not oc.logits[b].any()
        # the next step starts from the same state on both sides
        comp.canvas.copy_(full.canvas)
        comp.prev_argmax.copy_(full.prev_argmax)
        comp.stable_count.copy_(full.stable_count)


def test_compacted_steps_batch_64_across_tile_shapes():
    """64 toy canvases (1,024 tokens: the long-call expert tiles and dense shapes) on caches of
    ragged lengths from 0 to 40; as canvases freeze, the live steps fall under 1,024 tokens and
    take the decoder-step shapes while the full step keeps the long-call ones.  State and live
    outputs bit for bit, step by step."""
    dims = synth.dims_tiny()
    mnp = synth.make_model(dims, seed=0, norm_gain_std=0.1, lm_std=1.0)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    B, C, V, cap = 64, dims["C"], dims["V"], 64
    cache = synth.make_cache(dims, B, cap, 40, seed=2)
    lens = np.random.default_rng(3).integers(0, 41, size=B)
    for b, n in enumerate(lens):
        for lst in (cache["k"], cache["v"]):
            for a in lst:
                a[b, :, n:] = 0.0
    cache["len"] = lens
    kv = driver.KVCache.from_host(dims, cache, cap, DEV)
    ws = driver.workspace(model.workspace_bytes(B))
    p = driver.sched_params("entropy_bound", max_steps=12, seed=6, temperature=0.6)
    ids = list(range(200, 200 + B))
    full, comp = (driver.SamplerState(B, C, DEV, canvas_ids=ids) for _ in range(2))
    driver.canvas_init(driver.eb_params(seed=6), full, V)
    driver.canvas_init(driver.eb_params(seed=6), comp, V)
    of, oc = driver.StepOut(B, C, V, DEV), driver.StepOut(B, C, V, DEV)
    n_live = []
    for s in range(12):
        live = [b for b in range(B) if not bool(comp.done[b])]
        if not live:
            break
        n_live.append(len(live))
        driver.decoder_step_sched(model, kv, s, p, full, of, ws)
        driver.decoder_step_live(model, kv, s, p, comp, oc, live, ws)
        torch.cuda.synchronize()
        _state_equal(full, comp)
        lv = torch.tensor(live, device=DEV)
        for a, b in ((of.logits, oc.logits), (of.entropy, oc.entropy), (of.argmax, oc.argmax),
                     (of.commit_now, oc.commit_now)):
            assert torch.equal(a[lv], b[lv])
    print(f"live canvases per step: {n_live}", flush=True)
    assert any(0 < n < B for n in n_live), "the canvases froze together: no compacted step"
    assert bool(full.done.all())
