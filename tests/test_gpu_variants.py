"""GPU parity on shapes beyond the toy config: ragged batches, sliding-window layers, GQA, a shared
expert of a different width, per-canvas cache lengths, a frozen canvas, and determinism.

Model: 3 layers, d 64, 4 query / 2 KV heads of 32, 8 experts top-2 (inner 64) + shared expert
(inner 96), V 768, canvas 40, window 48 with layer 1 global (global_every 2), batch 3 with
cache lengths 100 / 37 / 64 (N(0,1) entries).
"""
import copy

import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from oracle import model as om
from oracle import sampler as osamp
from tests.parity_util import assert_close_rel, compare_eb_step, routing_certified

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dims():
    return dict(n_layers=3, d=64, hq=4, hkv=2, dh=32, E=8, top_k=2, F=64, Fs=96, V=768, C=40,
                window=48, global_every=2, eps=1e-6)


def _setup(lens=(100, 37, 64), cap=160, lm_std=1.0):
    dims = _dims()
    mnp = synth.make_model(dims, seed=3, norm_gain_std=0.1, lm_std=lm_std)
    B = len(lens)
    cache = synth.make_cache(dims, B, cap, max(lens), seed=4)
    for b, n in enumerate(lens):               # ragged lengths: entries past len[b] are zero
        for lst in (cache["k"], cache["v"]):
            for a in lst:
                a[b, :, n:] = 0.0
    cache["len"] = np.array(lens, dtype=np.int64)
    return dims, mnp, cache, B, cap


def _cache64(cache):
    return dict(k=[a.astype(np.float64) for a in cache["k"]],
                v=[a.astype(np.float64) for a in cache["v"]], len=np.array(cache["len"]))


def test_ragged_windowed_batch_steps_with_frozen_canvas():
    dims, mnp, cache, B, cap = _setup()
    m64 = synth.model_to_f64(mnp)
    c64 = _cache64(cache)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    kv = driver.KVCache.from_host(dims, cache, cap, DEV)
    ws = driver.workspace(model.workspace_bytes(B))
    params = dict(osamp.default_params(), max_steps=6)
    seed, ids = 9, [4, 7, 1]
    p = driver.eb_params_from_dict(params, seed)
    gs = driver.SamplerState(B, dims["C"], DEV, canvas_ids=ids)
    st = osamp.new_state(osamp.init_canvas(seed, ids, dims["C"], dims["V"]))
    st["done"][1] = True                       # canvas 1 is frozen: it must never change
    out = driver.StepOut(B, dims["C"], dims["V"], DEV)
    exact = 0
    for s in range(6):
        gs.load_host(st)
        driver.decoder_step(model, kv, s, p, gs, out, ws)
        torch.cuda.synchronize()
        zr, z64, _ = om.decoder_forward(st["canvas"], m64, c64)
        zg = out.logits.float().cpu().numpy()
        cert = routing_certified(dims, mnp, model, kv, ws, c64, st["canvas"],
                                 check_layers=True)[-1]
        cert = cert.reshape(B, dims["C"])
        assert cert.sum() >= cert.size // 4
        assert_close_rel(zg[cert], zr[cert], what=f"logits s={s} (certified rows)")
        err = np.abs(zg - z64).max(axis=-1)
        before = copy.deepcopy(st)
        ref = osamp.eb_step(zr, s, params, st, seed, ids)
        exact += int(compare_eb_step(f"s={s}", params, seed, ids, before, st, ref, gs.host(),
                                     out, z64, err))
        assert np.array_equal(gs.host()["canvas"][1], before["canvas"][1])
        if st["done"].all():
            break
    assert exact >= 1


def test_ragged_windowed_batch_append():
    dims, mnp, cache, B, cap = _setup()
    m64 = synth.model_to_f64(mnp)
    c64 = _cache64(cache)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    kv = driver.KVCache.from_host(dims, cache, cap, DEV)
    ws = driver.workspace(model.workspace_bytes(B))
    tokens = np.random.default_rng(5).integers(0, dims["V"], size=(B, dims["C"]))
    masks = routing_certified(dims, mnp, model, kv, ws, c64, tokens, causal=True)
    driver.kv_append_canvas(model, kv, torch.tensor(tokens, dtype=torch.int32, device=DEV), ws)
    torch.cuda.synchronize()
    om.encoder_append(tokens, m64, c64)
    assert kv.lengths() == [int(x) for x in c64["len"]]
    for layer in range(dims["n_layers"]):
        cert = masks[layer].reshape(B, dims["C"])
        for b in range(B):
            n0 = int(c64["len"][b]) - dims["C"]
            n1 = int(c64["len"][b])
            ok = cert[b]
            kg = kv.k[layer, b, :, n0:n1].float().cpu().numpy()[:, ok]
            vg = kv.v[layer, b, :, n0:n1].float().cpu().numpy()[:, ok]
            assert_close_rel(kg, c64["k"][layer][b, :, n0:n1][:, ok], what=f"K {layer} b {b}")
            assert_close_rel(vg, c64["v"][layer][b, :, n0:n1][:, ok], what=f"V {layer} b {b}")
            # entries before the append are untouched
            assert np.array_equal(kv.k[layer, b, :, :n0].float().cpu().numpy(),
                                  cache["k"][layer][b, :, :n0])


def test_decoder_step_is_deterministic():
    dims, mnp, cache, B, cap = _setup(lm_std=0.02)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    kv = driver.KVCache.from_host(dims, cache, cap, DEV)
    ws = driver.workspace(model.workspace_bytes(B))
    p = driver.eb_params(max_steps=6, seed=3)
    results = []
    for _ in range(2):
        gs = driver.SamplerState(B, dims["C"], DEV)
        driver.canvas_init(p, gs, dims["V"])
        out = driver.StepOut(B, dims["C"], dims["V"], DEV)
        for s in range(3):
            driver.decoder_step(model, kv, s, p, gs, out, ws)
        torch.cuda.synchronize()
        results.append((out.logits.clone(), out.entropy.clone(), gs.canvas.clone()))
    assert torch.equal(results[0][0], results[1][0])
    assert torch.equal(results[0][1], results[1][1])
    assert torch.equal(results[0][2], results[1][2])


def test_capacity_and_state_errors_enqueue_nothing():
    dims, mnp, cache, B, cap = _setup(lens=(150, 37, 64), cap=160)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    kv = driver.KVCache.from_host(dims, cache, cap, DEV)
    ws = driver.workspace(model.workspace_bytes(B))
    before = kv.k.clone()
    tok = torch.zeros((B, dims["C"]), dtype=torch.int32, device=DEV)
    with pytest.raises(driver._lib.DgError, match="CAPACITY"):
        driver.kv_append_canvas(model, kv, tok, ws)
    torch.cuda.synchronize()
    assert kv.lengths() == [150, 37, 64] and torch.equal(before, kv.k)
    gs = driver.SamplerState(B, dims["C"], DEV)
    out = driver.StepOut(B, dims["C"], dims["V"], DEV)
    with pytest.raises(driver._lib.DgError, match="STATE"):
        driver.decoder_step(model, kv, 6, driver.eb_params(max_steps=6), gs, out, ws)
