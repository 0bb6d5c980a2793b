"""GPU parity of the fp8 (OCP e4m3) configuration and of the FFN / LM-head stage entry points.

Integer decisions (the e4m3 codes, decided in binary32 from identical inputs) are compared
bit-exactly; the stage outputs (FFN residual increment, logits, entropies) within the stated
tolerance on every row, the oracle taking the GPU's expert set wherever the two sides' router
logits sit at a near-tie (checked for validity first); the end-to-end decoder run (a batch of 4
ragged caches, sliding-window and global layers) like the bf16 runs.
"""
import copy

import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from oracle import model as om
from oracle import sampler as osamp
from oracle.numerics import e4m3_code, quantize_rows_e4m3, round_bf16
from tests.parity_util import (FP8_CHAIN_ARRAY_TOL, FP8_CHAIN_TOL, GpuChain, argmax_certified,
                               assert_close_rel, assert_entropy_close, compare_eb_step,
                               entropy_sensitivity, entropy_tolerance, ffn_forced)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ffn_stages_on_oracle_states(dims, m64, c64, model, ws, canvas, force):
    """Every FFN (the quantised half of a layer) from the oracle's own post-attention state, on
    every row, with the oracle taking the GPU's expert sets at near-ties.  force: the GPU chain's
    expert sets per layer (the oracle's states follow the same choices)."""
    B, C = np.asarray(canvas).shape
    h = m64["embed"][np.asarray(canvas)]
    for layer, lw in enumerate(m64["layers"]):
        h_mid, _, _ = om.attention_block(h, lw, dims, layer, c64["k"][layer], c64["v"][layer],
                                         c64["len"], causal=False)
        inc_g, inc_r, _ = ffn_forced(model, lw, dims, layer, B, h_mid, ws, f"fp8 FFN {layer}")
        assert_close_rel(inc_g, inc_r, what=f"fp8 FFN increment, layer {layer}")
        h, _ = om.ffn_block(h_mid, lw, dims, force[layer])


def _oracle_final_hidden(canvas, m64, c64, force):
    """The oracle's residual stream after the last decoder layer, [B * C, d] (forced sets)."""
    dims = m64["dims"]
    h = m64["embed"][np.asarray(canvas)]
    for layer, lw in enumerate(m64["layers"]):
        h, _, _, _ = om.layer_forward(h, lw, dims, layer, c64["k"][layer], c64["v"][layer],
                                      c64["len"], causal=False, force_idx=force[layer])
    return h.reshape(-1, dims["d"])


def test_quantize_rows_bit_exact_bf16_and_f32():
    rng = np.random.default_rng(11)
    w = rng.standard_normal((96, 320)) * np.exp2(rng.uniform(-30, 12, (96, 1)))
    w[5] = 0.0
    w[7] *= np.exp2(rng.uniform(-30, 0, 320))          # wide spread: subnormal codes and zeros
    w = synth.to_bf16_values(w)
    wt = torch.from_numpy(w).to(DEV, torch.bfloat16)
    codes = torch.empty((96, 320), dtype=torch.uint8, device=DEV)
    scales = torch.empty(96, dtype=torch.float32, device=DEV)
    driver.quantize_rows_fp8(wt, codes, scales)
    q, s = quantize_rows_e4m3(w.astype(np.float64))
    assert np.array_equal(codes.cpu().numpy(), e4m3_code(q))
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), s)

    x = (rng.standard_normal((300, 704)) * np.exp2(rng.uniform(-20, 20, (300, 1)))).astype(np.float32)
    x[3, :17] = -0.0
    xt = torch.from_numpy(x).to(DEV)
    codes = torch.empty((300, 704), dtype=torch.uint8, device=DEV)
    scales = torch.empty(300, dtype=torch.float32, device=DEV)
    driver.quantize_rows_fp8(xt, codes, scales)
    q, s = quantize_rows_e4m3(x)
    assert np.array_equal(codes.cpu().numpy(), e4m3_code(q))
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), s)


def test_pack_fp8_layout():
    rng = np.random.default_rng(12)
    rows, cols = 48, 192
    c = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    ct = torch.from_numpy(c).to(DEV)
    out = torch.empty_like(ct)
    driver.pack_weight_fp8(ct, out)
    n, k = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
    dst = ((n // 16 * (cols // 64) + k // 64) * 64 + (k % 64) // 16 * 16 + n % 16) * 16 + k % 16
    want = np.empty(rows * cols, dtype=np.uint8)
    want[dst.ravel()] = c.ravel()
    assert np.array_equal(out.cpu().numpy().ravel(), want)


def _mid_dims(**kw):
    d = dict(n_layers=2, d=256, hq=4, hkv=2, dh=64, E=16, top_k=4, F=128, Fs=192, V=4096, C=64,
             window=0, global_every=1, eps=1e-6)
    d.update(kw)
    return d


def _ffn_case(dims, wdtype, B, seed):
    mnp = synth.make_model(dims, seed=seed, norm_gain_std=0.1)
    m64 = synth.model_to_f64(mnp)
    ref_model = om.quantize_model_e4m3(m64) if wdtype == "e4m3" else m64
    model = driver.Model(synth.model_to_device(mnp, DEV), wdtype=wdtype)
    ws = driver.workspace(model.workspace_bytes(B))
    T = B * dims["C"]
    h = synth.hidden_states(T, dims["d"], seed=seed + 1).astype(np.float64)
    for layer in range(dims["n_layers"]):
        lw = ref_model["layers"][layer]
        delta, f, swaps = ffn_forced(model, lw, dims, layer, B, h, ws, f"{wdtype} FFN {layer}")
        err = np.linalg.norm(delta - f, axis=1) / np.linalg.norm(f, axis=1)
        print(f"{wdtype} layer {layer}: FFN increment worst row rel err {err.max():.2e}, "
              f"near-tie expert swaps {swaps}/{T}")
        assert_close_rel(delta, f, what=f"{wdtype} FFN layer {layer}")


@pytest.mark.parametrize("wdtype", ["bf16", "e4m3"])
def test_ffn_stage_mid_size(wdtype):
    _ffn_case(_mid_dims(), wdtype, B=2, seed=21)


def test_ffn_stage_full_width_fp8():
    _ffn_case(synth.dims_full(n_layers=1, vocab=256), "e4m3", B=1, seed=22)


def _lm_head_case(dims, wdtype, B, seed, step):
    mnp = synth.make_model(dims, seed=seed, norm_gain_std=0.1, lm_std=0.1)
    m64 = synth.model_to_f64(mnp)
    w_lm = m64["w_lm"]
    s_lm = None
    if wdtype == "e4m3":
        w_lm, s_lm = quantize_rows_e4m3(w_lm)
    model = driver.Model(synth.model_to_device(mnp, DEV), wdtype=wdtype)
    ws = driver.workspace(model.workspace_bytes(B))
    T = B * dims["C"]
    h = synth.hidden_states(T, dims["d"], seed=seed + 1)
    params = osamp.default_params()
    p = driver.eb_params_from_dict(params, seed)
    out = driver.StepOut(B, dims["C"], dims["V"], DEV)
    driver.lm_head_forward(model, B, torch.from_numpy(h).to(DEV), step, p, out, ws)
    torch.cuda.synchronize()
    z64 = om.linear(om.rms_norm(h.astype(np.float64), m64["final_norm"], dims["eps"]), w_lm, s_lm)
    zr = round_bf16(z64)
    zg = out.logits.float().cpu().numpy().reshape(T, -1)
    assert_close_rel(zg, zr, what=f"{wdtype} logits")
    inv_t = osamp.inv_temperature_f32(step, params["max_steps"])
    h_ref, a_ref = osamp.entropy_argmax(zr, inv_t)
    dz = np.abs(zg - z64).max(axis=1)
    tol = entropy_tolerance(h_ref, dz * float(inv_t), entropy_sensitivity(z64, inv_t))
    assert_entropy_close(out.entropy.cpu().numpy().reshape(-1), h_ref, f"{wdtype} entropy", tol)
    ag = out.argmax.cpu().numpy().reshape(-1)
    n_exact = 0
    for t in range(T):
        if ag[t] != a_ref[t]:
            assert not argmax_certified(z64[t], dz[t]), f"argmax differs at certified row {t}"
        else:
            n_exact += 1
    print(f"{wdtype} LM head: argmax equal on {n_exact}/{T} rows, mean H {h_ref.mean():.3f}")
    assert n_exact >= T // 2


@pytest.mark.parametrize("wdtype", ["bf16", "e4m3"])
def test_lm_head_stage_mid_size(wdtype):
    _lm_head_case(_mid_dims(), wdtype, B=2, seed=31, step=40)


def test_lm_head_stage_full_vocab_fp8():
    dims = synth.dims_full(n_layers=1)
    dims.update(E=8, top_k=2, F=64, Fs=64)          # the FFN is not exercised here
    _lm_head_case(dims, "e4m3", B=1, seed=32, step=47)


def test_fp8_decoder_steps_batched_windowed():
    """C5-shaped at small width: 4 canvases with ragged caches, windowed layers 0, 1, 3, 4 and
    global layers 2, 5 (window 48 over caches of up to 180), e4m3 experts and LM head."""
    dims = dict(n_layers=6, d=128, hq=4, hkv=2, dh=32, E=8, top_k=2, F=128, Fs=128, V=2048, C=40,
                window=48, global_every=3, eps=1e-6)
    lens = (180, 37, 120, 64)
    mnp = synth.make_model(dims, seed=41, norm_gain_std=0.1, lm_std=0.5)
    m64 = om.quantize_model_e4m3(synth.model_to_f64(mnp))
    B, cap = len(lens), 240
    cache = synth.make_cache(dims, B, cap, max(lens), seed=42)
    for b, n in enumerate(lens):
        for lst in (cache["k"], cache["v"]):
            for a in lst:
                a[b, :, n:] = 0.0
    cache["len"] = np.array(lens, dtype=np.int64)
    c64 = dict(k=[a.astype(np.float64) for a in cache["k"]],
               v=[a.astype(np.float64) for a in cache["v"]], len=np.array(cache["len"]))
    model = driver.Model(synth.model_to_device(mnp, DEV), wdtype="e4m3")
    kv = driver.KVCache.from_host(dims, cache, cap, DEV)
    ws = driver.workspace(model.workspace_bytes(B))
    params = dict(osamp.default_params(), max_steps=5)
    seed, ids = 43, [0, 1, 2, 3]
    p = driver.eb_params_from_dict(params, seed)
    gs = driver.SamplerState(B, dims["C"], DEV, canvas_ids=ids)
    st = osamp.new_state(osamp.init_canvas(seed, ids, dims["C"], dims["V"]))
    out = driver.StepOut(B, dims["C"], dims["V"], DEV)
    exact = 0
    for s in range(params["max_steps"]):
        gs.load_host(st)
        driver.decoder_step(model, kv, s, p, gs, out, ws)
        torch.cuda.synchronize()
        chain = GpuChain(dims, model, kv, ws, st["canvas"], mnp["embed"])
        zr, z64, infos = om.decoder_forward(st["canvas"], m64, c64, force_idx=chain.idx)
        chain.check(infos, dims["top_k"], f"fp8 s={s}")
        zg = out.logits.float().cpu().numpy()
        # every FFN (the quantised half of a layer) from the oracle's own post-attention state
        _ffn_stages_on_oracle_states(dims, m64, c64, model, ws, st["canvas"], chain.idx)
        # the LM head from the oracle's final hidden state: logits at the stated tolerance
        h_fin = _oracle_final_hidden(st["canvas"], m64, c64, chain.idx)
        lm = driver.StepOut(B, dims["C"], dims["V"], DEV)
        driver.lm_head_forward(model, B, torch.from_numpy(h_fin.astype(np.float32)).to(DEV), s,
                               p, lm, ws)
        torch.cuda.synchronize()
        assert_close_rel(lm.logits.float().cpu().numpy(), zr, what=f"fp8 LM head s={s}")
        # end to end: e4m3 codes flip where upstream float differences cross a rounding
        # boundary; FP8_CHAIN_TOL is the bound for chained fp8 stages
        rel = np.linalg.norm(zg - zr, axis=-1) / np.linalg.norm(zr, axis=-1)
        print(f"fp8 step {s}: end-to-end logits worst row rel err {rel.max():.2e}, "
              f"median {np.median(rel):.2e}")
        assert_close_rel(zg, zr, rel=FP8_CHAIN_TOL, what=f"fp8 logits s={s}")
        assert np.linalg.norm(zg - zr) <= FP8_CHAIN_ARRAY_TOL * np.linalg.norm(zr)
        # the sampler on these logits: decisions robust to the observed logit error must match
        # exactly, the rest must be valid (the rule's choice on the GPU's own entropies); the
        # sampler's exact decisions on identical logits are pinned by the sampler tests
        err = np.abs(zg - z64).max(axis=-1)
        before = copy.deepcopy(st)
        ref = osamp.eb_step(zr, s, params, st, seed, ids)
        exact += int(compare_eb_step(f"fp8 s={s}", params, seed, ids, before, st, ref, gs.host(),
                                     out, z64, err))
        if st["done"].all():
            break
    print(f"fp8 run: {exact} canvas-steps compared exactly")
