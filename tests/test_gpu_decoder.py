"""GPU parity of the decoder path (dg_decoder_step, dg_kv_append_canvas, dg_layer_forward).

Workloads: the 2-layer toy decoder (d 64, 4 heads of 16, 8 experts top-2 + shared, V 512,
canvas 16, 32 prompt tokens prefilled through the encoder append) run for 8 EB steps in lockstep
with the oracle, a "hot" variant with a sharper LM head so that commits happen mid-run, and one
full-width layer (d 2816, 16/8 heads of 256, 128 experts top-8 + shared, F 704) over a 256-token
canvas with a 2,048-entry N(0,1) cache, as decoder and as encoder.
"""
import copy

import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from oracle import model as om
from oracle import sampler as osamp
from tests.parity_util import (GpuChain, assert_close_rel, check_forced_routing,
                               compare_eb_step)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cache64(cache):
    return dict(k=[a.astype(np.float64) for a in cache["k"]],
                v=[a.astype(np.float64) for a in cache["v"]], len=np.array(cache["len"]))


def _prefill_both(dims, model_np, model_dev, prompt, cap):
    """Prompt prefill: the GPU appends it canvas by canvas, the oracle encodes it in one pass."""
    m64 = synth.model_to_f64(model_np)
    ref = _cache64(synth.empty_cache(dims, 1, cap))
    om.encoder_append(prompt[None], m64, ref)
    kv = driver.KVCache(dims, 1, cap, DEV)
    model = driver.Model(model_dev)
    ws = driver.workspace(model.workspace_bytes(1))
    C = dims["C"]
    for c0 in range(0, prompt.shape[0], C):
        tok = torch.tensor(prompt[None, c0:c0 + C], dtype=torch.int32, device=DEV)
        driver.kv_append_canvas(model, kv, tok, ws)
    torch.cuda.synchronize()
    return m64, ref, kv, model, ws


@pytest.mark.parametrize("hot", [False, True])
def test_tiny_prefill_and_8_step_lockstep(hot):
    dims = synth.dims_tiny()
    mnp = synth.make_model(dims, seed=0, norm_gain_std=0.1, lm_std=1.0 if hot else 0.02)
    mdev = synth.model_to_device(mnp, DEV)
    prompt = synth.prompt_ids(32, dims["V"])
    cap = 64
    m64, ref_cache, kv, model, ws = _prefill_both(dims, mnp, mdev, prompt, cap)
    assert kv.lengths() == [32]
    for layer in range(dims["n_layers"]):
        kg = kv.k[layer].float().cpu().numpy()[:, :, :32]
        vg = kv.v[layer].float().cpu().numpy()[:, :, :32]
        assert_close_rel(kg, ref_cache["k"][layer][:, :, :32], what=f"prefill K layer {layer}")
        assert_close_rel(vg, ref_cache["v"][layer][:, :, :32], what=f"prefill V layer {layer}")

    params = dict(osamp.default_params(), max_steps=8)
    seed, ids = 2, [0]
    p = driver.eb_params_from_dict(params, seed)
    gs = driver.SamplerState(1, dims["C"], DEV)
    driver.canvas_init(p, gs, dims["V"])
    st = osamp.new_state(osamp.init_canvas(seed, ids, dims["C"], dims["V"]))
    assert np.array_equal(gs.host()["canvas"], st["canvas"])
    out = driver.StepOut(1, dims["C"], dims["V"], DEV)
    commits = exact = 0
    for s in range(8):
        # every step starts from the oracle's state (oracle -> GPU only), so each step is
        # compared on identical canvases even after a near-tie decision
        gs.load_host(st)
        driver.decoder_step(model, kv, s, p, gs, out, ws)
        torch.cuda.synchronize()
        chain = GpuChain(dims, model, kv, ws, st["canvas"], mnp["embed"])
        zr, z64, infos = om.decoder_forward(st["canvas"], m64, ref_cache, force_idx=chain.idx)
        chain.check(infos, dims["top_k"], f"s={s}")
        zg = out.logits.float().cpu().numpy()
        assert_close_rel(zg, zr, what=f"logits s={s} (all rows)")
        err = np.abs(zg - z64).max(axis=-1)
        before = copy.deepcopy(st)
        ref = osamp.eb_step(zr, s, params, st, seed, ids)
        ok = compare_eb_step(f"hot={hot} s={s}", params, seed, ids, before, st, ref, gs.host(),
                             out, z64, err)
        commits += int(ref["commit_now"].sum())
        exact += int(ok)
        print(f"step {s}: commits {int(ref['commit_now'].sum())}, mean H "
              f"{ref['entropy'].mean():.4f}, {'exact' if ok else 'near-tie (validity checked)'}")
        if st["done"].all():
            break
    assert st["done"].all()
    assert exact >= 1
    if hot:
        assert commits == dims["C"]


def _full_layer_setup(B=1, cache_len=2048, window=0, global_every=1):
    dims = synth.dims_full(n_layers=1, vocab=256)
    dims.update(window=window, global_every=global_every)
    rng = np.random.default_rng(0)
    mnp = dict(dims=dims, layers=[synth.make_layer(dims, rng, norm_gain_std=0.1)],
               embed=np.zeros((256, dims["d"]), np.float32),
               final_norm=np.ones(dims["d"], np.float32),
               w_lm=np.zeros((256, dims["d"]), np.float32))
    cap = cache_len + dims["C"]
    cache = synth.make_cache(dims, B, cap, cache_len, seed=1)
    h = synth.hidden_states(B * dims["C"], dims["d"], seed=1).reshape(B, dims["C"], dims["d"])
    return dims, mnp, cache, h, cap


@pytest.mark.parametrize("causal", [0, 1])
def test_full_width_layer(causal):
    dims, mnp, cache, h, cap = _full_layer_setup()
    mdev = synth.model_to_device(mnp, DEV)
    model = driver.Model(mdev)
    kv = driver.KVCache.from_host(dims, cache, cap, DEV)
    ws = driver.workspace(model.workspace_bytes(1))
    T = dims["C"]
    hg = torch.from_numpy(h.reshape(T, -1).astype(np.float32)).to(DEV)
    rl = torch.zeros((T, dims["E"]), dtype=torch.float32, device=DEV)
    ti = torch.zeros((T, dims["top_k"]), dtype=torch.int32, device=DEV)
    gt = torch.zeros((T, dims["top_k"]), dtype=torch.float32, device=DEV)
    driver.layer_forward(model, kv, 0, causal, hg, ws, rl, ti, gt)
    torch.cuda.synchronize()

    lw = synth.model_to_f64(mnp)["layers"][0]
    c64 = _cache64(cache)
    h_ref, k_ref, v_ref, info = om.layer_forward(h.astype(np.float64), lw, dims, 0, np.stack(
        [c64["k"][0][b] for b in range(1)]), np.stack([c64["v"][0][b] for b in range(1)]),
        c64["len"], causal=bool(causal))
    # router: logits within tolerance; top-k ids exact where the k-th/(k+1)-th gap is certified
    rg = rl.cpu().numpy()
    r_ref = info["router_logits"]
    assert_close_rel(rg, r_ref, what="router logits")
    rerr = np.abs(rg - r_ref).max(axis=1)
    tig = ti.cpu().numpy()
    k = dims["top_k"]
    sets = orders = 0
    for t in range(T):
        srt = np.sort(r_ref[t])[::-1]
        gaps = srt[:k] - srt[1:k + 1]
        margin = 2 * rerr[t] + 1e-7
        if gaps[-1] > margin:      # the selected set is unambiguous
            assert set(tig[t]) == set(info["topk_idx"][t]), f"top-k set differs at token {t}"
            sets += 1
            if gaps.min() > margin:  # and so is the descending order
                assert list(tig[t]) == list(info["topk_idx"][t]), f"top-k order at token {t}"
                assert_close_rel(gt.cpu().numpy()[t], info["gates"][t], what=f"gates t={t}")
                orders += 1
    print(f"router: {sets}/{T} sets and {orders}/{T} orders certified")
    assert sets >= T // 2
    # outputs: every token at the stated tolerance, the oracle taking the GPU's expert set where
    # the router logits sit at a k-th/(k+1)-th near-tie (checked for validity)
    hout = hg.cpu().numpy()
    swaps = check_forced_routing(r_ref, rg, tig, k, "full-width layer")
    h_f, _, _, _ = om.layer_forward(h.astype(np.float64), lw, dims, 0, np.stack(
        [c64["k"][0][b] for b in range(1)]), np.stack([c64["v"][0][b] for b in range(1)]),
        c64["len"], causal=bool(causal), force_idx=tig.reshape(1, T, k))
    h_f = h_f.reshape(T, -1)
    print(f"near-tie expert swaps: {swaps}/{T}")
    assert_close_rel(hout, h_f, what="layer output (all tokens)")
    # the layer's increment on its own (the residual input passes through unchanged)
    h_in = h.reshape(T, -1).astype(np.float64)
    assert_close_rel(hout - h_in, h_f - h_in, what="layer increment (all tokens)")
    if causal:
        kgpu = kv.k[0].float().cpu().numpy()[0, :, 2048:2048 + T]
        vgpu = kv.v[0].float().cpu().numpy()[0, :, 2048:2048 + T]
        assert_close_rel(kgpu, k_ref[0].transpose(1, 0, 2), what="appended K")
        assert_close_rel(vgpu, v_ref[0].transpose(1, 0, 2), what="appended V")
