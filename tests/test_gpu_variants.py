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
from tests.parity_util import (GpuChain, assert_close_rel, check_forced_routing,
                               compare_eb_step)

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
        chain = GpuChain(dims, model, kv, ws, st["canvas"], mnp["embed"])
        zr, z64, infos = om.decoder_forward(st["canvas"], m64, c64, force_idx=chain.idx)
        chain.check(infos, dims["top_k"], f"s={s}")
        zg = out.logits.float().cpu().numpy()
        assert_close_rel(zg, zr, what=f"logits s={s} (all rows)")
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
    chain = GpuChain(dims, model, kv, ws, tokens, mnp["embed"], causal=True)
    driver.kv_append_canvas(model, kv, torch.tensor(tokens, dtype=torch.int32, device=DEV), ws)
    torch.cuda.synchronize()
    force = chain.idx[:-1] + [None]     # the last layer's FFN does not reach the cache
    om.encoder_append(tokens, m64, c64, force_idx=force)
    assert kv.lengths() == [int(x) for x in c64["len"]]
    for layer in range(dims["n_layers"]):
        for b in range(B):
            n0 = int(c64["len"][b]) - dims["C"]
            n1 = int(c64["len"][b])
            kg = kv.k[layer, b, :, n0:n1].float().cpu().numpy()
            vg = kv.v[layer, b, :, n0:n1].float().cpu().numpy()
            assert_close_rel(kg, c64["k"][layer][b, :, n0:n1], what=f"K {layer} b {b}")
            assert_close_rel(vg, c64["v"][layer][b, :, n0:n1], what=f"V {layer} b {b}")
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


@pytest.mark.parametrize("d,top_k,E", [(1056, 10, 16), (3072, 8, 16), (256, 2, 6),
                                         (256, 16, 256)])
def test_layer_row_shapes(d, top_k, E):
    """One decoder layer over 2 canvases at model widths whose token rows end in a partial
    1024-column chunk (d 1056) or fill three chunks exactly (d 3072), with up to 10 routed
    experts per token, an expert count that is not a multiple of 4 (6: the router's output
    rows are stored element by element), and the routing maxima the C ABI accepts (256
    experts, 16 routed per token): the per-token row kernels (residual + norm, combine + next
    norm) and the routing against the oracle on every row (the oracle takes the GPU's expert
    set at router near-ties, checked for validity)."""
    dims = dict(n_layers=1, d=d, hq=4, hkv=2, dh=64, E=E, top_k=top_k, F=128, Fs=64, V=256,
                C=40, window=0, global_every=1, eps=1e-6)
    rng = np.random.default_rng(11)
    mnp = dict(dims=dims, layers=[synth.make_layer(dims, rng, norm_gain_std=0.1)],
               embed=np.zeros((256, d), np.float32), final_norm=np.ones(d, np.float32),
               w_lm=np.zeros((256, d), np.float32))
    B, cap, n = 2, 120, 70
    cache = synth.make_cache(dims, B, cap, n, seed=12)
    T = B * dims["C"]
    h = synth.hidden_states(T, d, seed=13)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    kv = driver.KVCache.from_host(dims, cache, cap, DEV)
    ws = driver.workspace(model.workspace_bytes(B))
    hg = torch.from_numpy(h.astype(np.float32)).to(DEV)
    rl = torch.zeros((T, dims["E"]), dtype=torch.float32, device=DEV)
    ti = torch.zeros((T, top_k), dtype=torch.int32, device=DEV)
    gt = torch.zeros((T, top_k), dtype=torch.float32, device=DEV)
    driver.layer_forward(model, kv, 0, 0, hg, ws, rl, ti, gt)
    torch.cuda.synchronize()
    lw = synth.model_to_f64(mnp)["layers"][0]
    k64 = cache["k"][0].astype(np.float64)
    v64 = cache["v"][0].astype(np.float64)
    h_ref, _, _, info = om.layer_forward(h.astype(np.float64).reshape(B, dims["C"], d), lw, dims,
                                         0, k64, v64, np.array(cache["len"]), causal=False)
    h_ref = h_ref.reshape(T, d)
    rg = rl.cpu().numpy()
    r_ref = info["router_logits"].reshape(T, -1)
    assert_close_rel(rg, r_ref, what="router logits")
    tig = ti.cpu().numpy().astype(np.int64)
    swaps = check_forced_routing(r_ref, rg, tig, top_k, f"d={d}")
    h_ref, _, _, _ = om.layer_forward(h.astype(np.float64).reshape(B, dims["C"], d), lw, dims,
                                      0, k64, v64, np.array(cache["len"]), causal=False,
                                      force_idx=tig.reshape(B, dims["C"], top_k))
    h_ref = h_ref.reshape(T, d)
    print(f"d={d} top_k={top_k} E={E}: near-tie expert swaps {swaps}/{T}")
    hout = hg.cpu().numpy()
    assert_close_rel(hout - h, h_ref - h, what=f"layer increment d={d} top_k={top_k} (all rows)")


def test_router_exact_ties_lowest_id_first():
    """Duplicated router rows give bit-identical logits (same products, same order): the top-k
    keeps the lower expert id ahead of its twin, and picks it alone when only one fits."""
    dims = dict(n_layers=1, d=64, hq=4, hkv=2, dh=16, E=8, top_k=3, F=64, Fs=64, V=256, C=40,
                window=0, global_every=1, eps=1e-6)
    rng = np.random.default_rng(21)
    lw = synth.make_layer(dims, rng, norm_gain_std=0.1)
    twins = [(2, 5), (1, 7)]
    for lo, hi in twins:
        lw["w_router"][hi] = lw["w_router"][lo]
    mnp = dict(dims=dims, layers=[lw], embed=np.zeros((256, 64), np.float32),
               final_norm=np.ones(64, np.float32), w_lm=np.zeros((256, 64), np.float32))
    cache = synth.make_cache(dims, 1, 80, 30, seed=22)
    T = dims["C"]
    model = driver.Model(synth.model_to_device(mnp, DEV))
    kv = driver.KVCache.from_host(dims, cache, 80, DEV)
    ws = driver.workspace(model.workspace_bytes(1))
    hg = torch.from_numpy(synth.hidden_states(T, 64, seed=23).astype(np.float32)).to(DEV)
    rl = torch.zeros((T, 8), dtype=torch.float32, device=DEV)
    ti = torch.zeros((T, 3), dtype=torch.int32, device=DEV)
    gt = torch.zeros((T, 3), dtype=torch.float32, device=DEV)
    driver.layer_forward(model, kv, 0, 0, hg, ws, rl, ti, gt)
    torch.cuda.synchronize()
    r = rl.cpu().numpy()
    sel = ti.cpu().numpy()
    seen_both = seen_one = 0
    for lo, hi in twins:
        assert np.array_equal(r[:, lo], r[:, hi])
    for t in range(T):
        # the selection is the rank order of (logit desc, id asc) over the GPU's own logits
        order = sorted(range(8), key=lambda e: (-r[t, e], e))[:3]
        assert list(sel[t]) == order, t
        for lo, hi in twins:
            if lo in sel[t] and hi in sel[t]:
                i = list(sel[t]).index(lo)
                assert sel[t][i + 1] == hi
                seen_both += 1
            elif hi in sel[t]:
                raise AssertionError(f"token {t}: expert {hi} chosen without its lower twin {lo}")
            elif lo in sel[t]:
                seen_one += 1
    print(f"twin pairs selected together {seen_both}, lower twin alone {seen_one}")
    assert seen_both + seen_one > 0


@pytest.mark.parametrize("off", [1, 4, 16, 32, 256, 1024])
def test_lm_head_statistics_exact_ties(off):
    """Duplicated LM-head rows (row v equals row v ^ off) give bit-identical logits, so every
    logit value occurs at a pair of vocabulary rows.  The pairs sit, by offset: among one lane's
    4 consecutive rows (1), in other lane groups (4), in a wave's other 16-row tile (16), in
    another wave (32), in another 256-row workgroup block (256, 1024).  The fused statistics must
    return the lower row of its pair, within the certified logit error of the maximum, and count
    the duplicate in the entropy."""
    from oracle.numerics import round_bf16
    from tests.parity_util import assert_entropy_close, entropy_sensitivity, entropy_tolerance
    dims = dict(n_layers=1, d=128, hq=4, hkv=2, dh=32, E=8, top_k=2, F=64, Fs=64, V=2048, C=40,
                window=0, global_every=1, eps=1e-6)
    mnp = synth.make_model(dims, seed=50 + off, norm_gain_std=0.1, lm_std=0.1)
    w = mnp["w_lm"]
    V = dims["V"]
    for v in range(V):
        if v & off:
            w[v] = w[v ^ off]
    m64 = synth.model_to_f64(mnp)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    B, T = 1, dims["C"]
    ws = driver.workspace(model.workspace_bytes(B))
    h = synth.hidden_states(T, dims["d"], seed=60 + off)
    params = osamp.default_params()
    step = 30
    out = driver.StepOut(B, dims["C"], V, DEV)
    driver.lm_head_forward(model, B, torch.from_numpy(h).to(DEV), step,
                           driver.eb_params_from_dict(params, 1), out, ws)
    torch.cuda.synchronize()
    z64 = om.linear(om.rms_norm(h.astype(np.float64), m64["final_norm"], dims["eps"]),
                    m64["w_lm"])
    zr = round_bf16(z64)
    zg = out.logits.float().cpu().numpy().reshape(T, -1)
    assert_close_rel(zg, zr, what="logits")
    # the GPU's own logits are exactly paired
    assert np.array_equal(zg[:, np.arange(V) & off == 0], zg[:, np.arange(V) & off != 0])
    ag = out.argmax.cpu().numpy().reshape(-1)
    dz = np.abs(zg - z64).max(axis=1)
    for t in range(T):
        assert ag[t] & off == 0, f"token {t}: argmax {ag[t]} is the higher row of its pair"
        assert zg[t, ag[t]] == zg[t].max(), f"token {t}: argmax is not a maximum of the logits"
        assert zr[t, ag[t]] >= zr[t].max() - 2.0 * dz[t] - 2.0 ** -7 * abs(zr[t].max())
    inv_t = osamp.inv_temperature_f32(step, params["max_steps"])
    h_ref, _ = osamp.entropy_argmax(zr, inv_t)
    tol = entropy_tolerance(h_ref, dz * float(inv_t), entropy_sensitivity(z64, inv_t))
    assert_entropy_close(out.entropy.cpu().numpy().reshape(-1), h_ref, "paired-row entropy", tol)
