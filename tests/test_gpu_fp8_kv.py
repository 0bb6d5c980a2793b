"""GPU parity of the fp8 (e4m3) KV cache: attention over e4m3 cache rows and e4m3 canvas rows,
with the query rows quantised the same way (QK^T on the e4m3 MFMA, P V on the bf16 one), and the
encoder pass storing its quantised key and value rows.

Workloads (caches: random e4m3 codes with fp32 row scales, drawn as codes by the synthetic-input
module):
- one layer at head_dim 128 and 256 (4 query / 2 KV heads, 2 canvases of 40 positions, cache
  lengths 700 / 333: 12 and 6 key tiles of 64 ending ragged, so the key range is split and merged)
  in the three attention modes: global bidirectional, a 48-position sliding window, and causal
  canvas keys (the encoder pass, whose cache rows [len, len + C) are compared too);
- the same layer over the largest canvas the C ABI accepts (1,024 positions), global and causal,
  on caches of 300 entries and of none;
- a 2-layer model with head_dim 128: a 40-token prompt prefilled into an empty fp8 cache in two
  calls (16 + 24), then one decoder step over a 16-position canvas, against the oracle's encoding
  and decoder pass (the oracle takes the GPU's expert sets at router near-ties).

Both sides quantise in binary32 with the same rule from the bf16 QKV product of the bf16 normed
input, so a code differs only where the two sides' bf16 values differ at an e4m3 rounding
boundary: from identical layer inputs, cache rows (compared as codes times scales) are held to the
stated tolerance with at least 99% of the values identical.  After a layer whose outputs differ by
rounding, the e4m3 codes of the next layer flip where those differences cross a rounding
boundary, so the chained prefill and the decoder logits are held to the chained e4m3 bound.
"""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from oracle import model as om
from oracle.numerics import e4m3_value
from tests.parity_util import (FP8_CHAIN_ARRAY_TOL, FP8_CHAIN_TOL, REL_TOL, GpuChain,
                               assert_close_rel, check_forced_routing, oracle_encode_forced,
                               prefill_chain)

pytestmark = pytest.mark.gpu
DEV = "cuda"
E4M3_TABLE = e4m3_value(np.arange(256))


def decode(codes, scales):
    """Values of e4m3 rows: codes [..., dh] times their row scales [...], as float64."""
    return E4M3_TABLE[np.asarray(codes)] * np.asarray(scales, dtype=np.float64)[..., None]


def oracle_cache(cache):
    return dict(k=[decode(c, s) for c, s in zip(cache["k"], cache["k_scale"])],
                v=[decode(c, s) for c, s in zip(cache["v"], cache["v_scale"])],
                len=np.array(cache["len"]))


def compare_rows(kv, layer, ref_k, ref_v, rows, what, rel=REL_TOL, min_same=0.99):
    """GPU cache rows [lo_b, lo_b + n) of every canvas against the oracle's values
    ref_k/ref_v [B, Hkv, n, dh] (rel: row tolerance; min_same: least fraction of identical
    values); rows: (lo_b per canvas, n)."""
    lo, n = rows
    same = total = 0
    for name, ref, codes, sc in (("k", ref_k, kv.k, kv.k_scale), ("v", ref_v, kv.v, kv.v_scale)):
        for b, l0 in enumerate(lo):
            c = codes[layer, b, :, l0:l0 + n].cpu().numpy()
            s = sc[layer, b, :, l0:l0 + n].cpu().numpy()
            assert_close_rel(decode(c, s), ref[b], rel=rel, what=f"{what} cache {name} canvas {b}")
            eq = decode(c, s) == ref[b]
            same += int(eq.sum())
            total += eq.size
    assert same >= min_same * total, f"{what}: only {same}/{total} cached values identical"
    return same, total


@pytest.mark.parametrize("mode", ["global", "window", "causal"])
@pytest.mark.parametrize("dh", [128, 256])
def test_fp8_kv_layer(dh, mode):
    _fp8_layer_case(dh, mode, (700, 333), 760)


@pytest.mark.parametrize("mode", ["global", "window", "causal"])
def test_fp8_kv_layer_short_and_empty_cache(mode):
    """Head_dim 256 on a 20-entry cache (the 48-position window then starts at position 0) and
    an empty one (canvas keys only)."""
    _fp8_layer_case(256, mode, (20, 0), 64)


@pytest.mark.parametrize("mode", ["global", "causal"])
@pytest.mark.parametrize("dh", [128, 256])
def test_fp8_kv_layer_canvas_1024(dh, mode):
    """The largest canvas the C ABI accepts (1,024 positions: 32 canvas key tiles, and in causal
    mode a canvas mask that ends in a different tile for each query block) on e4m3 caches of
    300 entries and of none, decoder and encoder pass."""
    _fp8_layer_case(dh, mode, (300, 0), 1400, C=1024)


def _fp8_layer_case(dh, mode, lens, cap, C=40):
    window = 48 if mode == "window" else 0
    causal = 1 if mode == "causal" else 0
    dims = dict(n_layers=1, d=64, hq=4, hkv=2, dh=dh, E=8, top_k=2, F=64, Fs=64, V=256, C=C,
                window=window, global_every=2, eps=1e-6, kv_dtype="e4m3")
    rng = np.random.default_rng(41 + dh)
    mnp = dict(dims=dims, layers=[synth.make_layer(dims, rng, norm_gain_std=0.1)],
               embed=np.zeros((256, 64), np.float32), final_norm=np.ones(64, np.float32),
               w_lm=np.zeros((256, 64), np.float32))
    mnp["layers"][0]["w_qkv"] = mnp["layers"][0]["w_qkv"] * 4    # score std about 2
    B, C = len(lens), dims["C"]
    cache = synth.make_cache_fp8(dims, B, cap, max(lens), seed=42)
    cache["len"] = np.array(lens, dtype=np.int64)
    T = B * C
    h = synth.hidden_states(T, 64, seed=43)
    print(f"fp8 kv case dh={dh} mode={mode} lens={lens} C={C}", flush=True)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    kv = driver.KVCache.from_host(dims, cache, cap, DEV)
    ws = driver.workspace(model.workspace_bytes(B))
    hg = torch.from_numpy(h.astype(np.float32)).to(DEV)
    rl = torch.zeros((T, 8), dtype=torch.float32, device=DEV)
    ti = torch.zeros((T, 2), dtype=torch.int32, device=DEV)
    driver.layer_forward(model, kv, 0, causal, hg, ws, rl, ti, None)
    torch.cuda.synchronize()
    lw = synth.model_to_f64(mnp)["layers"][0]
    c64 = oracle_cache(cache)
    args = (h.astype(np.float64).reshape(B, C, 64), lw, dims, 0, c64["k"][0], c64["v"][0],
            np.array(lens))
    _, _, _, info = om.layer_forward(*args, causal=bool(causal))
    rg = rl.cpu().numpy()
    assert_close_rel(rg, info["router_logits"].reshape(T, -1), what=f"router logits dh={dh} {mode}")
    tig = ti.cpu().numpy().astype(np.int64)
    check_forced_routing(info["router_logits"].reshape(T, -1), rg, tig, 2, f"dh={dh} {mode}")
    h_ref, k_ref, v_ref, _ = om.layer_forward(*args, causal=bool(causal),
                                              force_idx=tig.reshape(B, C, 2))
    assert_close_rel(hg.cpu().numpy() - h, h_ref.reshape(T, 64) - h,
                     what=f"fp8 kv layer increment dh={dh} {mode}")
    if causal:
        same, total = compare_rows(kv, 0, k_ref.transpose(0, 2, 1, 3), v_ref.transpose(0, 2, 1, 3),
                                   (lens, C), f"dh={dh} append")
        print(f"  appended rows: {same}/{total} values identical", flush=True)
    # rows before len are never written
    assert np.array_equal(kv.k[0, 0, :, :lens[0]].cpu().numpy(), cache["k"][0][0, :, :lens[0]])


def test_fp8_kv_prefill_then_decode():
    dims = dict(n_layers=2, d=64, hq=4, hkv=2, dh=128, E=8, top_k=2, F=128, Fs=128, V=512, C=16,
                window=0, global_every=1, eps=1e-6, kv_dtype="e4m3")
    mnp = synth.make_model(dims, seed=7, norm_gain_std=0.1, lm_std=1.0)
    for lw in mnp["layers"]:
        lw["w_qkv"] = lw["w_qkv"] * 4
    m64 = synth.model_to_f64(mnp)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    cap, n_prompt = 64, 40
    prompt = synth.prompt_ids(n_prompt, dims["V"], seed=8)
    kv = driver.KVCache(dims, 1, cap, DEV)
    ws = driver.workspace(max(model.workspace_bytes(1), model.append_workspace_bytes(1, 24)))
    print("fp8 kv prefill 16 + 24", flush=True)
    idx, logits, _ = prefill_chain(dims, model, kv, ws, prompt, (16, 24), mnp["embed"])
    assert kv.lengths() == [n_prompt]
    # the oracle's encoding of the prompt (one pass: a causal prefill does not depend on the
    # split), with the GPU's expert sets where they are valid near-ties
    ref, infos = oracle_encode_forced(dims, mnp, prompt, cap, idx)
    for l, (info, rl, ix) in enumerate(zip(infos, logits, idx)):
        check_forced_routing(info["router_logits"], rl, ix, dims["top_k"], f"prefill layer {l}")
    # layer 0's rows come from identical inputs (the embedding rows); layer 1's from residual
    # streams that differ by layer 0's rounding, so their codes flip where those differences
    # cross a rounding boundary (the chained e4m3 bound)
    same, total = compare_rows(kv, 0, ref["k"][0][:, :, :n_prompt], ref["v"][0][:, :, :n_prompt],
                               ([0], n_prompt), "prefill layer 0")
    print(f"prefill layer 0: {same}/{total} cached values identical", flush=True)
    same, total = compare_rows(kv, 1, ref["k"][1][:, :, :n_prompt], ref["v"][1][:, :, :n_prompt],
                               ([0], n_prompt), "prefill layer 1", rel=FP8_CHAIN_TOL, min_same=0.5)
    print(f"prefill layer 1: {same}/{total} cached values identical", flush=True)
    # one decoder step over a canvas, against the oracle on its own cache
    canvas = synth.prompt_ids(dims["C"], dims["V"], seed=9)[None]
    chain = GpuChain(dims, model, kv, ws, canvas, mnp["embed"])
    zr, _, infos = om.decoder_forward(canvas, m64, ref, force_idx=chain.idx)
    chain.check(infos, dims["top_k"], "fp8 kv decode")
    st = driver.SamplerState(1, dims["C"], DEV)
    st.canvas.copy_(torch.from_numpy(canvas.astype(np.int32)))
    out = driver.StepOut(1, dims["C"], dims["V"], DEV)
    driver.decoder_step(model, kv, 0, driver.eb_params(), st, out, ws)
    torch.cuda.synchronize()
    zg = out.logits.float().cpu().numpy()
    rel = np.linalg.norm(zg - zr, axis=-1) / np.linalg.norm(zr, axis=-1)
    print(f"fp8 kv decoder logits: worst row rel err {rel.max():.2e}, median {np.median(rel):.2e}",
          flush=True)
    assert_close_rel(zg, zr, rel=FP8_CHAIN_TOL, what="fp8 kv decoder logits")
    assert np.linalg.norm(zg - zr) <= FP8_CHAIN_ARRAY_TOL * np.linalg.norm(zr)


# --- full size: the long-context configuration's attention shapes -------------------------------
LENS = (131072, 131072, 130001, 100003)
ROWS = np.array([0, 1, 37, 100, 127, 128, 200, 255])      # sampled canvas positions


@pytest.fixture(scope="module")
def full_case():
    """Two full-width layers (d 2816, 16/8 heads of 256, 128 experts top-8 + shared) with an e4m3
    cache: layer 0 sliding-window (1,024), layer 1 global; 4 canvases of 256 on caches of LENS."""
    dims = synth.dims_full(n_layers=2)
    dims.update(window=1024, global_every=2, kv_dtype="e4m3")
    B, C = len(LENS), dims["C"]
    cap = max(LENS) + C
    w = synth.make_model_device(dims, DEV, seed=15)
    # the oracle's copy first: the model repacks its matrices in place
    lws = [{kk: vv.float().cpu().numpy().astype(np.float64) for kk, vv in lw.items()}
           for lw in w["layers"]]
    model = driver.Model(w)
    k, v, ks, vs = synth.make_cache_fp8_device(dims, B, cap, max(LENS), DEV, seed=16)
    for b, n in enumerate(LENS):
        for t in (k, v):
            t[:, b, :, n:] = 0
        for t in (ks, vs):
            t[:, b, :, n:] = 1
    kv = driver.KVCache(dims, B, cap, DEV, k, v, LENS, ks, vs)
    ws = driver.workspace(model.workspace_bytes(B))
    h = synth.hidden_states(B * C, dims["d"], seed=17)
    torch.cuda.synchronize()
    print("full-size fp8 kv case ready", flush=True)
    return dict(dims=dims, B=B, C=C, model=model, kv=kv, ws=ws, h=h, lws=lws)


def _cache_rows(kv, layer, b, lo, hi):
    """The oracle's copy of cache rows [lo, hi) of canvas b: codes times scales (float64)."""
    return (decode(kv.k[layer, b, :, lo:hi].cpu().numpy(), kv.k_scale[layer, b, :, lo:hi].cpu().numpy()),
            decode(kv.v[layer, b, :, lo:hi].cpu().numpy(), kv.v_scale[layer, b, :, lo:hi].cpu().numpy()))


@pytest.mark.parametrize("layer", [0, 1])
def test_fp8_kv_full_size_layer(full_case, layer):
    """One layer over the 4 canvases (the launch shapes of the long-context decoder step), from
    the same hidden states on both sides, compared on the sampled rows of every canvas: router
    logits, then the layer increment with the oracle taking the GPU's expert sets at near-ties.
    A windowed query sees only the last window - 1 cache positions, so the oracle gets those."""
    c = full_case
    d, B, C = c["dims"], c["B"], c["C"]
    T, E, k = B * C, d["E"], d["top_k"]
    print(f"full-size fp8 kv layer {layer} ({'global' if layer else 'windowed'})", flush=True)
    hg = torch.from_numpy(c["h"].astype(np.float32)).to(DEV)
    rl = torch.zeros((T, E), dtype=torch.float32, device=DEV)
    ti = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    driver.layer_forward(c["model"], c["kv"], layer, 0, hg, c["ws"], rl, ti, None)
    torch.cuda.synchronize()
    sel = (np.arange(B)[:, None] * C + ROWS[None, :]).reshape(-1)
    h64 = c["h"].astype(np.float64).reshape(B, C, -1)
    lw = c["lws"][layer]
    mids = []
    for b, n in enumerate(LENS):
        lo = n - d["window"] + 1 if layer == 0 else 0
        kc, vc = _cache_rows(c["kv"], layer, b, lo, n)
        mid, _, _ = om.attention_block(h64[b:b + 1], lw, d, layer, kc[None], vc[None],
                                       np.array([n - lo]), False, rows=ROWS)
        mids.append(mid)
        del kc, vc
        print(f"  oracle attention canvas {b} ({n - lo} cached keys)", flush=True)
    h_mid = np.concatenate(mids)                             # [B, R, d]
    _, info = om.ffn_block(h_mid, lw, d)
    rg = rl.cpu().numpy()[sel]
    r_ref = info["router_logits"].reshape(len(sel), -1)
    assert_close_rel(rg, r_ref, what=f"router logits layer {layer} (sampled rows)")
    tig = ti.cpu().numpy().astype(np.int64)[sel]
    swaps = check_forced_routing(r_ref, rg, tig, k, f"full-size layer {layer}")
    h_out, _ = om.ffn_block(h_mid, lw, d, tig.reshape(B, len(ROWS), k))
    inc_g = hg.cpu().numpy().astype(np.float64)[sel] - h64.reshape(T, -1)[sel]
    inc_r = (h_out - h64[:, ROWS]).reshape(len(sel), -1)
    assert_close_rel(inc_g, inc_r, what=f"fp8 kv layer {layer} increment (sampled rows)")
    print(f"  sampled rows {len(sel)}, near-tie expert swaps {swaps}", flush=True)


# --- the generation loop on an e4m3 cache -----------------------------------------------------
def _fp8_toy(B):
    """A 2-layer model with head_dim 128 and a sharp LM head (commits and adaptive stops within
    a few steps) on an e4m3 cache that a chunked prefill fills with a 32-token prompt each."""
    dims = dict(n_layers=2, d=64, hq=4, hkv=2, dh=128, E=8, top_k=2, F=128, Fs=128, V=512, C=16,
                window=0, global_every=1, eps=1e-6, kv_dtype="e4m3")
    mnp = synth.make_model(dims, seed=11, norm_gain_std=0.1, lm_std=1.0)
    for lw in mnp["layers"]:
        lw["w_qkv"] = lw["w_qkv"] * 4
    model = driver.Model(synth.model_to_device(mnp, DEV))
    prompt = np.stack([synth.prompt_ids(32, dims["V"], seed=20 + b) for b in range(B)])
    kv = driver.KVCache(dims, B, 128, DEV)
    ws = driver.workspace(model.append_workspace_bytes(B, 32))
    driver.kv_append_tokens(model, kv, torch.tensor(prompt, dtype=torch.int32, device=DEV), ws)
    torch.cuda.synchronize()
    return dims, model, kv


@pytest.mark.parametrize("kind", ["entropy_bound", "discrete_ddim"])
def test_fp8_kv_generate_compacted_matches_uncompacted(kind):
    """dg_generate on an e4m3 cache, with and without frozen-canvas compaction: tokens, canvases,
    steps per canvas and the cache (codes and scales) bit for bit."""
    B = 3
    p = driver.sched_params(kind, max_steps=10, seed=9, temperature=0.7, corrector_steps=2,
                            corrector_k=3)
    res = []
    for compact in (False, True):
        dims, model, kv = _fp8_toy(B)
        st = driver.SamplerState(B, dims["C"], DEV)
        out = driver.StepOut(B, dims["C"], dims["V"], DEV)
        print(f"fp8 kv generate {kind} compact={compact}", flush=True)
        tokens, n, steps = driver.generate(model, kv, p, st, out, 3 * dims["C"],
                                           compact_frozen=compact)
        torch.cuda.synchronize()
        res.append((tokens.cpu().numpy(), n, steps, kv.k.clone(), kv.v.clone(),
                    kv.k_scale.clone(), kv.v_scale.clone(), kv.lengths()))
    a, b = res
    assert np.array_equal(a[0], b[0]) and a[1] == b[1] and a[2] == b[2]
    for x, y in zip(a[3:7], b[3:7]):
        assert torch.equal(x, y)
    assert a[7] == b[7] == [32 + a[1] * 16] * B
    print(f"  {a[1]} canvases, steps {a[2]}", flush=True)


def test_fp8_kv_generate_matches_python_loop():
    """dg_generate on an e4m3 cache against the same loop over the step calls (canvas init,
    decoder steps until every canvas is done, the append), bit for bit."""
    B = 2
    dims, model, kv = _fp8_toy(B)
    _, _, kv2 = _fp8_toy(B)
    p = driver.eb_params(max_steps=8, seed=3)
    st = driver.SamplerState(B, dims["C"], DEV)
    out = driver.StepOut(B, dims["C"], dims["V"], DEV)
    tok, n, steps = driver.generate(model, kv, p, st, out, 2 * dims["C"])
    torch.cuda.synchronize()
    ws = driver.workspace(model.workspace_bytes(B))
    ref, ref_steps = [], []
    for c in range(2):
        s2 = driver.SamplerState(B, dims["C"], DEV, canvas_ids=[c * B + b for b in range(B)])
        driver.canvas_init(p, s2, dims["V"])
        k = 0
        for s in range(8):
            driver.decoder_step(model, kv2, s, p, s2, out, ws)
            k += 1
            if bool(s2.done.all()):
                break
        driver.kv_append_canvas(model, kv2, s2.canvas, ws)
        ref.append(s2.canvas.cpu().numpy())
        ref_steps.append(k)
    torch.cuda.synchronize()
    assert n == 2 and steps == ref_steps
    assert np.array_equal(tok.cpu().numpy(), np.concatenate(ref, axis=1))
    for x, y in ((kv.k, kv2.k), (kv.v, kv2.v), (kv.k_scale, kv2.k_scale), (kv.v_scale, kv2.v_scale)):
        assert torch.equal(x, y)


def test_fp8_kv_compacted_steps_bit_identical_with_staggered_freezes():
    """dg_decoder_step_live over the live canvases only, on an e4m3 cache, against the full
    step: state and live outputs bit for bit while the canvases freeze at different steps (a
    loose entropy bound and adaptive stop make them freeze early)."""
    B = 3
    dims, model, kv = _fp8_toy(B)
    C, V = dims["C"], dims["V"]
    kv.len[1] = 20   # different visible cache lengths per canvas
    kv.len[2] = 27
    ws = driver.workspace(model.workspace_bytes(B))
    p = driver.sched_params("entropy_bound", max_steps=16, seed=4, entropy_bound=4.0,
                            stop_entropy=0.5)
    full, comp = (driver.SamplerState(B, C, DEV, canvas_ids=[5, 1, 9]) for _ in range(2))
    driver.canvas_init(driver.eb_params(seed=4), full, V)
    driver.canvas_init(driver.eb_params(seed=4), comp, V)
    of, oc = driver.StepOut(B, C, V, DEV), driver.StepOut(B, C, V, DEV)
    staggered = False
    for s in range(16):
        live = [b for b in range(B) if not bool(comp.done[b])]
        if not live:
            break
        staggered |= 0 < len(live) < B
        print(f"fp8 kv compaction step {s}: live canvases {live}", flush=True)
        driver.decoder_step_sched(model, kv, s, p, full, of, ws)
        driver.decoder_step_live(model, kv, s, p, comp, oc, live, ws)
        torch.cuda.synchronize()
        hf, hc = full.host(), comp.host()
        for k in hf:
            assert np.array_equal(hf[k], hc[k]), k
        for b in live:
            assert torch.equal(of.logits[b], oc.logits[b])
            assert torch.equal(of.entropy[b], oc.entropy[b])
    assert staggered, "the canvases froze together: the workload does not stagger"


def test_fp8_kv_decoder_step_and_append_under_graph_capture():
    """A decoder step and a canvas append on an e4m3 cache enqueue kernels only (the canvas rows'
    quantiser included): each call captured in a HIP graph and replayed 3 times from the same
    state, with eager work between the replays, reproduces the eager call bit for bit."""
    from tests.test_gpu_graph import _check_replays
    B = 2
    dims, model, kv = _fp8_toy(B)
    C, V = dims["C"], dims["V"]
    ws = driver.workspace(model.workspace_bytes(B))
    p = driver.eb_params(max_steps=8, seed=5)
    st = driver.SamplerState(B, C, DEV)
    driver.canvas_init(p, st, V)
    out = driver.StepOut(B, C, V, DEV)
    for s in (0, 5):
        print(f"fp8 kv graph: decoder step {s}", flush=True)
        _check_replays(lambda: driver.decoder_step(model, kv, s, p, st, out, ws), st, out,
                       f"fp8 kv step {s}")
    # the append: the cache rows it writes, replayed from the same lengths
    tokens = st.canvas.clone()
    n0 = kv.lengths()
    eager = None
    for r in range(4):
        for b in range(B):
            kv.len[b] = n0[b]
        if r == 0:
            driver.kv_append_canvas(model, kv, tokens, ws)
            torch.cuda.synchronize()
            eager = [t.clone() for t in (kv.k, kv.v, kv.k_scale, kv.v_scale)]
            for t in (kv.k, kv.v):
                t[:, :, :, n0[0]:].zero_()
            continue
        if r == 1:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                driver.kv_append_canvas(model, kv, tokens, ws)
            for b in range(B):
                kv.len[b] = n0[b]
        for t in (kv.k, kv.v):
            t[:, :, :, n0[0]:].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, e in zip((kv.k, kv.v, kv.k_scale, kv.v_scale), eager):
            assert torch.equal(a, e), f"append replay {r}"
    del g
