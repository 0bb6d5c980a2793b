"""GPU parity of the chunked prefill (dg_kv_append_tokens).

The encoder pass over a prompt split into consecutive calls of any size must give the prompt's
one-pass causal encoding (chunk invariance, up to rounding).

Workloads:
- the 2-layer toy decoder (d 64, 4 heads of 16, 8 experts top-2 + shared, V 512): a 96-token
  prompt appended in one call and in ragged splits (40 + 56; 1 + 16 + 79), each compared layer by
  layer with the oracle's one-pass causal encoding of the whole prompt;
- a mid-width model with the decoder's attention shape per head (d 128, 4 query / 2 KV heads of
  256, 16 experts top-4 + shared): a 1,024-token prompt in one call, in four canvas-sized calls
  and in a ragged split (300 + 724), each against the oracle's one-pass encoding, with at most 1%
  of the token rows outside the tolerance (routing near-ties);
- the toy decoder with a 24-token sliding window on layer 0: 96 tokens in 4 calls of 24, against
  the oracle encoding with the same split (the window applies to cached keys only, so a windowed
  prefill depends on the split);
- two full-width layers (d 2816, 16/8 heads of 256, 128 experts top-8 + shared): a 1,024-token
  prompt on top of a 512-entry N(0,1) cache, appended in one call and in a ragged split
  (300 + 724), against four canvas appends of 256 tokens (the path the decoder tests compare with
  the oracle). Layer 0's keys and values come from the embedding, the norm and the QKV product
  alone, whose per-row arithmetic does not depend on the split, so they must agree bit for bit.
  Layer 1's depend on attention over a different key split and on the routing: they are
  compared at the stated tolerance on every token whose layer-0 expert set is the same in both
  runs (the layer chains of both runs, which write the same caches bit for bit, give the sets);
  at least 95% of the tokens must have the same set (the rest are router near-ties: a token
  whose 8th and 9th expert logits nearly tie may take a different, equally valid expert).
"""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from block_diffusion_decoding_canvas_amd._lib import DgError
from oracle import model as om
from tests.parity_util import (assert_close_rel, check_forced_routing, oracle_encode_forced,
                               prefill_chain)

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL = 2e-2


def _append_split(model, kv, prompt, split, ws):
    c0 = 0
    for n in split:
        tok = torch.tensor(prompt[None, c0:c0 + n], dtype=torch.int32, device=DEV)
        driver.kv_append_tokens(model, kv, tok, ws)
        c0 += n
    assert c0 == prompt.shape[0]


def _check_prefill(dims, mnp, model, prompt, split, cap, window_split=None):
    """Prefill the prompt with the given split twice: through dg_kv_append_tokens, and layer by
    layer (dg_layer_forward_tokens) capturing the expert sets.  The two write the same keys and
    values bit for bit; every key and value row is then compared with the oracle's encoding, the
    oracle taking the GPU's expert set at router near-ties (checked for validity)."""
    n = prompt.shape[0]
    kv = driver.KVCache(dims, 1, cap, DEV)
    ws = driver.workspace(model.append_workspace_bytes(1, max(split)))
    _append_split(model, kv, prompt, split, ws)
    kv2 = driver.KVCache(dims, 1, cap, DEV)
    idx, logits, _ = prefill_chain(dims, model, kv2, ws, prompt, split, mnp["embed"])
    torch.cuda.synchronize()
    assert kv.lengths() == kv2.lengths() == [n]
    assert torch.equal(kv.k, kv2.k) and torch.equal(kv.v, kv2.v)
    ref, infos = oracle_encode_forced(dims, mnp, prompt, cap, idx, window_split)
    swaps = [check_forced_routing(info["router_logits"], rl, ix, dims["top_k"], f"layer {l}")
             for l, (info, rl, ix) in enumerate(zip(infos, logits, idx))]
    print(f"  near-tie expert swaps per layer: {swaps}", flush=True)
    for layer in range(dims["n_layers"]):
        kg = kv.k[layer].float().cpu().numpy()[:, :, :n]
        vg = kv.v[layer].float().cpu().numpy()[:, :, :n]
        assert_close_rel(kg, ref["k"][layer][:, :, :n], what=f"K layer {layer} split {split}")
        assert_close_rel(vg, ref["v"][layer][:, :, :n], what=f"V layer {layer} split {split}")
    # nothing written past the prompt
    assert not kv.k[:, :, :, n:].any() and not kv.v[:, :, :, n:].any()
    return kv


@pytest.mark.parametrize("split", [(96,), (40, 56), (1, 16, 79)])
def test_prefill_tiny_matches_oracle(split):
    dims = synth.dims_tiny()
    mnp = synth.make_model(dims, seed=0, norm_gain_std=0.1)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    prompt = synth.prompt_ids(96, dims["V"], seed=5)
    print(f"prefill case tiny split {split}", flush=True)
    _check_prefill(dims, mnp, model, prompt, split, 128)


@pytest.fixture(scope="module")
def full_width():
    dims = synth.dims_full(n_layers=2)
    weights = synth.make_model_device(dims, DEV, seed=0)
    return dims, driver.Model(weights)


def _full_cache(dims, cap, length):
    kc, vc = synth.make_cache_device(dims, 1, cap, length, DEV, seed=1)
    return driver.KVCache(dims, 1, cap, DEV, kc, vc, [length])


def _chain_sets(dims, model, kv, ws, prompt, split):
    """The prefill of prompt into canvas 0 of kv, layer by layer through dg_layer_forward_tokens
    (the kernels and launch shapes of dg_kv_append_tokens / dg_kv_append_canvas), returning the
    layer-0 expert set of every token, sorted [n, k]."""
    embed = model.weights["embed"]
    k = dims["top_k"]
    sets, c0 = [], 0
    for n in split:
        rows = torch.tensor(prompt[c0:c0 + n], dtype=torch.int64, device=DEV)
        h = torch.index_select(embed, 0, rows).float()
        for layer in range(dims["n_layers"]):
            rl = torch.zeros((n, dims["E"]), dtype=torch.float32, device=DEV)
            ti = torch.zeros((n, k), dtype=torch.int32, device=DEV)
            driver.layer_forward_tokens(model, kv, layer, h, ws, rl, ti)
            if layer == 0:
                sets.append(np.sort(ti.cpu().numpy(), axis=1))
        kv.len[0] += n
        c0 += n
    torch.cuda.synchronize()
    return np.concatenate(sets)


@pytest.mark.parametrize("split", [(1024,), (300, 724)])
def test_prefill_full_width_chunk_invariance(full_width, split):
    """The split prefill against four canvas appends.  Layer 0's keys and values must agree bit
    for bit.  Layer 1's are compared on every token whose layer-0 expert set is the same in both
    runs (a token whose 8th and 9th router logits nearly tie may take a different expert in each
    run: a different but valid routing); those differ only by rounding."""
    dims, model = full_width
    length, n = 512, 1024
    cap = length + n
    prompt = synth.prompt_ids(n, dims["V"], seed=7)
    print(f"prefill case full width split {split}", flush=True)
    canvas_split = (dims["C"],) * (n // dims["C"])
    ref = _full_cache(dims, cap, length)
    ws_c = driver.workspace(model.workspace_bytes(1))
    for c0 in range(0, n, dims["C"]):
        driver.kv_append_canvas(model, ref, torch.tensor(prompt[None, c0:c0 + dims["C"]],
                                                         dtype=torch.int32, device=DEV), ws_c)
    got = _full_cache(dims, cap, length)
    ws = driver.workspace(model.append_workspace_bytes(1, max(split)))
    _append_split(model, got, prompt, split, ws)
    torch.cuda.synchronize()
    assert got.lengths() == ref.lengths() == [cap]
    # the layer chains of both runs write the same caches as the entry points, with their expert
    # sets
    ref_c = _full_cache(dims, cap, length)
    sets_ref = _chain_sets(dims, model, ref_c, ws, prompt, canvas_split)
    got_c = _full_cache(dims, cap, length)
    sets_got = _chain_sets(dims, model, got_c, ws, prompt, split)
    assert torch.equal(ref_c.k, ref.k) and torch.equal(ref_c.v, ref.v)
    assert torch.equal(got_c.k, got.k) and torch.equal(got_c.v, got.v)
    same = (sets_ref == sets_got).all(axis=1)
    print(f"  tokens with the same layer-0 expert set: {int(same.sum())} of {n}", flush=True)
    assert same.mean() >= 0.95
    sl = slice(length, cap)
    for name in ("k", "v"):
        a = getattr(got, name)[0][0, :, sl]
        b = getattr(ref, name)[0][0, :, sl]
        assert torch.equal(a, b), f"layer 0 {name}: split {split} differs from canvas appends"
        a = getattr(got, name)[1][0, :, sl].float().cpu().numpy().transpose(1, 0, 2)[same]
        b = getattr(ref, name)[1][0, :, sl].float().cpu().numpy().transpose(1, 0, 2)[same]
        assert_close_rel(a.reshape(a.shape[0], -1), b.reshape(b.shape[0], -1),
                         what=f"layer 1 {name} split {split} (same expert sets)")


def test_prefill_errors_leave_cache_untouched(full_width):
    dims, model = full_width
    kv = _full_cache(dims, 600, 512)
    ws = driver.workspace(model.append_workspace_bytes(1, 64))
    tok = torch.zeros((1, 100), dtype=torch.int32, device=DEV)
    with pytest.raises(DgError):
        driver.kv_append_tokens(model, kv, tok, ws)         # 512 + 100 > cap 600
    with pytest.raises(DgError):
        driver.kv_append_tokens(model, kv, tok[:, :80], ws)  # workspace sized for 64 tokens
    assert kv.lengths() == [512]
    driver.kv_append_tokens(model, kv, tok[:, :64], ws)
    torch.cuda.synchronize()
    assert kv.lengths() == [576]


def _mid_dims():
    # head_dim 256 (the decoder's attention configuration), small width otherwise
    return dict(n_layers=2, d=128, hq=4, hkv=2, dh=256, E=16, top_k=4, F=128, Fs=128, V=512,
                C=256, window=0, global_every=1, eps=1e-6)


@pytest.mark.parametrize("split", [(1024,), (256, 256, 256, 256), (300, 724)])
def test_prefill_mid_width_matches_oracle(split):
    dims = _mid_dims()
    mnp = synth.make_model(dims, seed=0, norm_gain_std=0.1)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    prompt = synth.prompt_ids(1024, dims["V"], seed=9)
    print(f"prefill case mid width split {split}", flush=True)
    _check_prefill(dims, mnp, model, prompt, split, 1024)


@pytest.mark.parametrize("split", [(24, 24, 24, 24), (8, 16, 24, 24, 24)])
def test_prefill_windowed_chunk_invariance(split):
    """Sliding-window layers.  A call holds at most `window` new tokens, so every earlier new
    token of the call is less than `window` positions back, and cached keys are windowed: any such
    split encodes each token over exactly the keys less than `window` positions back, the plain
    causal sliding-window rule, whatever the split.  Layer 0 keeps a 24-token window, layer 1 is
    global; 96 tokens in two different splits, each compared with the oracle (which encodes in
    the same calls) and with each other.  The oracle's one-pass encoding of all 96 tokens would
    let the first layer see every earlier new token, past the window, so it is not the
    reference here."""
    dims = dict(synth.dims_tiny(), window=24, global_every=2)
    mnp = synth.make_model(dims, seed=3, norm_gain_std=0.1)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    prompt = synth.prompt_ids(96, dims["V"], seed=11)
    print(f"prefill case windowed tiny, split {split}", flush=True)
    kv = _check_prefill(dims, mnp, model, prompt, split, 128, window_split=split)
    other = (24, 24, 24, 24) if split != (24, 24, 24, 24) else (8, 16, 24, 24, 24)
    kv_o = driver.KVCache(dims, 1, 128, DEV)
    ws = driver.workspace(model.append_workspace_bytes(1, 24))
    _append_split(model, kv_o, prompt, other, ws)
    torch.cuda.synchronize()
    for layer in range(dims["n_layers"]):
        assert_close_rel(kv.k[layer].float().cpu().numpy()[:, :, :96],
                         kv_o.k[layer].float().cpu().numpy()[:, :, :96].astype(np.float64),
                         what=f"K layer {layer}: split {split} against {other}")
        assert_close_rel(kv.v[layer].float().cpu().numpy()[:, :, :96],
                         kv_o.v[layer].float().cpu().numpy()[:, :, :96].astype(np.float64),
                         what=f"V layer {layer}: split {split} against {other}")


BENCH_ROWS = np.array([0, 1, 2, 63, 64, 127, 128, 511, 1000, 1023, 1024, 1535, 1536, 2000,
                       2046, 2047])


def test_prefill_bench_chunk_matches_oracle():
    """The benchmark's prefill configuration: a 2,048-token call on the full-width layers
    (d 2816, 16/8 heads of 256, 128 experts top-8 + shared; 128-row expert tiles on 8 waves,
    128-token QKV tiles, 64-token router tiles), appended after 2,048 cached N(0,1) entries.
    Layer 0's keys and values (every row) and the GPU's residual stream after layer 0 and layer
    1's keys and values (sampled rows) against the oracle, which takes the GPU's expert set at
    router near-ties; rows are independent given the keys and values they attend to, so the
    oracle computes layer 0's keys for every row and the rest for the sampled rows only."""
    dims = synth.dims_full(n_layers=2, vocab=4096)
    mnp = synth.make_model(dims, seed=0, norm_gain_std=0.1)
    L0, n = 2048, 2048
    cap = L0 + n
    cache = synth.make_cache(dims, 1, cap, L0, seed=1)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    prompt = synth.prompt_ids(n, dims["V"], seed=13)
    print("prefill case full width, one 2,048-token call after 2,048 cached entries", flush=True)
    kv = driver.KVCache.from_host(dims, cache, cap, DEV)
    ws = driver.workspace(model.append_workspace_bytes(1, n))
    _append_split(model, kv, prompt, (n,), ws)
    kv2 = driver.KVCache.from_host(dims, cache, cap, DEV)
    idx, logits, h_after0 = prefill_chain(dims, model, kv2, ws, prompt, (n,), mnp["embed"])
    torch.cuda.synchronize()
    assert kv.lengths() == kv2.lengths() == [cap]
    assert torch.equal(kv.k, kv2.k) and torch.equal(kv.v, kv2.v)
    m64 = synth.model_to_f64(mnp)
    lw0, lw1 = m64["layers"]
    kc = [a[0].astype(np.float64) for a in cache["k"]]        # [Hkv, cap, dh] per layer
    vc = [a[0].astype(np.float64) for a in cache["v"]]
    # layer 0: every new key and value (per-row functions of the embedding)
    h0 = m64["embed"][prompt]
    q0, k0, v0 = om.split_qkv(om.rms_norm(h0, lw0["attn_norm"], dims["eps"]) @ lw0["w_qkv"].T,
                              dims)
    assert_close_rel(kv.k[0, 0, :, L0:].float().cpu().numpy(), k0.transpose(1, 0, 2),
                     what="layer 0 K (all rows)")
    assert_close_rel(kv.v[0, 0, :, L0:].float().cpu().numpy(), v0.transpose(1, 0, 2),
                     what="layer 0 V (all rows)")
    # layer 0 at the sampled rows: causal attention over the cache and the earlier new tokens,
    # O projection, the FFN with the GPU's expert sets
    R = BENCH_ROWS
    o = om.attention(q0[R], kc[0][:, :L0], vc[0][:, :L0], k0, v0, np.ones((len(R), L0), bool),
                     True, q_pos=R)
    h_mid = h0[R] + o.reshape(len(R), -1) @ lw0["w_o"].T
    f, info = om.moe(om.rms_norm(h_mid, lw0["ffn_norm"], dims["eps"]), lw0, dims["top_k"],
                     force_idx=idx[0][0, R])
    swaps = check_forced_routing(info["router_logits"], logits[0][R], idx[0][0, R],
                                 dims["top_k"], "layer 0 (sampled rows)")
    h1 = h_mid + f
    assert_close_rel(h_after0[R] - h0[R], h1 - h0[R], what="layer 0 increment (sampled rows)")
    # layer 1's keys and values at the sampled rows
    _, k1, v1 = om.split_qkv(om.rms_norm(h1, lw1["attn_norm"], dims["eps"]) @ lw1["w_qkv"].T,
                             dims)
    assert_close_rel(kv.k[1, 0, :, L0 + R].float().cpu().numpy(), k1.transpose(1, 0, 2),
                     what="layer 1 K (sampled rows)")
    assert_close_rel(kv.v[1, 0, :, L0 + R].float().cpu().numpy(), v1.transpose(1, 0, 2),
                     what="layer 1 V (sampled rows)")
    print(f"  bench chunk: near-tie expert swaps at the sampled rows {swaps}/{len(R)}")
