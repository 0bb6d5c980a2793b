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
  Layer 1's depend on attention over a different key split and on the routing. Both runs carry
  their own rounding (each about 0.4% from fp64), so they are compared per token row: the
  relative norm of a row's difference must be within the tolerance for at least 95% of the rows
  (the rest are routing near-ties, measured at about 2%: a token whose 8th and 9th expert logits
  nearly tie may take a different expert in each run), and over all rows.
"""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from block_diffusion_decoding_canvas_amd._lib import DgError
from oracle import model as om
from tests.parity_util import assert_close_rel

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


@pytest.mark.parametrize("split", [(96,), (40, 56), (1, 16, 79)])
def test_prefill_tiny_matches_oracle(split):
    dims = synth.dims_tiny()
    mnp = synth.make_model(dims, seed=0, norm_gain_std=0.1)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    prompt = synth.prompt_ids(96, dims["V"], seed=5)
    cap = 128
    kv = driver.KVCache(dims, 1, cap, DEV)
    ws = driver.workspace(model.append_workspace_bytes(1, max(split)))
    print(f"prefill case tiny split {split}", flush=True)
    _append_split(model, kv, prompt, split, ws)
    torch.cuda.synchronize()
    assert kv.lengths() == [96]
    ref = synth.empty_cache(dims, 1, cap)
    ref = dict(k=[a.astype(np.float64) for a in ref["k"]], v=[a.astype(np.float64) for a in ref["v"]],
               len=np.array(ref["len"]))
    om.encoder_append(prompt[None], synth.model_to_f64(mnp), ref)
    for layer in range(dims["n_layers"]):
        kg = kv.k[layer].float().cpu().numpy()[:, :, :96]
        vg = kv.v[layer].float().cpu().numpy()[:, :, :96]
        assert_close_rel(kg, ref["k"][layer][:, :, :96], what=f"K layer {layer} split {split}")
        assert_close_rel(vg, ref["v"][layer][:, :, :96], what=f"V layer {layer} split {split}")
    # nothing written past the prompt
    assert not kv.k[:, :, :, 96:].any() and not kv.v[:, :, :, 96:].any()


@pytest.fixture(scope="module")
def full_width():
    dims = synth.dims_full(n_layers=2)
    weights = synth.make_model_device(dims, DEV, seed=0)
    return dims, driver.Model(weights)


def _full_cache(dims, cap, length):
    kc, vc = synth.make_cache_device(dims, 1, cap, length, DEV, seed=1)
    return driver.KVCache(dims, 1, cap, DEV, kc, vc, [length])


@pytest.mark.parametrize("split", [(1024,), (300, 724)])
def test_prefill_full_width_chunk_invariance(full_width, split):
    dims, model = full_width
    length, n = 512, 1024
    cap = length + n
    prompt = synth.prompt_ids(n, dims["V"], seed=7)
    print(f"prefill case full width split {split}", flush=True)
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
    sl = slice(length, cap)
    for name in ("k", "v"):
        a = getattr(got, name)[0][0, :, sl]
        b = getattr(ref, name)[0][0, :, sl]
        assert torch.equal(a, b), f"layer 0 {name}: split {split} differs from canvas appends"
        a = getattr(got, name)[1][0, :, sl].float().cpu().numpy()      # [Hkv, n, dh]
        b = getattr(ref, name)[1][0, :, sl].float().cpu().numpy()
        rel = np.linalg.norm(a - b) / np.linalg.norm(b)
        assert rel <= REL, f"layer 1 {name}: relative norm {rel:.3g}"
        da = (a - b).transpose(1, 0, 2).reshape(n, -1)
        row_rel = np.linalg.norm(da, axis=1) / np.linalg.norm(b.transpose(1, 0, 2).reshape(n, -1),
                                                               axis=1)
        ok = row_rel <= REL
        assert ok.mean() >= 0.95, f"layer 1 {name}: {int((~ok).sum())} of {n} token rows differ"


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
    n, cap = 1024, 1024
    prompt = synth.prompt_ids(n, dims["V"], seed=9)
    kv = driver.KVCache(dims, 1, cap, DEV)
    ws = driver.workspace(model.append_workspace_bytes(1, max(split)))
    print(f"prefill case mid width split {split}", flush=True)
    _append_split(model, kv, prompt, split, ws)
    torch.cuda.synchronize()
    ref = synth.empty_cache(dims, 1, cap)
    ref = dict(k=[a.astype(np.float64) for a in ref["k"]], v=[a.astype(np.float64) for a in ref["v"]],
               len=np.array(ref["len"]))
    om.encoder_append(prompt[None], synth.model_to_f64(mnp), ref)
    for layer in range(dims["n_layers"]):
        for name in ("k", "v"):
            a = getattr(kv, name)[layer].float().cpu().numpy()[0]       # [Hkv, n, dh]
            b = ref[name][layer][0]
            rms = np.sqrt(np.mean(b * b))
            ok = (np.abs(a - b) <= REL * np.abs(b) + REL * rms).all(axis=(0, 2))
            rel = np.linalg.norm(a - b) / np.linalg.norm(b)
            bad = np.nonzero(~ok)[0]
            print(f"  layer {layer} {name}: rel {rel:.3g}, bad rows {bad.size}: {bad[:12]}",
                  flush=True)
            assert rel <= REL and ok.mean() >= 0.99, f"layer {layer} {name} split {split}"


def test_prefill_windowed_matches_oracle_chunk_by_chunk():
    """Sliding-window layers: with the window on cached keys only (the canvas, here the new
    tokens, is always fully visible), a windowed prefill depends on the split, so the oracle
    encodes with the same split.  Layer 0 keeps a 24-token window, layer 1 is global; 96 tokens
    in 4 calls of 24, so from the second call on the window cuts into earlier calls' keys."""
    dims = dict(synth.dims_tiny(), window=24, global_every=2)
    mnp = synth.make_model(dims, seed=3, norm_gain_std=0.1)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    prompt = synth.prompt_ids(96, dims["V"], seed=11)
    cap, split = 128, (24, 24, 24, 24)
    kv = driver.KVCache(dims, 1, cap, DEV)
    ws = driver.workspace(model.append_workspace_bytes(1, 24))
    print("prefill case windowed tiny, 4 x 24", flush=True)
    _append_split(model, kv, prompt, split, ws)
    torch.cuda.synchronize()
    ref = synth.empty_cache(dims, 1, cap)
    ref = dict(k=[a.astype(np.float64) for a in ref["k"]], v=[a.astype(np.float64) for a in ref["v"]],
               len=np.array(ref["len"]))
    m64 = synth.model_to_f64(mnp)
    c0 = 0
    for n in split:
        om.encoder_append(prompt[None, c0:c0 + n], m64, ref)
        c0 += n
    for layer in range(dims["n_layers"]):
        assert_close_rel(kv.k[layer].float().cpu().numpy()[:, :, :96], ref["k"][layer][:, :, :96],
                         what=f"K layer {layer} (windowed)")
        assert_close_rel(kv.v[layer].float().cpu().numpy()[:, :, :96], ref["v"][layer][:, :, :96],
                         what=f"V layer {layer} (windowed)")
