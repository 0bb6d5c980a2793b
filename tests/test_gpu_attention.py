"""GPU parity of canvas attention at every supported head_dim, through one decoder layer.

Each case runs one layer over 2 canvases of 40 positions with cache lengths 700 / 333 (740 and
373 keys: 12 and 6 key tiles of 64, both ending in a ragged tile, so the key range is split over
several workgroups and merged), 4 query / 2 KV heads, and compares the layer's increment of the
residual stream with the oracle on every row (the oracle takes the GPU's expert set at
router near-ties, checked for validity).  Modes: global
bidirectional (the decoder), a 48-position sliding window (decoder, windowed layer), and causal
canvas keys (the encoder pass that appends a finished canvas).  At head_dim 128 and 256 the
same cases also run on a 20-entry cache (shorter than the window) and an empty one.
"""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from oracle import model as om
from tests.parity_util import assert_close_rel, check_forced_routing

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("mode", ["global", "window", "causal"])
@pytest.mark.parametrize("dh", [16, 32, 64, 128, 256])
def test_attention_head_dims(dh, mode):
    _attention_case(dh, mode, (700, 333), 760)


@pytest.mark.parametrize("mode", ["global", "window", "causal"])
@pytest.mark.parametrize("dh", [128, 256])
def test_attention_short_and_empty_cache(dh, mode):
    """A 20-entry cache (shorter than the 48-position window, so the window starts at position
    0) and an empty one (canvas keys only)."""
    _attention_case(dh, mode, (20, 0), 64)


def _attention_case(dh, mode, lens, cap):
    window = 48 if mode == "window" else 0
    causal = 1 if mode == "causal" else 0
    dims = dict(n_layers=1, d=64, hq=4, hkv=2, dh=dh, E=8, top_k=2, F=64, Fs=64, V=256, C=40,
                window=window, global_every=2, eps=1e-6)
    rng = np.random.default_rng(31 + dh)
    mnp = dict(dims=dims, layers=[synth.make_layer(dims, rng, norm_gain_std=0.1)],
               embed=np.zeros((256, 64), np.float32), final_norm=np.ones(64, np.float32),
               w_lm=np.zeros((256, 64), np.float32))
    B = len(lens)
    cache = synth.make_cache(dims, B, cap, max(lens), seed=32)
    for b, n in enumerate(lens):
        for lst in (cache["k"], cache["v"]):
            for a in lst:
                a[b, :, n:] = 0.0
    cache["len"] = np.array(lens, dtype=np.int64)
    T = B * dims["C"]
    h = synth.hidden_states(T, 64, seed=33)
    print(f"attention case dh={dh} mode={mode} lens={lens}", flush=True)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    kv = driver.KVCache.from_host(dims, cache, cap, DEV)
    ws = driver.workspace(model.workspace_bytes(B))
    hg = torch.from_numpy(h.astype(np.float32)).to(DEV)
    rl = torch.zeros((T, 8), dtype=torch.float32, device=DEV)
    ti = torch.zeros((T, 2), dtype=torch.int32, device=DEV)
    gt = torch.zeros((T, 2), dtype=torch.float32, device=DEV)
    driver.layer_forward(model, kv, 0, causal, hg, ws, rl, ti, gt)
    torch.cuda.synchronize()
    lw = synth.model_to_f64(mnp)["layers"][0]
    h_ref, _, _, info = om.layer_forward(
        h.astype(np.float64).reshape(B, dims["C"], 64), lw, dims, 0,
        cache["k"][0].astype(np.float64), cache["v"][0].astype(np.float64),
        np.array(cache["len"]), causal=bool(causal))
    h_ref = h_ref.reshape(T, 64)
    r_ref = info["router_logits"].reshape(T, -1)
    rg = rl.cpu().numpy()
    # the router logits depend on the attention output only through the residual stream, so
    # they check attention before any expert choice
    assert_close_rel(rg, r_ref, what=f"router logits dh={dh} {mode}")
    # every row: the oracle takes the GPU's expert set at router near-ties (checked first)
    tig = ti.cpu().numpy().astype(np.int64)
    check_forced_routing(r_ref, rg, tig, 2, f"dh={dh} {mode}")
    h_ref, _, _, _ = om.layer_forward(
        h.astype(np.float64).reshape(B, dims["C"], 64), lw, dims, 0,
        cache["k"][0].astype(np.float64), cache["v"][0].astype(np.float64),
        np.array(cache["len"]), causal=bool(causal), force_idx=tig.reshape(B, dims["C"], 2))
    h_ref = h_ref.reshape(T, 64)
    hout = hg.cpu().numpy()
    assert_close_rel(hout - h, h_ref - h, what=f"layer increment dh={dh} {mode} (all rows)")
