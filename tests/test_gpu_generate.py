"""GPU parity of the outer generation loop (dg_generate).

Workload: the 2-layer toy decoder with a sharp LM head (commits, adaptive stops and EOS happen
within a few canvases), a 32-token prompt per sequence written by the chunked prefill, 40 tokens
to generate (3 canvases of 16).
- Against the same loop written in Python over the step calls (dg_canvas_init, dg_decoder_step
  with the done flags read after every step, dg_kv_append_canvas) with canvas ids c * B + b,
  for 2 sequences: tokens, canvases, steps per canvas and the cache agree bit for bit.
- Against the oracle's loop (oracle/generate.py) for 1 sequence: tokens, canvases and steps per
  canvas agree exactly, without and with an EOS id taken from the first canvas (one canvas).
- Two sequences with an EOS id that one of them produces only in its second canvas: the loop
  stops after that canvas, with the tokens of the full run.
"""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from oracle import generate as og
from oracle import model as om
from oracle import sampler as osamp

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu_setup(batch):
    dims = synth.dims_tiny()
    mnp = synth.make_model(dims, seed=0, norm_gain_std=0.1, lm_std=1.0)
    model = driver.Model(synth.model_to_device(mnp, DEV))
    prompt = np.stack([synth.prompt_ids(32, dims["V"], seed=1 + b) for b in range(batch)])
    kv = driver.KVCache(dims, batch, 128, DEV)
    ws = driver.workspace(model.append_workspace_bytes(batch, 32))
    driver.kv_append_tokens(model, kv, torch.tensor(prompt, dtype=torch.int32, device=DEV), ws)
    torch.cuda.synchronize()
    return dims, mnp, model, prompt, kv


def test_generate_matches_python_loop():
    B = 2
    dims, mnp, model, prompt, kv = _gpu_setup(B)
    _, _, _, _, kv2 = _gpu_setup(B)
    p = driver.eb_params_from_dict(dict(osamp.default_params(), max_steps=8), 2)
    print("generate case: C loop vs Python loop, B 2", flush=True)
    state = driver.SamplerState(B, dims["C"], DEV)
    out = driver.StepOut(B, dims["C"], dims["V"], DEV)
    tok, n, steps = driver.generate(model, kv, p, state, out, gen_length=40)
    torch.cuda.synchronize()
    # the same loop over the step calls
    ws = driver.workspace(model.workspace_bytes(B))
    ref_tok, ref_steps = [], []
    for c in range(3):
        st = driver.SamplerState(B, dims["C"], DEV, canvas_ids=[c * B + b for b in range(B)])
        driver.canvas_init(p, st, dims["V"])
        k = 0
        for s in range(8):
            driver.decoder_step(model, kv2, s, p, st, out, ws)
            k += 1
            if bool(st.done.all()):
                break
        ref_tok.append(st.canvas.clone())
        driver.kv_append_canvas(model, kv2, st.canvas, ws)
        ref_steps.append(k)
    torch.cuda.synchronize()
    assert n == 3 and steps == ref_steps
    assert torch.equal(tok, torch.cat(ref_tok, dim=1))
    assert kv.lengths() == kv2.lengths() == [32 + 48] * B
    assert torch.equal(kv.k, kv2.k) and torch.equal(kv.v, kv2.v)


@pytest.mark.parametrize("use_eos", [False, True])
def test_generate_matches_oracle(use_eos):
    dims, mnp, model, prompt, kv = _gpu_setup(1)
    params = dict(osamp.default_params(), max_steps=8)
    m64 = synth.model_to_f64(mnp)
    cache = synth.empty_cache(dims, 1, 128)
    cache = dict(k=[a.astype(np.float64) for a in cache["k"]],
                 v=[a.astype(np.float64) for a in cache["v"]], len=np.array(cache["len"]))
    om.encoder_append(prompt, m64, cache)
    eos = -1
    if use_eos:
        probe = og.generate(m64, {k: ([a.copy() for a in v] if isinstance(v, list) else v.copy())
                                  for k, v in cache.items()}, params, 2, gen_length=16)
        eos = int(probe["tokens"][0, 5])
    ref = og.generate(m64, cache, params, 2, gen_length=40, eos_id=eos)
    print(f"generate case: against the oracle, eos {eos}", flush=True)
    state = driver.SamplerState(1, dims["C"], DEV)
    out = driver.StepOut(1, dims["C"], dims["V"], DEV)
    tok, n, steps = driver.generate(model, kv, driver.eb_params_from_dict(params, 2), state, out,
                                    gen_length=40, eos_token_id=eos)
    torch.cuda.synchronize()
    assert n == ref["canvases"] == (1 if use_eos else 3)
    assert steps == ref["steps"]
    np.testing.assert_array_equal(tok.cpu().numpy(), ref["tokens"])


def test_generate_eos_waits_for_every_sequence():
    """Two sequences: an EOS id that sequence 0 produces in its first canvas and sequence 1 only
    in its second stops the native loop after the second canvas, with the tokens of the full
    run."""
    B = 2
    dims, mnp, model, prompt, kv = _gpu_setup(B)
    p = driver.eb_params_from_dict(dict(osamp.default_params(), max_steps=8), 2)
    state = driver.SamplerState(B, dims["C"], DEV)
    out = driver.StepOut(B, dims["C"], dims["V"], DEV)
    full, n, _ = driver.generate(model, kv, p, state, out, gen_length=48)
    t = full.cpu().numpy()
    canv = [[set(t[b, 16 * c:16 * c + 16].tolist()) for c in range(3)] for b in range(B)]
    cands = [v for v in sorted(canv[0][0]) if v not in canv[1][0] and v in canv[1][1]]
    cands += [v for v in sorted(canv[1][0]) if v not in canv[0][0] and v in canv[0][1]]
    assert n == 3 and cands, "no token with the needed pattern"
    _, _, _, _, kv2 = _gpu_setup(B)
    print(f"generate case: EOS {cands[0]} with 2 sequences", flush=True)
    tok, n2, _ = driver.generate(model, kv2, p, state, out, gen_length=48, eos_token_id=cands[0])
    torch.cuda.synchronize()
    assert n2 == 2
    assert torch.equal(tok, full[:, :32])
    assert kv2.lengths() == [32 + 32] * B
