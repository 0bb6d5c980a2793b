"""One small invocation of the hot path on cuda:0, checked against the oracle (used by smoke()):
the toy decoder prefills a 32-token prompt through the encoder append, then runs one
entropy-bound denoising step over a 16-token canvas."""
import copy

import numpy as np
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from oracle import model as om
from oracle import sampler as osamp
from tests.parity_util import GpuChain, assert_close_rel, compare_eb_step


def run_smoke():
    assert torch.cuda.is_available(), "smoke() needs a GPU"
    dims = synth.dims_tiny()
    mnp = synth.make_model(dims, seed=0, norm_gain_std=0.1, lm_std=1.0)
    m64 = synth.model_to_f64(mnp)
    model = driver.Model(synth.model_to_device(mnp, "cuda"))
    kv = driver.KVCache(dims, 1, 64, "cuda")
    ws = driver.workspace(model.workspace_bytes(1))
    prompt = synth.prompt_ids(32, dims["V"])
    for c0 in (0, 16):
        tok = torch.tensor(prompt[None, c0:c0 + 16], dtype=torch.int32, device="cuda")
        driver.kv_append_canvas(model, kv, tok, ws)
    ref_cache = synth.empty_cache(dims, 1, 64)
    ref_cache = dict(k=[a.astype(np.float64) for a in ref_cache["k"]],
                     v=[a.astype(np.float64) for a in ref_cache["v"]], len=ref_cache["len"])
    om.encoder_append(prompt[None], m64, ref_cache)

    params = dict(osamp.default_params(), max_steps=8)
    seed, ids = 2, [0]
    p = driver.eb_params_from_dict(params, seed)
    gs = driver.SamplerState(1, dims["C"], "cuda")
    driver.canvas_init(p, gs, dims["V"])
    st = osamp.new_state(osamp.init_canvas(seed, ids, dims["C"], dims["V"]))
    out = driver.StepOut(1, dims["C"], dims["V"], "cuda")
    driver.decoder_step(model, kv, 0, p, gs, out, ws)
    torch.cuda.synchronize()
    chain = GpuChain(dims, model, kv, ws, st["canvas"], mnp["embed"])
    zr, z64, infos = om.decoder_forward(st["canvas"], m64, ref_cache, force_idx=chain.idx)
    chain.check(infos, dims["top_k"], "smoke")
    zg = out.logits.float().cpu().numpy()
    assert_close_rel(zg, zr, what="smoke logits")
    before = copy.deepcopy(st)
    ref = osamp.eb_step(zr, 0, params, st, seed, ids)
    exact = compare_eb_step("smoke", params, seed, ids, before, st, ref, gs.host(), out, z64,
                            np.abs(zg - z64).max(axis=-1))
    print(f"smoke: prefill + one decoder step on cuda:0 match the oracle "
          f"({'exact' if exact else 'near-tie checked'} sampler decisions)")
