"""One small invocation of the hot path on cuda:0, checked against the oracle (used by smoke())."""
import copy

import numpy as np
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from oracle import sampler as osamp


def run_smoke():
    assert torch.cuda.is_available(), "smoke() needs a GPU"
    B, C, V = 1, 16, 512
    params = dict(osamp.default_params(), max_steps=8)
    seed, ids = 2, [0]
    st = driver.SamplerState(B, C, "cuda")
    p = driver.eb_params_from_dict(params, seed)
    driver.canvas_init(p, st, V)
    ref = osamp.new_state(osamp.init_canvas(seed, ids, C, V))
    assert np.array_equal(st.host()["canvas"], ref["canvas"])
    z = synth.to_bf16_values(np.random.default_rng(0).standard_normal((B, C, V)) * 8.0)
    out = driver.StepOut(B, C, V, "cuda", with_logits=False)
    driver.eb_sample(synth.to_device_bf16(z, "cuda"), 3, p, st, out)
    torch.cuda.synchronize()
    r = osamp.eb_step(z.astype(np.float64), 3, params, copy.deepcopy(ref), seed, ids)
    assert np.array_equal(out.argmax.cpu().numpy(), r["argmax"])
    assert np.allclose(out.entropy.cpu().numpy(), r["entropy"], rtol=2e-2, atol=1e-6)
    print("smoke: sampler step on cuda:0 matches the oracle")
