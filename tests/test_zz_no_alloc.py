"""The allocation-free sampler entry point (dg_eb_sample_noalloc) against dg_eb_sample, through
the C ABI: two calls in a row on the standalone sampler workload, the second with a smaller
input, each compared bit for bit (entropies, argmax, commit mask, the whole sampler state) with
dg_eb_sample on a copy of the same state; plus the size limit."""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from block_diffusion_decoding_canvas_amd._lib import DgError

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(B, C, V, ids, step, logits, seed):
    params = driver.eb_params(seed=seed)
    a = driver.SamplerState(B, C, DEV, canvas_ids=ids)
    b = driver.SamplerState(B, C, DEV, canvas_ids=ids)
    driver.canvas_init(params, a, V)
    driver.canvas_init(params, b, V)
    oa = driver.StepOut(B, C, V, DEV, with_logits=False)
    ob = driver.StepOut(B, C, V, DEV, with_logits=False)
    driver.eb_sample(logits, step, params, a, oa)
    driver.eb_sample_noalloc(logits, step, params, b, ob)
    torch.cuda.synchronize()
    for name in ("entropy", "argmax", "commit_now"):
        assert torch.equal(getattr(oa, name), getattr(ob, name)), name
    ha, hb = a.host(), b.host()
    for k in ha:
        assert np.array_equal(ha[k], hb[k]), k
    return int(oa.commit_now.sum())


def test_noalloc_matches_workspace_entry_point():
    print("no-alloc case 1: B 1, C 256, V 262144, step 36", flush=True)
    z, _ = synth.sampler_logits(256, 262144, seed=1)
    big = torch.from_numpy(z.reshape(1, 256, 262144)).to(DEV, torch.bfloat16)
    n1 = _pair(1, 256, 262144, [0], 36, big, seed=2)
    del big
    print("no-alloc case 2: B 3, C 40, V 8192, step 46", flush=True)
    z2, _ = synth.sampler_logits(120, 8192, seed=3)
    small = torch.from_numpy(z2.reshape(3, 40, 8192)).to(DEV, torch.bfloat16)
    n2 = _pair(3, 40, 8192, [4, 0, 9], 46, small, seed=5)
    assert n1 > 0 and n2 > 0          # the candidate kernels ran in both calls


def test_noalloc_rejects_oversize():
    lib = driver._lib.load()
    cap = lib.dg_eb_sample_noalloc_max_bytes()
    assert cap == 8 << 20
    B, C, V = 32, 256, 262144
    assert lib.dg_eb_workspace_bytes(B, C, V) > cap
    logits = torch.zeros((1, 256), dtype=torch.bfloat16, device=DEV)
    st = driver.SamplerState(B, C, DEV)
    out = driver.StepOut(B, C, V, DEV, with_logits=False)
    with pytest.raises(DgError, match="WORKSPACE"):
        driver.check(lib.dg_eb_sample_noalloc(driver.ptr(logits), B, C, V, 0,
                                              driver.ctypes.byref(driver.eb_params()),
                                              driver.ctypes.byref(st.struct()),
                                              driver.ctypes.byref(out.struct()),
                                              driver.stream_ptr()), "noalloc")
