"""GPU parity of the pipeline's other schedulers (dg_sample, dg_decoder_step_sched) against the
oracle (oracle/schedulers.py), on identical bf16 logits.

Workloads: the standalone sampler's row mix (peaked rows with one logit 12 over N(0,1), N(0, 2)
rows and N(0, 0.1) rows) at V 262,144 (block refinement) and V 65,536 (DDIM, whose every row
draws from its posterior each step), greedy and sampled temperatures, threshold, quota, editing,
predictor, corrector and final steps; both schedulers on canvases of 1 and 1,024 positions (the
C ABI's canvas-length extremes) at V 512; and the toy decoder with a sharp LM head run through
dg_decoder_step_sched in lockstep with the oracle.

Integers are compared exactly wherever the oracle's decision is robust to the GPU's float error:
confidences (fp32 from the merged row statistics) within 1e-5 relative of the threshold or of the
confidence at the commit boundary, and Gumbel draws whose top-2 score gap is below 1e-5, are
certified near-ties; there the GPU's choice is only checked for validity.
"""
import copy

import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver, synth
from oracle import model as om
from oracle import sampler as osamp
from oracle import schedulers as osch
from tests.parity_util import GpuChain, assert_close_rel, assert_entropy_close, entropy_tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda"
CONF_TOL = 1e-5
GAP_TOL = 1e-5


def _logits(B, C, V, seed):
    z, _ = synth.sampler_logits(B * C, V, seed=seed)
    return z.reshape(B, C, V)


def _state_with_commits(z, ids, seed, frac, rng):
    B, C, V = z.shape
    st = osamp.new_state(osamp.init_canvas(seed, ids, C, V))
    st["committed"][:] = rng.random((B, C)) < frac
    return st


def _run_gpu(zt, step, params_dict, seed, ids, st):
    B, C, V = zt.shape
    gs = driver.SamplerState(B, C, DEV, canvas_ids=ids)
    gs.load_host(st)
    out = driver.StepOut(B, C, V, DEV, with_logits=False)
    driver.sample(zt, step, driver.sched_params_from_dict(params_dict, seed), gs, out)
    torch.cuda.synchronize()
    return gs, out


def _br_robust(ref, before, params, b):
    """Is canvas b's block-refinement decision robust to a CONF_TOL relative confidence error
    and to GAP_TOL on the Gumbel draws?"""
    conf, gap = ref["conf"][b], ref["gap"][b]
    unc = np.nonzero(~before["committed"][b])[0]
    tol = CONF_TOL * np.abs(conf) + 1e-9
    if np.any(np.abs(conf[unc] - params["threshold"]) <= tol[unc]):
        return False
    order = sorted(unc, key=lambda i: (-conf[i], i))
    n = len(ref["selected"][b])
    if 0 < n < len(order) and conf[order[n - 1]] - conf[order[n]] <= tol[order[n - 1]]:
        return False
    if params["editing_threshold"] >= 0:
        com = np.nonzero(before["committed"][b])[0]
        if np.any(np.abs(conf[com] - params["editing_threshold"]) <= tol[com]):
            return False
    need = unc if params["editing_threshold"] < 0 else np.arange(len(conf))
    return not np.any(gap[need] <= GAP_TOL)


def _compare_br(zt, z64, step, params, seed, ids, st):
    before = copy.deepcopy(st)
    gs, out = _run_gpu(zt, step, params, seed, ids, st)
    ref = osch.block_refinement_step(z64, step, params, st, seed, ids)
    assert_entropy_close(out.entropy.cpu().numpy(), ref["entropy"], f"BR entropy s={step}")
    assert np.array_equal(out.argmax.cpu().numpy(), ref["argmax"])
    g = gs.host()
    cn = out.commit_now.cpu().numpy().astype(bool)
    exact = 0
    for b in range(z64.shape[0]):
        if not _br_robust(ref, before, params, b):
            # near-tie: only positions uncommitted before the step can commit in it
            assert not np.any(cn[b] & before["committed"][b])
            continue
        assert np.array_equal(cn[b], ref["commit_now"][b]), f"commit mask b={b} s={step}"
        for k in ("canvas", "committed", "done", "stable_count", "prev_argmax"):
            assert np.array_equal(g[k][b], st[k][b]), f"{k} b={b} s={step}"
        exact += 1
    return exact, int(ref["commit_now"].sum()), sum(len(e) for e in ref["edited"])


@pytest.mark.parametrize("temperature,editing", [(0.0, -1.0), (0.5, -1.0), (0.5, 0.3)])
def test_block_refinement_standalone(temperature, editing):
    B, C, V = 2, 256, 262144
    z = _logits(B, C, V, seed=21)
    zt = torch.from_numpy(z).to(DEV, torch.bfloat16)
    z64 = z.astype(np.float64)
    params = osch.default_params(osch.BLOCK_REFINEMENT)
    params.update(temperature=temperature, editing_threshold=editing, stop_entropy=-1.0)
    seed, ids = 5, [3, 8]
    rng = np.random.default_rng(22)
    total = 0
    for step, frac in [(0, 0.0), (20, 0.4), (47, 0.7)]:
        print(f"BR case T={temperature} edit={editing} step {step}", flush=True)
        st = _state_with_commits(z, ids, seed, frac, rng)
        exact, commits, edits = _compare_br(zt, z64, step, params, seed, ids, st)
        print(f"  exact canvases {exact}/{B}, commits {commits}, edits {edits}", flush=True)
        assert exact >= 1
        total += commits
    assert total > 0


def _ddim_robust(ref, conf_gpu_free, b, before, z64, params, inv_t):
    gap = ref["gap"][b]
    rows = ref["resampled"][b]
    if np.any(gap[rows] <= GAP_TOL):
        return False
    if ref["phase"][0] == "correct":
        C = z64.shape[1]
        x = before["canvas"][b]
        if params["temperature"] > 0:
            conf = np.array([osch.model_probs(z64[b, i], inv_t)[x[i]] for i in range(C)])
        else:
            conf = (x == z64[b].argmax(axis=1)).astype(np.float64)
        order = sorted(range(C), key=lambda i: (conf[i], i))
        k = int(params["corrector_k"])
        # greedy confidences are exactly 0 or 1 on both sides: ties break by position, exactly
        if params["temperature"] > 0 and 0 < k < C and \
                conf[order[k]] - conf[order[k - 1]] <= CONF_TOL * conf[order[k]] + 1e-12:
            return False
    return True


@pytest.mark.parametrize("temperature", [0.0, 0.8])
def test_discrete_ddim_standalone(temperature):
    B, C, V, S = 2, 48, 65536, 10
    z = _logits(B, C, V, seed=31)
    zt = torch.from_numpy(z).to(DEV, torch.bfloat16)
    z64 = z.astype(np.float64)
    params = osch.default_params(osch.DISCRETE_DDIM)
    params.update(max_steps=S, temperature=temperature, corrector_steps=3, corrector_k=7,
                  stop_entropy=-1.0)
    seed, ids = 9, [1, 4]
    inv_t = osch.inv_temperature_f32(temperature)
    st = osamp.new_state(osamp.init_canvas(seed, ids, C, V))
    exact = 0
    for step in (0, 3, 5, 6, 8, 9):       # predictor, predictor, predictor, corrector x2, final
        print(f"DDIM case T={temperature} step {step}", flush=True)
        before = copy.deepcopy(st)
        gs, out = _run_gpu(zt, step, params, seed, ids, st)
        ref = osch.discrete_ddim_step(z64, step, params, st, seed, ids)
        assert_entropy_close(out.entropy.cpu().numpy(), ref["entropy"], f"DDIM entropy s={step}")
        g = gs.host()
        cn = out.commit_now.cpu().numpy().astype(bool)
        assert np.array_equal(cn, ref["commit_now"])
        for b in range(B):
            if not _ddim_robust(ref, None, b, before, z64, params, inv_t):
                st["canvas"][b] = g["canvas"][b]          # continue from the GPU's valid draw
                continue
            for k in ("canvas", "committed", "done", "stable_count", "prev_argmax"):
                assert np.array_equal(g[k][b], st[k][b]), f"{k} b={b} s={step}"
            exact += 1
        print(f"  phase {ref['phase'][0]}, resampled {[len(r) for r in ref['resampled']]}",
              flush=True)
    assert exact >= 10
    assert st["done"].all() and st["committed"].all()


@pytest.mark.parametrize("kind", [osch.BLOCK_REFINEMENT, osch.DISCRETE_DDIM])
def test_decoder_step_sched_lockstep(kind):
    """The toy decoder with a sharp LM head through dg_decoder_step_sched, every step from the
    oracle's state: logits at the stated tolerance (the oracle takes the GPU's expert sets at
    router near-ties), then the scheduler's decisions on those logits, exactly where robust."""
    dims = synth.dims_tiny()
    mnp = synth.make_model(dims, seed=0, norm_gain_std=0.1, lm_std=1.0)
    m64 = synth.model_to_f64(mnp)
    cache = synth.make_cache(dims, 1, 64, 32, seed=1)
    c64 = dict(k=[a.astype(np.float64) for a in cache["k"]],
               v=[a.astype(np.float64) for a in cache["v"]], len=np.array(cache["len"]))
    model = driver.Model(synth.model_to_device(mnp, DEV))
    kv = driver.KVCache.from_host(dims, cache, 64, DEV)
    ws = driver.workspace(model.workspace_bytes(1))
    S = 8
    params = osch.default_params(kind)
    params.update(max_steps=S, temperature=0.7)
    if kind == osch.DISCRETE_DDIM:
        params.update(corrector_steps=2, corrector_k=4)
    seed, ids = 2, [0]
    p = driver.sched_params_from_dict(params, seed)
    gs = driver.SamplerState(1, dims["C"], DEV)
    st = osamp.new_state(osamp.init_canvas(seed, ids, dims["C"], dims["V"]))
    out = driver.StepOut(1, dims["C"], dims["V"], DEV)
    inv_t = osch.inv_temperature_f32(params["temperature"])
    for s in range(S):
        gs.load_host(st)
        driver.decoder_step_sched(model, kv, s, p, gs, out, ws)
        torch.cuda.synchronize()
        chain = GpuChain(dims, model, kv, ws, st["canvas"], mnp["embed"])
        zr, z64, infos = om.decoder_forward(st["canvas"], m64, c64, force_idx=chain.idx)
        chain.check(infos, dims["top_k"], f"{kind} s={s}")
        zg = out.logits.float().cpu().numpy()
        assert_close_rel(zg, zr, what=f"{kind} logits s={s}")
        # the scheduler's decisions on the GPU's own logits (its exactness on identical logits
        # is what the standalone tests pin); the logits' error shows in the entropies only
        before = copy.deepcopy(st)
        zg64 = zg.astype(np.float64)
        if kind == osch.BLOCK_REFINEMENT:
            ref = osch.block_refinement_step(zg64, s, params, st, seed, ids)
            robust = _br_robust(ref, before, params, 0)
        else:
            ref = osch.discrete_ddim_step(zg64, s, params, st, seed, ids)
            robust = _ddim_robust(ref, None, 0, before, zg64, params, inv_t)
        h_ref, _ = osamp.entropy_argmax(zr, inv_t)
        dz = np.abs(zg - z64).max(axis=-1) * float(inv_t)
        from tests.parity_util import entropy_sensitivity
        tol = entropy_tolerance(h_ref, dz, entropy_sensitivity(z64, inv_t))
        assert_entropy_close(out.entropy.cpu().numpy(), h_ref, f"{kind} entropy s={s}", tol)
        g = gs.host()
        if robust:
            assert np.array_equal(out.commit_now.cpu().numpy().astype(bool), ref["commit_now"])
            for k in ("canvas", "committed", "done"):
                assert np.array_equal(g[k], st[k]), f"{kind} {k} s={s}"
        else:
            st = {k: np.array(v) for k, v in g.items()}
        print(f"{kind} step {s}: commits {int(ref['commit_now'].sum())}, "
              f"{'exact' if robust else 'near-tie'}", flush=True)
        if st["done"].all():
            break
    assert st["done"].all()


@pytest.mark.parametrize("C", [1, 1024])
def test_block_refinement_canvas_extremes(C):
    """Block refinement on the smallest and the largest canvas the C ABI accepts (1 and 1,024
    positions; at 1,024 the confidence order spans the whole commit block), sampled with
    editing, against the oracle exactly where robust."""
    B, V = 2, 512
    z = _logits(B, C, V, seed=51 + C)
    zt = torch.from_numpy(z).to(DEV, torch.bfloat16)
    z64 = z.astype(np.float64)
    params = osch.default_params(osch.BLOCK_REFINEMENT)
    params.update(max_steps=8, temperature=0.5, editing_threshold=0.3, stop_entropy=-1.0)
    seed, ids = 6, [2, 5]
    rng = np.random.default_rng(52)
    exact_total = 0
    for step, frac in [(0, 0.0), (3, 0.4), (6, 0.7)]:
        print(f"BR C={C} step {step}", flush=True)
        st = _state_with_commits(z, ids, seed, frac, rng)
        exact, commits, edits = _compare_br(zt, z64, step, params, seed, ids, st)
        print(f"  exact canvases {exact}/{B}, commits {commits}, edits {edits}", flush=True)
        exact_total += exact
    assert exact_total >= 1


@pytest.mark.parametrize("C,k", [(1, 1), (1024, 300)])
def test_discrete_ddim_canvas_extremes(C, k):
    """Discrete DDIM with its leave-one-out corrector on the smallest and the largest canvas
    (1 and 1,024 positions; the corrector re-draws the k least confident), predictor,
    corrector and final steps, against the oracle exactly where robust."""
    B, V, S = 2, 512, 10
    z = _logits(B, C, V, seed=61 + C)
    zt = torch.from_numpy(z).to(DEV, torch.bfloat16)
    z64 = z.astype(np.float64)
    params = osch.default_params(osch.DISCRETE_DDIM)
    params.update(max_steps=S, temperature=0.8, corrector_steps=3, corrector_k=k,
                  stop_entropy=-1.0)
    seed, ids = 11, [0, 3]
    inv_t = osch.inv_temperature_f32(0.8)
    st = osamp.new_state(osamp.init_canvas(seed, ids, C, V))
    exact = 0
    for step in (0, 3, 5, 6, 8, 9):       # predictor, predictor, predictor, corrector x2, final
        print(f"DDIM C={C} step {step}", flush=True)
        before = copy.deepcopy(st)
        gs, out = _run_gpu(zt, step, params, seed, ids, st)
        ref = osch.discrete_ddim_step(z64, step, params, st, seed, ids)
        assert_entropy_close(out.entropy.cpu().numpy(), ref["entropy"], f"DDIM entropy s={step}")
        g = gs.host()
        cn = out.commit_now.cpu().numpy().astype(bool)
        assert np.array_equal(cn, ref["commit_now"])
        for b in range(B):
            if not _ddim_robust(ref, None, b, before, z64, params, inv_t):
                st["canvas"][b] = g["canvas"][b]          # continue from the GPU's valid draw
                continue
            for key in ("canvas", "committed", "done", "stable_count", "prev_argmax"):
                assert np.array_equal(g[key][b], st[key][b]), f"{key} b={b} s={step}"
            exact += 1
    assert exact >= 6
    assert st["done"].all() and st["committed"].all()
