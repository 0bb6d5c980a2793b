"""Comparison helpers for GPU-vs-oracle parity.

Floating-point results are compared within the stated tolerance.  Integer results that a float
decides (commit sets, stop decisions, argmax, Gumbel candidates) must match exactly whenever the
oracle's fp64 decision is robust to the float error actually observed; a decision closer to its
threshold than that error is reported as a certified near-tie and skipped.
"""
import numpy as np

# tolerances for hidden states, logits and entropies: bf16 inputs, fp32 accumulation
REL_TOL = 2e-2
# End-to-end bound for chained e4m3 stages (the stages themselves are held to REL_TOL from
# identical inputs).  An e4m3 quantiser (relative step D <= 2^-3) fed two inputs that differ by
# a relative d flips a code with probability ~ d / D, so its outputs differ by ~ sqrt(d D) in
# RMS: more than d whenever d < D.  Chained through the layers, the two sides' differences
# therefore grow towards the step D itself and no further (each side is within D / 2 of its own
# unquantised values): per row 2 D, over the whole array D.
FP8_CHAIN_TOL = 0.25
FP8_CHAIN_ARRAY_TOL = 0.125


def assert_close_rel(gpu, ref, rel=REL_TOL, what=""):
    """Hidden states, logits, cache rows: every row (vector along the last axis) within
    ||a - b||_2 <= rel ||b||_2, the whole array too, and no element beyond
    rel |b| + 4 rel rms(row) (a guard against isolated gross errors)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    g2 = gpu.reshape(-1, gpu.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    err = np.linalg.norm(g2 - r2, axis=1)
    nrm = np.linalg.norm(r2, axis=1)
    worst = np.max(err / np.maximum(nrm, 1e-30))
    assert np.all(err <= rel * nrm + 1e-30), f"{what}: worst row rel L2 error {worst:.3e}"
    assert np.linalg.norm(g2 - r2) <= rel * np.linalg.norm(r2) + 1e-30
    rms = np.sqrt(np.mean(r2 * r2, axis=1, keepdims=True))
    bad = np.abs(g2 - r2) > rel * np.abs(r2) + 4 * rel * rms
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond the outlier guard, worst "
                           f"{np.max(np.abs(g2 - r2)):.3e}")


def entropy_sensitivity(z_ref64, inv_t):
    """D = sum_v p_v |ln p_v + H| of softmax(z * inv_t) per row: |dH| <= D * max_v |dy_v| to
    first order, for a perturbation dy of the scaled logits."""
    y = np.asarray(z_ref64, dtype=np.float64) * np.float64(inv_t)
    y = y - y.max(axis=-1, keepdims=True)
    p = np.exp(y)
    p /= p.sum(axis=-1, keepdims=True)
    logp = np.log(np.where(p > 0, p, 1.0))
    h = -(p * logp).sum(axis=-1, keepdims=True)
    return (p * np.abs(logp + h)).sum(axis=-1)


def entropy_tolerance(h_ref, dy=None, sens=None):
    """2e-2 relative + 1e-6, plus (end to end) twice the first-order effect of the logit error."""
    tol = REL_TOL * np.abs(h_ref) + 1e-6
    if dy is not None:
        tol = tol + 2.0 * np.asarray(dy) * np.asarray(sens)
    return tol


def assert_entropy_close(h_gpu, h_ref, what="entropy", tol=None):
    h_gpu = np.asarray(h_gpu, dtype=np.float64)
    h_ref = np.asarray(h_ref, dtype=np.float64)
    if tol is None:
        tol = entropy_tolerance(h_ref)
    bad = np.abs(h_gpu - h_ref) > tol
    assert not bad.any(), (f"{what}: {bad.sum()} outside tolerance; worst abs err "
                           f"{np.max(np.abs(h_gpu - h_ref)):.3e}")


def selection_is_robust(h_ref, eps, uncommitted, bound):
    """Is the oracle's commit set unchanged under any perturbation |dH_i| <= eps_i?"""
    cand = [i for i in range(len(h_ref)) if uncommitted[i]]
    order = sorted(cand, key=lambda i: (h_ref[i], i))
    acc, n = 0.0, 0
    for i in order:
        if acc + h_ref[i] <= bound:
            acc += h_ref[i]
            n += 1
        else:
            break
    inside, outside = order[:n], order[n:]
    hi_in = max((h_ref[i] + eps[i] for i in inside), default=-np.inf)
    lo_out = min((h_ref[j] - eps[j] for j in outside), default=np.inf)
    if hi_in >= lo_out:
        return False                       # a member could swap with a non-member
    if inside and sum(h_ref[i] + eps[i] for i in inside) > bound:
        return False                       # the prefix might no longer fit
    if outside:
        nxt = min(outside, key=lambda j: h_ref[j] - eps[j])
        if sum(max(h_ref[i] - eps[i], 0.0) for i in inside) + h_ref[nxt] - eps[nxt] <= bound:
            return False                   # one more might fit
    return True


def mean_is_robust(h_ref, eps, threshold):
    m = float(np.mean(h_ref))
    return abs(m - threshold) > float(np.mean(eps)) + 1e-12


def argmax_certified(z_ref_row, err):
    """Is the argmax of the bf16-rounded logits unambiguous under a logit error <= err?"""
    z = np.asarray(z_ref_row, dtype=np.float64)
    top2 = np.partition(z, -2)[-2:]
    z1, z2 = top2[1], top2[0]
    return (z1 - z2) > 2.0 * err + 2.0 ** -7 * abs(z1)


def compare_eb_step(what, params, seed, ids, st_before, st_after, ref, gpu_state_host, gpu_out,
                    z_ref64, z_err=None):
    """Compare one EB step of the GPU with the oracle's (run on the oracle's own logits).

    ref: result of oracle.sampler.eb_step; st_after: oracle state after it.  z_err[b, i]: bound
    on |z_gpu - z_oracle| per row (None when both read the same logits).  Every canvas is
    checked: exactly where the oracle's decisions are robust to the float error observed, and
    for validity (the GPU's commit set is the rule's choice on its own entropies) where a
    certified near-tie leaves more than one correct answer.  Returns the number of canvases
    compared exactly (frozen canvases count as exact: they must not change at all)."""
    from oracle import sampler as osamp
    h_gpu = gpu_out.entropy.cpu().numpy().astype(np.float64)
    a_gpu = gpu_out.argmax.cpu().numpy().astype(np.int64)
    cn_gpu = gpu_out.commit_now.cpu().numpy().astype(bool)
    B, C = h_gpu.shape
    if z_err is None:
        z_err = np.zeros((B, C))
        tol = entropy_tolerance(ref["entropy"])
    else:
        inv_t = float(ref["inv_t"])
        tol = entropy_tolerance(ref["entropy"], z_err * inv_t,
                                entropy_sensitivity(z_ref64, ref["inv_t"]))
    assert_entropy_close(h_gpu, ref["entropy"], what, tol)
    g = gpu_state_host
    exact = 0
    for b in range(B):
        if st_before["done"][b]:
            assert np.array_equal(g["canvas"][b], st_before["canvas"][b]), "frozen canvas changed"
            exact += 1
            continue
        mism = np.nonzero(a_gpu[b] != ref["argmax"][b])[0]
        for i in mism:
            assert not argmax_certified(z_ref64[b, i], z_err[b, i]), \
                f"{what}: argmax differs at ({b},{i}) with a certified margin"
        eps = 2.0 * np.abs(h_gpu[b] - ref["entropy"][b]) + 1e-30
        unc = ~st_before["committed"][b]
        robust = mism.size == 0
        robust &= selection_is_robust(ref["entropy"][b], eps, unc, params["entropy_bound"])
        if params["stop_entropy"] >= 0:
            robust &= mean_is_robust(ref["entropy"][b], eps, params["stop_entropy"])
        if robust:
            for i in ref["selected"][b]:
                _, gap = osamp.gumbel_candidate(z_ref64[b, i], ref["inv_t"], seed, ids[b],
                                                ref["step"], i)
                if gap <= 2.0 * z_err[b, i] * float(ref["inv_t"]) + 1e-10 and \
                        g["canvas"][b][i] != st_after["canvas"][b][i]:
                    robust = False          # a near-tie Gumbel draw: both answers are correct
        if not robust:
            # near-tie: the GPU's commit set must still be the rule's choice on its own entropies
            if not g["done"][b]:
                sel, _, _ = osamp.select_commits(h_gpu[b], unc, params["entropy_bound"])
                want = np.zeros(C, dtype=bool)
                want[sel] = True
                assert np.array_equal(cn_gpu[b], want), f"{what}: GPU commit set invalid (b={b})"
            committed_before = st_before["committed"][b]
            assert np.array_equal(g["canvas"][b][committed_before],
                                  st_before["canvas"][b][committed_before]), \
                f"{what}: committed tokens changed (b={b})"
            continue
        assert np.array_equal(cn_gpu[b], ref["commit_now"][b]), f"{what}: commit mask (b={b})"
        for k in ("committed", "done", "stable_count", "prev_argmax"):
            assert np.array_equal(g[k][b], st_after[k][b]), f"{what}: {k} differs (b={b})"
        assert np.array_equal(g["canvas"][b], st_after["canvas"][b]), \
            f"{what}: canvas tokens differ (b={b})"
        exact += 1
    return exact


def routing_certified(dims, mnp, model, kv, ws, cache64, tokens, causal=False, margin=4.0,
                      ref_model=None, check_layers=False):
    """Per-position masks of canvas rows whose expert sets are certified in every layer so far.

    Each layer runs on the GPU (dg_layer_forward) from the oracle's own input to that layer
    (oracle -> GPU only); a row is certified in a layer when the oracle's gap between its k-th
    and (k+1)-th router logit exceeds `margin` times the largest router-logit error the GPU
    shows on that layer.  Returns a list: entry l is the mask of rows certified in layers < l
    (entry 0 is all True), for l = 0 .. n_layers.  causal: run the encoder layers (these write
    the rows' keys and values at [len, len + C) of the cache).  ref_model: the oracle's model
    when it differs from `mnp` (the e4m3-quantised model of the fp8 configuration).
    check_layers: also compare each layer's increment (output - input) with the oracle's on the
    rows certified in that layer, at the stated tolerance."""
    import torch
    from block_diffusion_decoding_canvas_amd import driver
    from oracle import model as om
    tokens = np.asarray(tokens)
    B, C = tokens.shape
    T, k = B * C, dims["top_k"]
    src = ref_model if ref_model is not None else mnp
    h = src["embed"][tokens].astype(np.float64)
    masks = [np.ones(T, dtype=bool)]
    for layer in range(dims["n_layers"]):
        h_next, _, _, info = om.layer_forward(h, src["layers"][layer], dims, layer,
                                              cache64["k"][layer], cache64["v"][layer],
                                              cache64["len"], causal=causal)
        hg = torch.from_numpy(h.reshape(T, -1).astype(np.float32)).to("cuda")
        rl = torch.zeros((T, dims["E"]), dtype=torch.float32, device="cuda")
        driver.layer_forward(model, kv, layer, int(causal), hg, ws, rl, None, None)
        torch.cuda.synchronize()
        r_ref = info["router_logits"]
        rerr = np.abs(rl.cpu().numpy() - r_ref).max()
        srt = -np.sort(-r_ref, axis=1)
        layer_cert = (srt[:, k - 1] - srt[:, k]) > margin * rerr + 1e-7
        if check_layers:
            h_in = h.reshape(T, -1).astype(np.float32).astype(np.float64)
            hout = hg.cpu().numpy().astype(np.float64)
            assert_close_rel(hout[layer_cert] - h_in[layer_cert],
                             h_next.reshape(T, -1)[layer_cert] - h_in[layer_cert],
                             what=f"layer {layer} increment (certified routing)")
        masks.append(masks[-1] & layer_cert)
        h = h_next
    return masks
