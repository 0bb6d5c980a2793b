"""Comparison helpers for GPU-vs-oracle parity.

Floating-point results are compared within the stated tolerance.  Integer results that a float
decides (commit sets, stop decisions, argmax, Gumbel candidates) must match exactly whenever the
oracle's fp64 decision is robust to the float error actually observed; a decision closer to its
threshold than that error is reported as a certified near-tie and skipped.
"""
import numpy as np

# tolerances for hidden states, logits and entropies: bf16 inputs, fp32 accumulation
REL_TOL = 2e-2


def assert_close_rel(gpu, ref, rel=REL_TOL, what=""):
    """Hidden states and logits: ||a-b|| <= rel ||b|| and |a-b| <= rel |b| + rel * rms(b)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    err = np.linalg.norm(gpu - ref)
    nrm = np.linalg.norm(ref)
    assert err <= rel * nrm + 1e-30, f"{what}: rel L2 error {err / max(nrm, 1e-30):.3e}"
    rms = np.sqrt(np.mean(ref * ref))
    bad = np.abs(gpu - ref) > rel * np.abs(ref) + rel * rms
    assert not bad.any(), (f"{what}: {bad.sum()} elements outside tolerance, worst "
                           f"{np.max(np.abs(gpu - ref)):.3e} (rms {rms:.3e})")


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
    on |z_gpu - z_oracle| per row (0 when both read the same logits).  Returns False when a
    certified near-tie prevents an exact comparison (the runs may diverge from here)."""
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
    for b in range(B):
        if st_before["done"][b]:
            assert np.array_equal(g["canvas"][b], st_before["canvas"][b]), "frozen canvas changed"
            continue
        for i in range(C):
            if a_gpu[b, i] != ref["argmax"][b, i]:
                assert not argmax_certified(z_ref64[b, i], z_err[b, i]), \
                    f"{what}: argmax differs at ({b},{i}) with a certified margin"
                return False
        eps = 2.0 * np.abs(h_gpu[b] - ref["entropy"][b]) + 1e-30
        unc = ~st_before["committed"][b]
        robust = selection_is_robust(ref["entropy"][b], eps, unc, params["entropy_bound"])
        if params["stop_entropy"] >= 0:
            robust &= mean_is_robust(ref["entropy"][b], eps, params["stop_entropy"])
        if not robust:
            # near-tie: the GPU's commit set must still be the rule's choice on its own entropies
            if not ref["finalised"][b] and not g["done"][b]:
                sel, _, _ = osamp.select_commits(h_gpu[b], unc, params["entropy_bound"])
                want = np.zeros(C, dtype=bool)
                want[sel] = True
                assert np.array_equal(cn_gpu[b], want), f"{what}: GPU commit set invalid (b={b})"
            return False
        assert np.array_equal(cn_gpu[b], ref["commit_now"][b]), f"{what}: commit mask (b={b})"
        for k in ("committed", "done", "stable_count", "prev_argmax"):
            assert np.array_equal(g[k][b], st_after[k][b]), f"{what}: {k} differs (b={b})"
        for i in ref["selected"][b]:
            _, gap = osamp.gumbel_candidate(z_ref64[b, i], ref["inv_t"], seed, ids[b],
                                            ref["step"], i)
            if gap > 2.0 * z_err[b, i] * float(ref["inv_t"]) + 1e-10:
                assert g["canvas"][b][i] == st_after["canvas"][b][i], f"{what}: candidate at {i}"
            elif g["canvas"][b][i] != st_after["canvas"][b][i]:
                return False
        others = [i for i in range(C) if i not in set(ref["selected"][b])]
        assert np.array_equal(g["canvas"][b][others], st_after["canvas"][b][others]), \
            f"{what}: renoised/finalised tokens differ"
    return True
