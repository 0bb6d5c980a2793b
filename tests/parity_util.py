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


def assert_entropy_close(h_gpu, h_ref, what="entropy"):
    h_gpu = np.asarray(h_gpu, dtype=np.float64)
    h_ref = np.asarray(h_ref, dtype=np.float64)
    bad = np.abs(h_gpu - h_ref) > REL_TOL * np.abs(h_ref) + 1e-6
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
