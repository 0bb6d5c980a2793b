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


# Elementwise guard.  The row bound ||a - b||_2 <= rel ||b||_2 allows an error field of RMS
# sigma = rel * rms(b).  For Gaussian errors of that RMS the union bound gives
# P(max_i |e_i| > t) <= 2 n exp(-t^2 / (2 sigma^2)) over the n elements of a row, so the largest
# element stays below t = sigma * sqrt(2 ln(2 n / GUARD_DELTA)) except with probability
# GUARD_DELTA.  An isolated gross error hides in the L2 norm of a long row (one element 10 rms off
# moves a 262,144-wide row's relative L2 by only 0.02) but not from this guard (0.127 rms there,
# 0.112 rms at n = 2816, 0.097 rms at n = 64).
GUARD_DELTA = 1e-3


def guard_factor(n, rel=REL_TOL):
    """Elementwise guard in units of rms(row) for rows of n elements (see GUARD_DELTA)."""
    return rel * np.sqrt(2.0 * np.log(2.0 * n / GUARD_DELTA))


def assert_close_rel(gpu, ref, rel=REL_TOL, what=""):
    """Hidden states, logits, cache rows: every row (vector along the last axis) within
    ||a - b||_2 <= rel ||b||_2, the whole array too, and no element beyond
    rel |b| + guard_factor(n) rms(row) (a guard against isolated gross errors)."""
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
    bad = np.abs(g2 - r2) > rel * np.abs(r2) + guard_factor(r2.shape[1], rel) * rms
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


# ---- routing near-ties: the GPU's expert choice, checked for validity, drives the oracle -------

def check_forced_routing(r_ref, r_gpu, idx_gpu, top_k, what=""):
    """Validity of the GPU's expert sets against the oracle's router logits.

    A near-tie between the k-th and (k+1)-th router logit leaves two correct expert sets, and
    which one a side picks depends on its rounding.  For every row the GPU's set must be a top-k
    of logits within that row's observed error of the oracle's: with err = max_e |r_gpu - r_ref|
    on the row, every chosen expert's oracle logit is >= every other expert's minus 2 err (ties
    and the k-th/(k+1)-th swaps inside that band are the only freedom).  The oracle is then run
    with the GPU's sets (oracle.model.route's force_idx), so every row can be compared at the
    stated tolerance.  Returns the number of rows whose set differs from the oracle's own."""
    r_ref = np.asarray(r_ref, dtype=np.float64).reshape(-1, np.shape(r_ref)[-1])
    r_gpu = np.asarray(r_gpu, dtype=np.float64).reshape(r_ref.shape)
    idx = np.asarray(idx_gpu, dtype=np.int64).reshape(-1, top_k)
    T, E = r_ref.shape
    err = np.abs(r_gpu - r_ref).max(axis=1)
    chosen = np.zeros((T, E), dtype=bool)
    np.put_along_axis(chosen, idx, True, axis=1)
    assert np.all(chosen.sum(axis=1) == top_k), f"{what}: repeated expert in a GPU top-k set"
    lo_in = np.where(chosen, r_ref, np.inf).min(axis=1)
    hi_out = np.where(chosen, -np.inf, r_ref).max(axis=1) if top_k < E else np.full(T, -np.inf)
    bad = lo_in < hi_out - 2.0 * err - 1e-12
    assert not bad.any(), (f"{what}: {bad.sum()} rows whose GPU expert set is not a top-{top_k} "
                           f"within the observed router error")
    own = np.argsort(-r_ref, axis=1, kind="stable")[:, :top_k]
    own_mask = np.zeros((T, E), dtype=bool)
    np.put_along_axis(own_mask, own, True, axis=1)
    return int(np.sum(np.any(own_mask != chosen, axis=1)))


class GpuChain:
    """The GPU's own layer chain, one dg_layer_forward call per layer on the GPU's residual
    stream, starting from the embedding rows (an exact bf16 -> fp32 copy, as the step's embed
    kernel makes).  These are the kernels, launch shapes and norm values of dg_decoder_step
    (causal = 0) and of the canvas append (causal = 1: each layer also writes its keys and
    values at [len, len + C)), so the chain's router logits and top-k sets are the step's own.

    Attributes: h (torch fp32 [T, d], the final residual stream), logits (per layer [T, E]),
    idx (per layer [B, C, k])."""

    def __init__(self, dims, model, kv, ws, tokens, embed, causal=False, n_layers=None):
        import torch
        from block_diffusion_decoding_canvas_amd import driver
        tokens = np.asarray(tokens)
        B, C = tokens.shape
        T, k = B * C, dims["top_k"]
        h0 = np.asarray(embed, dtype=np.float32)[tokens.reshape(-1)]
        self.h = torch.from_numpy(np.ascontiguousarray(h0)).to("cuda")
        self.logits, self.idx = [], []
        for layer in range(dims["n_layers"] if n_layers is None else n_layers):
            rl = torch.zeros((T, dims["E"]), dtype=torch.float32, device="cuda")
            ti = torch.zeros((T, k), dtype=torch.int32, device="cuda")
            driver.layer_forward(model, kv, layer, int(causal), self.h, ws, rl, ti, None)
            torch.cuda.synchronize()
            self.logits.append(rl.cpu().numpy().astype(np.float64))
            self.idx.append(ti.cpu().numpy().astype(np.int64).reshape(B, C, k))

    def check(self, infos, top_k, what=""):
        """check_forced_routing for every layer against the oracle's routing infos (run with
        force_idx = self.idx); returns the rows per layer whose set differs from the oracle's."""
        return [check_forced_routing(info["router_logits"], rl, ix, top_k, f"{what} layer {l}")
                for l, (info, rl, ix) in enumerate(zip(infos, self.logits, self.idx))]


def ffn_forced(model, lw_ref, dims, layer, batch, h, ws, what="", rows=None):
    """The FFN half-layer on the GPU (dg_ffn_forward) from the residual stream h [T, d] as fp32,
    and the oracle's FFN (weights lw_ref) on the same fp32 values with the GPU's expert sets,
    after checking them (check_forced_routing).  rows: compare only these token rows (the oracle
    computes only them).  Returns (GPU increment, oracle increment, rows with a near-tie expert
    swap), both increments [n, d] fp64."""
    import torch
    from block_diffusion_decoding_canvas_amd import driver
    from oracle import model as om
    h32 = np.ascontiguousarray(np.asarray(h, dtype=np.float32).reshape(-1, dims["d"]))
    T = h32.shape[0]
    hg = torch.from_numpy(h32.copy()).to("cuda")
    rl = torch.zeros((T, dims["E"]), dtype=torch.float32, device="cuda")
    ti = torch.zeros((T, dims["top_k"]), dtype=torch.int32, device="cuda")
    driver.ffn_forward(model, layer, batch, hg, ws, rl, ti)
    torch.cuda.synchronize()
    sel = np.arange(T) if rows is None else np.asarray(rows)
    h_in = h32[sel].astype(np.float64)
    idx = ti.cpu().numpy().astype(np.int64)[sel]
    f, info = om.moe(om.rms_norm(h_in, lw_ref["ffn_norm"], dims["eps"]), lw_ref, dims["top_k"],
                     force_idx=idx)
    swaps = check_forced_routing(info["router_logits"], rl.cpu().numpy()[sel], idx,
                                 dims["top_k"], what)
    return hg.cpu().numpy().astype(np.float64)[sel] - h_in, f, swaps


def prefill_chain(dims, model, kv, ws, prompt, split, embed):
    """The chunked prefill of prompt [n] into canvas 0.. of kv, run layer by layer through
    dg_layer_forward_tokens (the kernels and launch shapes dg_kv_append_tokens runs for each
    call), advancing kv.len after each call.  Returns (expert sets per layer [1, n, k], router
    logits per layer [n, E], residual stream after layer 0 [n, d] as fp64)."""
    import torch
    from block_diffusion_decoding_canvas_amd import driver
    prompt = np.asarray(prompt)
    k = dims["top_k"]
    idx = [[] for _ in range(dims["n_layers"])]
    logits = [[] for _ in range(dims["n_layers"])]
    h_after0 = []
    c0 = 0
    for n in split:
        h = torch.from_numpy(np.ascontiguousarray(
            np.asarray(embed, dtype=np.float32)[prompt[c0:c0 + n]])).to("cuda")
        for layer in range(dims["n_layers"]):
            rl = torch.zeros((n, dims["E"]), dtype=torch.float32, device="cuda")
            ti = torch.zeros((n, k), dtype=torch.int32, device="cuda")
            driver.layer_forward_tokens(model, kv, layer, h, ws, rl, ti)
            torch.cuda.synchronize()
            idx[layer].append(ti.cpu().numpy().astype(np.int64))
            logits[layer].append(rl.cpu().numpy().astype(np.float64))
            if layer == 0:
                h_after0.append(h.cpu().numpy().astype(np.float64))
        kv.len[0] += n
        c0 += n
    assert c0 == prompt.shape[0]
    return ([np.concatenate(x)[None] for x in idx], [np.concatenate(x) for x in logits],
            np.concatenate(h_after0))


def oracle_encode_forced(dims, mnp, prompt, cap, force, window_split=None):
    """The oracle's encoding of the prompt into an empty cache (one pass, or the given split),
    with the GPU's expert sets; returns (cache, routing infos per layer)."""
    from block_diffusion_decoding_canvas_amd import synth
    from oracle import model as om
    m64 = synth.model_to_f64(mnp)
    ref = synth.empty_cache(dims, 1, cap)
    ref = dict(k=[a.astype(np.float64) for a in ref["k"]], v=[a.astype(np.float64) for a in ref["v"]],
               len=np.array(ref["len"]))
    n_all = prompt.shape[0]
    infos = [None] * dims["n_layers"]
    parts = window_split or (n_all,)
    c0 = 0
    for n in parts:
        f = [x[:, c0:c0 + n] for x in force]
        h = m64["embed"][prompt[None, c0:c0 + n]]
        for layer, lw in enumerate(m64["layers"]):
            h, _, _, info = om.layer_forward(h, lw, dims, layer, ref["k"][layer], ref["v"][layer],
                                             ref["len"], causal=True, force_idx=f[layer])
            infos[layer] = info if infos[layer] is None else {
                key: np.concatenate([infos[layer][key], info[key]]) for key in info}
        om.encoder_append(prompt[None, c0:c0 + n], m64, ref, force_idx=f)
        c0 += n
    return ref, infos
