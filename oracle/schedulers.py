"""The pipeline's two other samplers, one denoising step at a time, written plainly in fp64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix (diffusers DiffusionGemmaPipeline docs, "Schedulers", "Predictor-corrector
sampling", the class text and the ``__call__`` parameters; the schedulers are interchangeable,
only the commit/renoise rule changes):
  * BlockRefinementScheduler, the pipeline's default: each step commits the highest-confidence
    tokens -- those above ``threshold``, plus a uniform per-step quota -- and renoises the rest
    (uniform corruption, no mask token); ``editing_threshold`` also lets it re-edit committed
    tokens; it samples at the pipeline's fixed ``temperature`` (0.0 is greedy);
  * DiscreteDDIMScheduler: samples every position from the exact discrete posterior of the
    uniform corruption process (D3PM); it takes no parameters and its last step deterministically
    commits the predicted tokens; it samples at the fixed ``temperature`` too;
  * its leave-one-out predictor-corrector: ``corrector_steps`` Gibbs sweeps resample the
    lowest-confidence positions (``corrector_k`` of them) from the single-coordinate
    conditional of the noisy marginal, which leaves that marginal unchanged; for uniform
    diffusion the leave-one-out posterior follows from the denoiser in closed form; the sweeps
    are taken out of the ``num_inference_steps`` budget (fewer predictor steps, the same number
    of model forwards);
  * adaptive stopping is the pipeline's, for every scheduler: a sample freezes once its argmax
    held for ``stability_threshold`` steps and its mean entropy of the scheduler-shaped logits is
    below ``confidence_threshold``.

Readings (the pages give no formulas for any of this):
  * temperature T: the candidate of a position is its argmax (lowest index on ties) when T = 0,
    else a Gumbel-max draw from softmax(z / T) with the entropy-bound sampler's Philox stream 1;
    the model distribution p = softmax(z * fp32(1 / T_eff)) with T_eff = T, or 1 when T = 0
    (greedy picks the argmax, and p, the confidences and the stop test's entropy then use the
    unshaped logits);
  * BlockRefinement: confidence = p(candidate); the step's quota is the even share of the canvas,
    q_s = floor((s+1) C / S) - floor(s C / S), which commits the whole canvas in S steps; a step
    commits, among the uncommitted positions, every one with confidence > threshold plus the q_s
    most confident of the others (descending confidence, lower position first on ties); the last
    step commits every remaining position; with editing_threshold >= 0 a position committed
    before the step takes its candidate when that differs from its token and its confidence is >
    editing_threshold; the uncommitted, unselected positions are renoised uniformly; a canvas is
    done when every position is committed and editing is off, and after its last step;
  * DiscreteDDIM: forward corruption q(x_t | x_0) = alpha(t) [x_t = x_0] + (1 - alpha(t)) / V
    with the linear schedule alpha(t) = 1 - t; with P = S - corrector_steps predictor steps, the
    predictor at call step s < P - 1 moves from t_s = 1 - s / P to t_{s+1}; each position draws
    its next token from sum_m p(m) q(x_{t_{s+1}} | x_{t_s} = current, x_0 = m) (Bayes' rule on
    the forward chain); the corrector sweeps are call steps P - 1 .. S - 2, at the last noisy
    level t_{P-1} = 1 / P; the final call step S - 1 sets every position to its argmax and
    commits the canvas; before that nothing is committed;
  * corrector: the confidence of a position is p(current token); a sweep resamples the
    corrector_k least confident (lower position first on ties), all from the same forward, each
    from alpha p_loo(k) + (1 - alpha) / V, where p_loo(m) is proportional to
    p(m) / q(current | x_0 = m) (the leave-one-out posterior: the denoiser's posterior divided by
    the likelihood of the coordinate it saw);
  * order inside a step: statistics, stability, finalise?, candidates, commit, edit, renoise.
"""
import numpy as np

from .sampler import entropy_argmax, gumbel_noise, uniform_tokens

BLOCK_REFINEMENT = "block_refinement"
DISCRETE_DDIM = "discrete_ddim"


def default_params(kind):
    """Constants of each scheduler; the adaptive-stop pair is the pipeline's default."""
    base = dict(max_steps=48, temperature=0.0, stop_entropy=0.005, stability=1)
    if kind == BLOCK_REFINEMENT:
        return dict(base, kind=kind, threshold=0.9, editing_threshold=-1.0)
    if kind == DISCRETE_DDIM:
        return dict(base, kind=kind, corrector_steps=0, corrector_k=0)
    raise ValueError(kind)


def inv_temperature_f32(temperature):
    """The fp32 multiplier of the logits: 1 / T, or 1 for greedy (T = 0)."""
    t = float(temperature)
    return np.float32(1.0 / t) if t > 0.0 else np.float32(1.0)


def model_probs(z_row, inv_t):
    """p = softmax(z * inv_t) of one row, fp64."""
    y = np.asarray(z_row, dtype=np.float64) * np.float64(inv_t)
    e = np.exp(y - y.max())
    return e / e.sum()


def quota(step, max_steps, canvas_len):
    """Block refinement's even per-step share of the canvas."""
    s, n, c = int(step), int(max_steps), int(canvas_len)
    return (s + 1) * c // n - s * c // n


def gumbel_sample(logw, seed, canvas_id, step, pos):
    """argmax_v (log w_v + g_v) with the sampler's Gumbel noise (Philox stream 1), lowest v on
    ties; also the top-2 score gap."""
    logw = np.asarray(logw, dtype=np.float64)
    score = logw + gumbel_noise(seed, canvas_id, step, pos, logw.shape[0])
    c = int(np.argmax(score))
    top2 = np.partition(score, -2)[-2:]
    return c, float(top2[1] - top2[0])


def candidate(z_row, temperature, inv_t, seed, canvas_id, step, pos):
    """The candidate token of a position and its confidence p(candidate)."""
    p = model_probs(z_row, inv_t)
    if float(temperature) > 0.0:
        c, gap = gumbel_sample(np.log(p), seed, canvas_id, step, pos)
    else:
        c, gap = int(np.argmax(z_row)), np.inf
    return c, float(p[c]), gap


# ---- the uniform (D3PM) corruption process ----------------------------------------------------

def alpha(t):
    """Probability that a token survives corruption to time t (linear schedule)."""
    return 1.0 - float(t)


def forward_prob(x_t, x0, t, vocab):
    """q(x_t | x_0) of the uniform corruption."""
    a = alpha(t)
    return a * (x_t == x0) + (1.0 - a) / vocab


def transition(t, vocab):
    """The forward corruption matrix Q_t[m, k] = q(x_t = k | x_0 = m) (a dense V x V array; the
    pins use it on small vocabularies)."""
    a = alpha(t)
    return a * np.eye(vocab) + (1.0 - a) / vocab


def apply_transition(r, t):
    """sum_m r(m) Q_t[m, k] for every k: Q_t is a times the identity plus (1 - a) / V times the
    all-ones matrix, so the product is a r + (1 - a) mean(r)."""
    r = np.asarray(r, dtype=np.float64)
    a = alpha(t)
    return a * r + (1.0 - a) * r.sum() / r.shape[0]


def ddim_posterior(p, current, t, t_next):
    """Distribution of the token at time t_next < t given the token `current` at time t, with
    x_0 ~ p: sum_m p(m) q(x_{t_next} = k | x_t = current, x_0 = m).  Bayes' rule on the forward
    chain gives q(k | j, m) = q(j | k; t given t_next) q(k | m; t_next) / q(j | m; t), where the
    one-step transition from t_next to t keeps a token with probability
    alpha(t) / alpha(t_next); the sum over m is the transition Q_{t_next} applied to
    r(m) = p(m) / q(j | m; t)."""
    p = np.asarray(p, dtype=np.float64)
    V = p.shape[0]
    j = int(current)
    k = np.arange(V)
    a_step = alpha(t) / alpha(t_next)
    step_prob = a_step * (j == k) + (1.0 - a_step) / V            # q(x_t = j | x_{t_next} = k)
    r = p / forward_prob(j, k, t, V)
    return step_prob * apply_transition(r, t_next)


def loo_posterior(p, current, t):
    """Leave-one-out posterior of a coordinate: p_loo(m) proportional to
    p(m) / q(x_t = current | x_0 = m)."""
    p = np.asarray(p, dtype=np.float64)
    V = p.shape[0]
    w = p / forward_prob(int(current), np.arange(V), t, V)
    return w / w.sum()


def corrector_conditional(p, current, t):
    """Single-coordinate conditional of the noisy marginal at time t:
    sum_m p_loo(m) q(x_t = k | x_0 = m) = alpha(t) p_loo(k) + (1 - alpha(t)) / V."""
    p_loo = loo_posterior(p, current, t)
    V = p_loo.shape[0]
    return alpha(t) * p_loo + (1.0 - alpha(t)) / V


def ddim_phase(step, max_steps, corrector_steps):
    """What call step `step` does: ("predict", t, t_next), ("correct", t) or ("final",)."""
    S, c = int(max_steps), int(corrector_steps)
    P = S - c
    if not (0 <= c and P >= 1):
        raise ValueError("need 0 <= corrector_steps <= max_steps - 1")
    s = int(step)
    if s == S - 1:
        return ("final",)
    if s < P - 1:
        return ("predict", 1.0 - s / P, 1.0 - (s + 1) / P)
    return ("correct", 1.0 / P)


# ---- one step over a batch of canvases ----------------------------------------------------------

def _one_hot(i, n):
    v = np.zeros(n)
    v[int(i)] = 1.0
    return v


def _prelude(zb, step, params, state, b, inv_t):
    """Statistics, stability and the adaptive-stop test of canvas b (the pipeline's rule)."""
    h, a = entropy_argmax(zb, inv_t)
    if step >= 1 and np.array_equal(a, state["prev_argmax"][b]):
        state["stable_count"][b] += 1
    else:
        state["stable_count"][b] = 0
    state["prev_argmax"][b] = a
    stop = (params["stop_entropy"] >= 0
            and state["stable_count"][b] >= params["stability"]
            and float(np.mean(h)) < params["stop_entropy"])
    return h, a, stop


def _finalise(state, b, a, commit_now):
    unc = ~state["committed"][b]
    state["canvas"][b][unc] = a[unc]
    commit_now[b] = unc
    state["committed"][b][:] = True
    state["done"][b] = True


def block_refinement_step(z, step, params, state, seed, canvas_ids):
    """One BlockRefinement step over canvases; z [B, C, V] holds the bf16 logits (float64).
    state is updated in place.  Returns dict(entropy, argmax, commit_now, cand, conf, gap,
    selected, edited)."""
    z = np.asarray(z, dtype=np.float64)
    B, C, V = z.shape
    S, T = int(params["max_steps"]), float(params["temperature"])
    inv_t = inv_temperature_f32(T)
    ent = np.zeros((B, C))
    amax = np.zeros((B, C), dtype=np.int64)
    commit_now = np.zeros((B, C), dtype=bool)
    cand = np.full((B, C), -1, dtype=np.int64)
    conf = np.full((B, C), np.nan)
    gap = np.full((B, C), np.inf)
    selected, edited = [[] for _ in range(B)], [[] for _ in range(B)]
    editing = params["editing_threshold"] >= 0
    for b in range(B):
        if state["done"][b]:
            ent[b], amax[b] = entropy_argmax(z[b], inv_t)
            continue
        h, a, stop = _prelude(z[b], step, params, state, b, inv_t)
        ent[b], amax[b] = h, a
        unc = ~state["committed"][b]
        if stop:
            _finalise(state, b, a, commit_now)
            continue
        need = unc | state["committed"][b] if editing else unc
        for i in np.nonzero(need)[0]:
            cand[b, i], conf[b, i], gap[b, i] = candidate(z[b, i], T, inv_t, seed,
                                                           canvas_ids[b], step, i)
        order = sorted(np.nonzero(unc)[0], key=lambda i: (-conf[b, i], i))
        n_above = sum(1 for i in order if conf[b, i] > params["threshold"])
        n = len(order) if step == S - 1 else min(len(order), n_above + quota(step, S, C))
        sel = order[:n]
        selected[b] = list(sel)
        committed_before = state["committed"][b].copy()
        for i in sel:
            state["canvas"][b][i] = cand[b, i]
            state["committed"][b][i] = True
            commit_now[b, i] = True
        if editing:
            for i in np.nonzero(committed_before)[0]:
                if cand[b, i] != state["canvas"][b][i] and conf[b, i] > params["editing_threshold"]:
                    state["canvas"][b][i] = cand[b, i]
                    edited[b].append(int(i))
        rest = np.nonzero(unc & ~commit_now[b])[0]
        if rest.size:
            state["canvas"][b][rest] = uniform_tokens(seed, canvas_ids[b], step, rest, V)
        if step == S - 1 or (state["committed"][b].all() and not editing):
            state["done"][b] = True
    return dict(entropy=ent, argmax=amax, commit_now=commit_now, cand=cand, conf=conf, gap=gap,
                selected=selected, edited=edited, inv_t=inv_t, step=step)


def discrete_ddim_step(z, step, params, state, seed, canvas_ids):
    """One DiscreteDDIM call step (predictor, corrector sweep or the final deterministic step)
    over canvases; z [B, C, V] bf16 logits (float64); state updated in place.  Returns
    dict(entropy, argmax, commit_now, phase, resampled (positions drawn per canvas), gap)."""
    z = np.asarray(z, dtype=np.float64)
    B, C, V = z.shape
    S, T = int(params["max_steps"]), float(params["temperature"])
    inv_t = inv_temperature_f32(T)
    phase = ddim_phase(step, S, params["corrector_steps"])
    ent = np.zeros((B, C))
    amax = np.zeros((B, C), dtype=np.int64)
    commit_now = np.zeros((B, C), dtype=bool)
    gap = np.full((B, C), np.inf)
    resampled = [[] for _ in range(B)]
    for b in range(B):
        if state["done"][b]:
            ent[b], amax[b] = entropy_argmax(z[b], inv_t)
            continue
        h, a, stop = _prelude(z[b], step, params, state, b, inv_t)
        ent[b], amax[b] = h, a
        if stop or phase[0] == "final":
            _finalise(state, b, a, commit_now)
            continue
        x = state["canvas"][b]
        probs = [model_probs(z[b, i], inv_t) if T > 0.0 else _one_hot(a[i], V) for i in range(C)]
        if phase[0] == "predict":
            rows = list(range(C))
        else:
            conf = [probs[i][x[i]] for i in range(C)]
            rows = sorted(range(C), key=lambda i: (conf[i], i))[:int(params["corrector_k"])]
        new = x.copy()
        for i in rows:
            if phase[0] == "predict":
                w = ddim_posterior(probs[i], x[i], phase[1], phase[2])
            else:
                w = corrector_conditional(probs[i], x[i], phase[1])
            with np.errstate(divide="ignore"):
                new[i], gap[b, i] = gumbel_sample(np.log(w), seed, canvas_ids[b], step, i)
        state["canvas"][b][:] = new
        resampled[b] = sorted(rows)
    return dict(entropy=ent, argmax=amax, commit_now=commit_now, phase=phase,
                resampled=resampled, gap=gap, inv_t=inv_t, step=step)
