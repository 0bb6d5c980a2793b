"""Entropy-bound (EB) sampler: one denoising step of the canvas, written plainly in fp64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix (DiffusionGemma model card, Best Practices section 1 "diffusion sampling
settings", in all three language versions; diffusers DiffusionGemmaPipeline docs, sections
"Schedulers" and "Adaptive stopping" and the ``__call__`` parameters):
  * at most 48 denoising steps per canvas;
  * a temperature used to shape the logits, decaying linearly from 0.8 at the first step to 0.4
    at the last one (EntropyBoundScheduler ``t_max`` / ``t_min``);
  * every step commits the lowest-entropy positions while their entropy, taken jointly, stays
    under ``entropy_bound`` = 0.1, so that roughly independent tokens are accepted together;
  * the positions not selected are fully renoised; the corruption is uniform (no mask token);
  * a canvas stops early only when its mean per-token entropy of the scheduler-shaped logits is
    below 0.005 and its argmax predictions have stayed the same for ``stability_threshold`` = 1
    step, i.e. on two consecutive steps; each sample in a batch freezes on its own;
    ``confidence_threshold=None`` always runs every step.

Readings taken where the pages are silent:
  * entropy in nats; T_s = t_max + (t_min - t_max) * s / (S - 1) in fp64, S = max_steps
    (S = 1 gives t_max); the device multiplies by fp32(1 / T_s), and so does this oracle;
  * the statistics read the bf16 logits the decoder returns; argmax is over those logits,
    lowest index on ties (the temperature does not move it);
  * "entropy jointly under the bound" is the sum of the marginal entropies of the positions
    committed in this step, summed in fp64 in ascending (entropy, position) order, <= bound;
    zero commits in a step are allowed;
  * committed positions keep their token and leave the pool; the committed value is a sample from
    softmax(z / T_s), drawn by the Gumbel-max rule with Philox noise;
  * the stop test compares the argmax at every position (committed ones included) with the
    previous step's, so it can hold from step 1 on; stop when stable_count >= stability and
    mean entropy < stop_entropy (strict), stop_entropy < 0 disables it;
  * a canvas is finalised when it stops, at the last step, or when nothing is left
    uncommitted; finalising sets every uncommitted position to its argmax; a canvas whose
    positions are all committed is done;
  * order inside a step: statistics, stability, finalise?, select, candidates, renoise;
  * Philox counters (see ``oracle/philox.py``): key = (seed low word, seed high word);
    counter = (w0, position, step tag, (canvas_id << 1) | stream).  Renoise and the initial
    canvas use stream 0, w0 = 0 and the first output word x0, token = (x0 * V) >> 32, with step
    tag = step (renoise) or 0xFFFFFFFF (initial canvas).  Gumbel noise for vocabulary entry v
    uses stream 1, w0 = v >> 2 and output word v & 3 = x; u = (x + 0.5) / 2**32;
    g = -ln(-ln u); the candidate is argmax_v (z_v * fp32(1/T_s) + g_v) in fp64, lowest v on ties.
"""
import numpy as np

from .philox import philox4x32_10, seed_key

INIT_STEP_TAG = 0xFFFFFFFF


def default_params():
    """Sampler constants as the pages give them (model card Best Practices section 1)."""
    return dict(max_steps=48, t_max=0.8, t_min=0.4, entropy_bound=0.1,
                stop_entropy=0.005, stability=1)


def temperature(step, max_steps, t_max=0.8, t_min=0.4):
    """Linear temperature schedule from t_max at step 0 to t_min at step max_steps - 1 (fp64)."""
    if max_steps <= 1:
        return float(t_max)
    return float(t_max) + (float(t_min) - float(t_max)) * float(step) / float(max_steps - 1)


def inv_temperature_f32(step, max_steps, t_max=0.8, t_min=0.4):
    """The fp32 multiplier 1 / T_s that shapes the logits."""
    return np.float32(1.0 / temperature(step, max_steps, t_max, t_min))


def entropy_argmax(z, inv_t):
    """Entropy (nats) of softmax(z * inv_t) along the last axis, and argmax of z (first index).

    z holds bf16 values as float64; inv_t is the fp32 multiplier.
    """
    z = np.asarray(z, dtype=np.float64)
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite logits")
    y = z * np.float64(inv_t)
    m = y.max(axis=-1, keepdims=True)
    e = np.exp(y - m)
    p = e / e.sum(axis=-1, keepdims=True)
    logp = np.log(np.where(p > 0, p, 1.0))
    h = -(p * logp).sum(axis=-1)
    return h, z.argmax(axis=-1)


def _philox_words(seed, w0, pos, step_tag, canvas_id, stream):
    k0, k1 = seed_key(seed)
    c3 = np.uint32(((int(canvas_id) << 1) | stream) & 0xFFFFFFFF)
    return philox4x32_10(w0, pos, np.uint32(step_tag & 0xFFFFFFFF), c3, k0, k1)


def uniform_tokens(seed, canvas_id, step_tag, positions, vocab):
    """Uniform token ids in [0, vocab) for the given canvas positions (stream 0)."""
    pos = np.asarray(positions, dtype=np.uint32)
    x0, _, _, _ = _philox_words(seed, np.zeros_like(pos), pos, step_tag, canvas_id, 0)
    return ((x0.astype(np.uint64) * np.uint64(vocab)) >> np.uint64(32)).astype(np.int64)


def gumbel_noise(seed, canvas_id, step, pos, vocab):
    """Gumbel(0, 1) noise g_v for every vocabulary entry of one position (fp64, stream 1)."""
    v = np.arange(vocab, dtype=np.uint64)
    w = _philox_words(seed, (v >> np.uint64(2)).astype(np.uint32), np.uint32(pos), step,
                      canvas_id, 1)
    words = np.stack(w, axis=0)                          # [4, vocab]
    x = words[(v & np.uint64(3)).astype(np.int64), np.arange(vocab)]
    u = (x.astype(np.float64) + 0.5) * 2.0 ** -32
    return -np.log(-np.log(u))


def gumbel_candidate(z_row, inv_t, seed, canvas_id, step, pos):
    """A draw from softmax(z_row * inv_t) by the Gumbel-max rule; also the top-2 score gap."""
    z_row = np.asarray(z_row, dtype=np.float64)
    score = z_row * np.float64(inv_t) + gumbel_noise(seed, canvas_id, step, pos, z_row.shape[0])
    c = int(np.argmax(score))
    top2 = np.partition(score, -2)[-2:] if score.shape[0] > 1 else np.array([score[0], -np.inf])
    return c, float(top2[1] - top2[0])


def init_canvas(seed, canvas_ids, canvas_len, vocab):
    """Initial canvases: independent uniform placeholder tokens (uniform corruption)."""
    return np.stack([uniform_tokens(seed, cid, INIT_STEP_TAG, np.arange(canvas_len), vocab)
                     for cid in canvas_ids])


def new_state(canvas):
    canvas = np.array(canvas, dtype=np.int64)
    b, c = canvas.shape
    return dict(canvas=canvas, committed=np.zeros((b, c), dtype=bool),
                prev_argmax=np.zeros((b, c), dtype=np.int64),
                stable_count=np.zeros(b, dtype=np.int64), done=np.zeros(b, dtype=bool))


def select_commits(h, uncommitted, bound):
    """Positions committed in a step: the longest (entropy, position)-ascending prefix of the
    uncommitted positions whose fp64 running entropy sum stays <= bound.

    Returns (selected positions in sorted order, sorted uncommitted order, running sums).
    """
    h = np.asarray(h, dtype=np.float64)
    cand = [i for i in range(h.shape[0]) if uncommitted[i]]
    order = sorted(cand, key=lambda i: (h[i], i))
    total = 0.0
    sums = []
    n = 0
    for i in order:
        nxt = total + h[i]
        sums.append(nxt)
        if nxt <= bound:
            total = nxt
            n += 1
        else:
            break
    return order[:n], order, sums


def eb_step(z, step, params, state, seed, canvas_ids):
    """One EB denoising step over a batch of canvases.

    z: [B, C, V] logits holding bf16 values (float64).  state: dict from ``new_state``; it is
    updated in place.  Returns dict(entropy [B,C], argmax [B,C], commit_now [B,C] bool,
    finalised [B] bool, selected list per canvas, sums list per canvas).
    """
    z = np.asarray(z, dtype=np.float64)
    bsz, clen, vocab = z.shape
    s_max = int(params["max_steps"])
    inv_t = inv_temperature_f32(step, s_max, params["t_max"], params["t_min"])
    ent = np.zeros((bsz, clen))
    amax = np.zeros((bsz, clen), dtype=np.int64)
    commit_now = np.zeros((bsz, clen), dtype=bool)
    finalised = np.zeros(bsz, dtype=bool)
    selected, sums_all = [], []
    for b in range(bsz):
        h, a = entropy_argmax(z[b], inv_t)
        ent[b], amax[b] = h, a
        selected.append([])
        sums_all.append([])
        if state["done"][b]:
            continue                                   # a frozen canvas never changes
        if step >= 1 and np.array_equal(a, state["prev_argmax"][b]):
            state["stable_count"][b] += 1
        else:
            state["stable_count"][b] = 0
        state["prev_argmax"][b] = a
        unc = ~state["committed"][b]
        stop = (params["stop_entropy"] >= 0
                and state["stable_count"][b] >= params["stability"]
                and float(np.mean(h)) < params["stop_entropy"])
        if stop or step == s_max - 1 or not unc.any():
            state["canvas"][b][unc] = a[unc]
            commit_now[b] = unc
            state["committed"][b][:] = True
            state["done"][b] = True
            finalised[b] = True
            continue
        sel, _, sums = select_commits(h, unc, params["entropy_bound"])
        selected[b] = sel
        sums_all[b] = sums
        for i in sel:
            c, _ = gumbel_candidate(z[b, i], inv_t, seed, canvas_ids[b], step, i)
            state["canvas"][b][i] = c
        sel_mask = np.zeros(clen, dtype=bool)
        sel_mask[sel] = True
        rest = np.nonzero(unc & ~sel_mask)[0]
        if rest.size:
            state["canvas"][b][rest] = uniform_tokens(seed, canvas_ids[b], step, rest, vocab)
        state["committed"][b][sel_mask] = True
        commit_now[b] = sel_mask
        if state["committed"][b].all():
            state["done"][b] = True
    return dict(entropy=ent, argmax=amax, commit_now=commit_now, finalised=finalised,
                selected=selected, sums=sums_all, inv_t=inv_t, step=step)
