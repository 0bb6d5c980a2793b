"""Pins of the oracle's BlockRefinement and DiscreteDDIM steps (oracle/schedulers.py): brute force
over explicit transition matrices on small vocabularies, invariants the pages state (the
corrector keeps the noisy marginal; the last DDIM step commits the predictions), closed forms,
library routines (scipy softmax and chi-square) and hand-built canvases."""
import copy

import numpy as np
import pytest
from scipy import special, stats

from oracle import sampler as osamp
from oracle import schedulers as osch


# ---- shared pieces ----------------------------------------------------------------------------

def test_quota_is_an_even_split_of_the_canvas():
    for C, S in [(256, 48), (16, 8), (40, 6), (7, 10), (1, 1)]:
        q = [osch.quota(s, S, C) for s in range(S)]
        assert sum(q) == C
        assert set(q) <= {C // S, -(-C // S)}
    q = [osch.quota(s, 48, 256) for s in range(48)]
    assert q.count(6) == 16 and q.count(5) == 32


def test_model_probs_and_temperature_multiplier():
    z = np.random.default_rng(0).standard_normal(300) * 3
    for T in (0.0, 0.5, 1.0, 1.7):
        inv = osch.inv_temperature_f32(T)
        assert inv == (np.float32(1.0) if T == 0 else np.float32(1.0 / T))
        assert np.allclose(osch.model_probs(z, inv), special.softmax(z * float(inv)),
                           rtol=1e-13, atol=1e-16)


def test_gumbel_sample_frequencies_match_weights():
    rng = np.random.default_rng(1)
    w = rng.uniform(0.1, 1.0, 6)
    w /= w.sum()
    counts = np.zeros(6)
    for pos in range(4000):
        c, _ = osch.gumbel_sample(np.log(w), 5, 3, 11, pos)
        counts[c] += 1
    assert stats.chisquare(counts, w * counts.sum()).pvalue > 1e-3


# ---- BlockRefinement ---------------------------------------------------------------------------

def _br_params(**kw):
    p = osch.default_params(osch.BLOCK_REFINEMENT)
    p.update(kw)
    return p


def _rows(C, V, seed, sharp=None):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((1, C, V))
    if sharp is not None:
        for i, s in enumerate(sharp):
            z[0, i, rng.integers(V)] += s
    return z


def test_block_refinement_greedy_commits_the_quota_by_confidence():
    """threshold above 1 (never met), T = 0: each step commits exactly its quota, the most
    confident uncommitted positions by softmax maximum (scipy), candidates are the argmax; the
    rest is renoised; after S steps everything is committed and the canvas is done."""
    C, V, S = 12, 40, 5
    p = _br_params(max_steps=S, threshold=2.0, stop_entropy=-1.0)
    st = osamp.new_state(osamp.init_canvas(3, [0], C, V))
    for s in range(S):
        z = _rows(C, V, 10 + s, sharp=np.linspace(0, 6, C))
        before = copy.deepcopy(st)
        ref = osch.block_refinement_step(z, s, p, st, 3, [0])
        conf = special.softmax(z[0], axis=1).max(axis=1)
        unc = np.nonzero(~before["committed"][0])[0]
        want = sorted(unc, key=lambda i: (-conf[i], i))[:osch.quota(s, S, C)]
        assert sorted(np.nonzero(ref["commit_now"][0])[0]) == sorted(want)
        assert np.allclose(ref["conf"][0, unc], conf[unc], rtol=1e-12)
        for i in want:
            assert st["canvas"][0][i] == np.argmax(z[0, i])
        rest = [i for i in unc if i not in want]
        assert np.array_equal(st["canvas"][0][rest],
                              osamp.uniform_tokens(3, 0, s, np.array(rest), V))
        committed_before = np.nonzero(before["committed"][0])[0]
        assert np.array_equal(st["canvas"][0][committed_before],
                              before["canvas"][0][committed_before])
    assert st["committed"].all() and st["done"].all()


def test_block_refinement_threshold_adds_to_the_quota():
    """Positions above the threshold all commit, plus the quota's most confident of the others;
    brute force: the committed set is the largest confidence-ordered prefix of that size."""
    C, V, S = 16, 64, 8
    z = _rows(C, V, 21, sharp=[12, 12, 12, 0, 0, 9, 0, 0, 12, 0, 0, 0, 3, 0, 0, 0])
    conf = special.softmax(z[0], axis=1).max(axis=1)
    for thr in (0.5, 0.95, 0.999):
        st = osamp.new_state(osamp.init_canvas(4, [0], C, V))
        ref = osch.block_refinement_step(z, 0, _br_params(max_steps=S, threshold=thr), st, 4, [0])
        above = set(np.nonzero(conf > thr)[0])
        others = sorted(set(range(C)) - above, key=lambda i: (-conf[i], i))
        want = above | set(others[:osch.quota(0, S, C)])
        assert set(np.nonzero(ref["commit_now"][0])[0]) == want, thr
    # threshold 0: every confidence is positive, so the whole canvas commits at once
    st = osamp.new_state(osamp.init_canvas(4, [0], C, V))
    ref = osch.block_refinement_step(z, 0, _br_params(max_steps=S, threshold=0.0), st, 4, [0])
    assert ref["commit_now"].all() and st["done"].all()


def test_block_refinement_ties_take_the_lower_position():
    C, V = 6, 10
    z = np.zeros((1, C, V))
    z[0, :, 3] = 2.0                                       # identical rows, identical confidence
    st = osamp.new_state(osamp.init_canvas(1, [0], C, V))
    ref = osch.block_refinement_step(z, 0, _br_params(max_steps=3, threshold=2.0), st, 1, [0])
    assert list(np.nonzero(ref["commit_now"][0])[0]) == [0, 1]


def test_block_refinement_sampled_candidates_and_confidence():
    """T > 0: the candidate is a draw from softmax(z / T) (chi-square over many positions of a
    fixed row), and its confidence is that distribution's probability of the draw."""
    V, T = 5, 0.7
    row = np.array([0.5, -1.0, 1.2, 0.0, 0.3])
    inv = osch.inv_temperature_f32(T)
    probs = special.softmax(row * float(inv))
    counts = np.zeros(V)
    for pos in range(3000):
        c, conf, _ = osch.candidate(row, T, inv, 9, 2, 4, pos)
        assert abs(conf - probs[c]) < 1e-13
        counts[c] += 1
    assert stats.chisquare(counts, probs * counts.sum()).pvalue > 1e-3


def test_block_refinement_editing():
    """A committed position whose candidate differs and is confident enough takes the candidate;
    a less confident one keeps its token; with editing off committed tokens never change."""
    C, V = 4, 20
    z = np.full((1, C, V), -5.0)
    z[0, 0, 7] = 8.0          # confident prediction 7
    z[0, 1, :] = 0.0
    z[0, 1, 9] = 0.5          # weak prediction 9 (confidence about 0.08)
    z[0, 2, 3] = 8.0
    z[0, 3, 4] = 8.0
    st0 = osamp.new_state(np.array([[1, 2, 3, 5]]))
    st0["committed"][0, :2] = True
    for e, want in [(0.5, [7, 2]), (-1.0, [1, 2])]:
        st = copy.deepcopy(st0)
        ref = osch.block_refinement_step(z, 1, _br_params(max_steps=4, threshold=2.0,
                                                          editing_threshold=e), st, 6, [0])
        assert list(st["canvas"][0, :2]) == want
        assert (ref["edited"][0] == [0]) == (e >= 0)
        assert st["committed"][0, :2].all()


def test_block_refinement_adaptive_stop_finalises_to_argmax():
    C, V = 8, 30
    z = np.full((1, C, V), -30.0)
    top = np.arange(C) * 3
    z[0, np.arange(C), top] = 30.0                         # entropy ~ 0
    st = osamp.new_state(osamp.init_canvas(2, [0], C, V))
    st["prev_argmax"][0] = top
    ref = osch.block_refinement_step(z, 3, _br_params(max_steps=10, threshold=2.0), st, 2, [0])
    assert st["done"][0] and st["committed"].all()
    assert np.array_equal(st["canvas"][0], top) and ref["commit_now"].all()


# ---- DiscreteDDIM ------------------------------------------------------------------------------

def _brute_posterior(p, j, t, t_next):
    """Mixture over x_0 ~ p of the conditional of x_{t_next} given (x_t = j, x_0), each found by
    normalising the explicit two-step joint Q_{t_next}[x0, k] Q_step[k, j] over k."""
    V = p.shape[0]
    a_step = osch.alpha(t) / osch.alpha(t_next)
    q_step = a_step * np.eye(V) + (1 - a_step) / V
    q_next = osch.transition(t_next, V)
    out = np.zeros(V)
    for m in range(V):
        joint = q_next[m, :] * q_step[:, j]
        out += p[m] * joint / joint.sum()
    return out


def test_transition_chapman_kolmogorov():
    V = 6
    for t, tn in [(1.0, 0.75), (0.5, 0.25), (0.2, 0.1)]:
        a_step = osch.alpha(t) / osch.alpha(tn)
        q_step = a_step * np.eye(V) + (1 - a_step) / V
        assert np.allclose(osch.transition(tn, V) @ q_step, osch.transition(t, V), atol=1e-15)
        r = np.random.default_rng(2).uniform(size=V)
        assert np.allclose(osch.apply_transition(r, t), r @ osch.transition(t, V), atol=1e-15)


@pytest.mark.parametrize("t,t_next", [(1.0, 0.9), (0.6, 0.4), (0.25, 0.125)])
def test_ddim_posterior_brute_force(t, t_next):
    rng = np.random.default_rng(3)
    V = 5
    for trial in range(6):
        p = rng.dirichlet(np.ones(V) * 0.5)
        if trial == 0:
            p = np.eye(V)[2]                                # a one-hot (greedy) denoiser
        for j in range(V):
            w = osch.ddim_posterior(p, j, t, t_next)
            assert np.all(w >= 0) and abs(w.sum() - 1) < 1e-13
            assert np.allclose(w, _brute_posterior(p, j, t, t_next), rtol=1e-12, atol=1e-15)


def test_ddim_posterior_closed_forms():
    V = 7
    p = np.random.default_rng(4).dirichlet(np.ones(V))
    # from pure noise (alpha(1) = 0) the current token carries nothing: forward-noise p
    b = osch.alpha(0.8)
    for j in range(V):
        assert np.allclose(osch.ddim_posterior(p, j, 1.0, 0.8), b * p + (1 - b) / V, atol=1e-15)
    # a perfect denoiser keeps the forward marginals: x_t ~ q_t(. | x0) maps to q_{t_next}(. | x0)
    for x0 in range(V):
        delta = np.eye(V)[x0]
        qt = osch.transition(0.6, V)[x0]
        mixed = sum(qt[j] * osch.ddim_posterior(delta, j, 0.6, 0.3) for j in range(V))
        assert np.allclose(mixed, osch.transition(0.3, V)[x0], atol=1e-15)


def test_corrector_recovers_the_prior_and_keeps_the_marginal():
    """For one coordinate with prior pi over x_0, the exact denoiser is p(m | j) proportional to
    pi(m) q(j | m); the leave-one-out posterior is pi for every observed j, and the corrector's
    conditional is the noisy marginal sum_m pi(m) q_t(k | m): a Gibbs update that leaves it
    unchanged (the property the pages state)."""
    V, t = 6, 0.4
    pi = np.random.default_rng(5).dirichlet(np.ones(V))
    Q = osch.transition(t, V)
    marginal = pi @ Q
    for j in range(V):
        p = pi * Q[:, j]
        p /= p.sum()
        assert np.allclose(osch.loo_posterior(p, j, t), pi, atol=1e-15)
        assert np.allclose(osch.corrector_conditional(p, j, t), marginal, atol=1e-15)


def test_ddim_phases():
    assert osch.ddim_phase(0, 48, 0) == ("predict", 1.0, 1.0 - 1 / 48)
    assert osch.ddim_phase(46, 48, 0) == ("predict", 1.0 - 46 / 48, 1.0 - 47 / 48)
    assert osch.ddim_phase(47, 48, 0) == ("final",)
    # two corrector sweeps out of the 48 forwards: 46 predictor steps, sweeps at 1 / 46
    assert osch.ddim_phase(44, 48, 2) == ("predict", 1.0 - 44 / 46, 1.0 - 45 / 46)
    assert osch.ddim_phase(45, 48, 2) == ("correct", 1.0 / 46)
    assert osch.ddim_phase(46, 48, 2) == ("correct", 1.0 / 46)
    assert osch.ddim_phase(47, 48, 2) == ("final",)
    kinds = [osch.ddim_phase(s, 10, 3)[0] for s in range(10)]
    assert kinds == ["predict"] * 6 + ["correct"] * 3 + ["final"]
    with pytest.raises(ValueError):
        osch.ddim_phase(0, 4, 4)


def _ddim_params(**kw):
    p = osch.default_params(osch.DISCRETE_DDIM)
    p.update(kw)
    return p


def test_ddim_step_predictor_final_and_corrector():
    C, V, S = 10, 24, 6
    rng = np.random.default_rng(6)
    z = rng.standard_normal((2, C, V)) * 2
    p = _ddim_params(max_steps=S, corrector_steps=2, corrector_k=3, temperature=0.8,
                     stop_entropy=-1.0)
    st = osamp.new_state(osamp.init_canvas(7, [0, 1], C, V))
    # predictor: every position redrawn from its posterior; nothing committed
    before = copy.deepcopy(st)
    ref = osch.discrete_ddim_step(z, 0, p, st, 7, [0, 1])
    assert ref["phase"][0] == "predict" and not ref["commit_now"].any()
    assert not st["committed"].any() and not st["done"].any()
    inv = osch.inv_temperature_f32(0.8)
    for b in range(2):
        for i in range(C):
            w = osch.ddim_posterior(special.softmax(z[b, i] * float(inv)), before["canvas"][b][i],
                                    *ref["phase"][1:])
            c, _ = osch.gumbel_sample(np.log(w), 7, b, 0, i)
            assert st["canvas"][b][i] == c
    # corrector sweep (step 3 of 6 with 2 sweeps: P = 4): the 3 least confident positions
    before = copy.deepcopy(st)
    ref = osch.discrete_ddim_step(z, 3, p, st, 7, [0, 1])
    assert ref["phase"] == ("correct", 0.25)
    for b in range(2):
        conf = [special.softmax(z[b, i] * float(inv))[before["canvas"][b][i]] for i in range(C)]
        want = sorted(sorted(range(C), key=lambda i: (conf[i], i))[:3])
        assert ref["resampled"][b] == want
        keep = [i for i in range(C) if i not in want]
        assert np.array_equal(st["canvas"][b][keep], before["canvas"][b][keep])
    # final step: every position takes its argmax and the canvas is committed and done
    ref = osch.discrete_ddim_step(z, S - 1, p, st, 7, [0, 1])
    assert np.array_equal(st["canvas"], z.argmax(axis=2))
    assert st["committed"].all() and st["done"].all() and ref["commit_now"].all()


def test_ddim_greedy_first_step_is_forward_noised_argmax():
    """Greedy (T = 0) from pure noise: a position keeps its argmax with probability
    b + (1 - b) / V and otherwise draws uniformly (b = alpha(t_1)); chi-square over positions."""
    C, V, S = 400, 8, 4
    z = np.random.default_rng(8).standard_normal((1, C, V))
    st = osamp.new_state(osamp.init_canvas(9, [0], C, V))
    osch.discrete_ddim_step(z, 0, _ddim_params(max_steps=S, stop_entropy=-1.0), st, 9, [0])
    b = osch.alpha(1.0 - 1.0 / S)
    hit = (st["canvas"][0] == z[0].argmax(axis=1)).sum()
    expect = C * (b + (1 - b) / V)
    assert stats.binomtest(int(hit), C, expect / C).pvalue > 1e-3
