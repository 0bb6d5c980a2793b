"""Pins of the oracle's EB sampler: closed forms, library routines, brute force, invariants."""
import copy
import itertools

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax
from scipy.stats import chisquare, entropy as sp_entropy

from oracle import sampler
from oracle.numerics import round_bf16

P = sampler.default_params()


# ---- entropy and argmax -------------------------------------------------------------------

def test_entropy_one_hot_is_zero():
    z = np.full((1, 512), -1e4)
    z[0, 77] = 0.0
    h, a = sampler.entropy_argmax(z, np.float32(1 / 0.8))
    assert h[0] == 0.0 and a[0] == 77


@pytest.mark.parametrize("logv", [9, 18])
def test_entropy_uniform_is_log_v(logv):
    h, _ = sampler.entropy_argmax(np.zeros((2, 1 << logv)), np.float32(1.25))
    assert np.allclose(h, logv * np.log(2.0), rtol=0, atol=1e-12)


def test_entropy_two_point_binary_entropy():
    for a, b, t in [(0.0, 1.0, 0.8), (3.0, -2.0, 0.4), (0.5, 0.5, 0.6)]:
        inv = np.float32(1.0 / t)
        h, _ = sampler.entropy_argmax(np.array([[a, b]]), inv)
        d = (a - b) * float(inv)
        p = 1.0 / (1.0 + np.exp(-d))
        assert abs(h[0] - sp_entropy([p, 1 - p])) < 1e-13


def test_entropy_matches_scipy_on_random_rows():
    rng = np.random.default_rng(0)
    z = round_bf16(rng.standard_normal((20, 1000)) * 3)
    inv = np.float32(1 / 0.53)
    h, a = sampler.entropy_argmax(z, inv)
    ref = np.array([sp_entropy(sp_softmax(row * np.float64(inv))) for row in z])
    assert np.allclose(h, ref, rtol=1e-12, atol=1e-14)
    assert np.array_equal(a, z.argmax(axis=1))


def test_entropy_temperature_scaling_invariance():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((4, 300))
    h1, _ = sampler.entropy_argmax(z, 1.0)
    h2, _ = sampler.entropy_argmax(z * 4.0, 0.25)
    assert np.allclose(h1, h2, rtol=1e-12)


def test_argmax_lowest_index_on_ties():
    z = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]])
    _, a = sampler.entropy_argmax(z, np.float32(1.25))
    assert list(a) == [1, 0]


def test_nonfinite_logits_raise():
    with pytest.raises(ValueError):
        sampler.entropy_argmax(np.array([[0.0, np.nan]]), 1.0)


# ---- temperature schedule ----------------------------------------------------------------

def test_schedule_endpoints_and_midpoints():
    assert sampler.temperature(0, 48) == 0.8
    assert abs(sampler.temperature(47, 48) - 0.4) < 1e-15
    assert abs(sampler.temperature(24, 49) - 0.6) < 1e-15
    for s in range(8):
        assert abs(sampler.temperature(s, 8) - (0.8 - 0.4 * s / 7)) < 1e-15
    assert sampler.temperature(0, 1) == 0.8
    assert sampler.inv_temperature_f32(47, 48) == np.float32(2.5)


# ---- commit selection -------------------------------------------------------------------

def _brute_force_selection(h, unc, bound):
    """Largest subset of uncommitted positions that (a) holds the lowest (entropy, position)
    keys among the uncommitted ones and (b) has summed entropy <= bound."""
    pool = [i for i in range(len(h)) if unc[i]]
    best = ()
    for r in range(len(pool) + 1):
        for sub in itertools.combinations(pool, r):
            rest = [j for j in pool if j not in sub]
            if sub and rest and max((h[i], i) for i in sub) > min((h[j], j) for j in rest):
                continue
            if sum(sorted(h[i] for i in sub)) <= bound and len(sub) >= len(best):
                best = sub
    return set(best)


def test_selection_matches_brute_force():
    rng = np.random.default_rng(2)
    for trial in range(300):
        c = int(rng.integers(1, 11))
        h = rng.choice([0.0, 0.01, 0.02, 0.03, 0.05, 0.1], size=c) if trial % 3 == 0 \
            else rng.exponential(0.04, size=c)
        unc = rng.random(c) < 0.8
        bound = float(rng.choice([0.0, 0.05, 0.1, 0.3, 10.0]))
        sel, _, _ = sampler.select_commits(h, unc, bound)
        assert set(sel) == _brute_force_selection(h, unc, bound)


def test_selection_invariants():
    rng = np.random.default_rng(3)
    for _ in range(200):
        h = rng.exponential(0.05, size=256)
        unc = rng.random(256) < 0.7
        sel, order, _ = sampler.select_commits(h, unc, 0.1)
        assert sum(h[i] for i in sel) <= 0.1
        others = [i for i in range(256) if unc[i] and i not in set(sel)]
        if sel and others:
            assert max(h[i] for i in sel) <= min(h[i] for i in others)
        if len(sel) < len(order):
            assert sum(h[i] for i in sel) + h[order[len(sel)]] > 0.1
        assert all(unc[i] for i in sel)


def test_selection_bound_zero_and_huge():
    h = np.array([0.0, 0.3, 0.0, 1e-9])
    unc = np.ones(4, dtype=bool)
    assert sampler.select_commits(h, unc, 0.0)[0] == [0, 2]
    assert sorted(sampler.select_commits(h, unc, 1e9)[0]) == [0, 1, 2, 3]


# ---- Gumbel-max candidates --------------------------------------------------------------

def test_gumbel_frequencies_match_softmax():
    z = np.array([0.0, 1.0, -0.5, 2.0, 0.25, -3.0])
    inv = np.float32(1 / 0.8)
    n = 20000
    counts = np.zeros(6)
    for k in range(n):
        c, _ = sampler.gumbel_candidate(z, inv, 7, k % 5, k // 256, k % 256)
        counts[c] += 1
    p = sp_softmax(z * np.float64(inv))
    assert chisquare(counts, p * n).pvalue > 1e-4


def test_gumbel_low_temperature_is_argmax_and_spike_wins():
    rng = np.random.default_rng(4)
    z = round_bf16(rng.standard_normal(512))
    for pos in range(20):
        assert sampler.gumbel_candidate(z, np.float32(1e6), 2, 0, 3, pos)[0] == int(z.argmax())
    z2 = np.zeros(512)
    z2[300] = 1e4
    assert sampler.gumbel_candidate(z2, np.float32(1.25), 2, 0, 3, 5)[0] == 300


# ---- whole steps: stop rule, freezing, finalisation, determinism ---------------------------

def _peaked(c, v, idx, gap=40.0):
    z = np.zeros((c, v))
    z[np.arange(c), idx] = gap
    return z


def test_stop_fires_on_second_stable_low_entropy_step():
    p = dict(P, entropy_bound=0.0)
    st = sampler.new_state(np.zeros((1, 4), dtype=np.int64))
    z = _peaked(4, 8, [1, 2, 3, 4])[None]
    r0 = sampler.eb_step(z, 0, p, st, 2, [0])
    assert not st["done"][0] and not r0["commit_now"].any()
    r1 = sampler.eb_step(z, 1, p, st, 2, [0])
    assert st["done"][0] and r1["finalised"][0]
    assert list(st["canvas"][0]) == [1, 2, 3, 4]


def test_flipped_argmax_delays_stop():
    p = dict(P, entropy_bound=0.0)
    st = sampler.new_state(np.zeros((1, 4), dtype=np.int64))
    sampler.eb_step(_peaked(4, 8, [1, 2, 3, 4])[None], 0, p, st, 2, [0])
    sampler.eb_step(_peaked(4, 8, [1, 2, 3, 5])[None], 1, p, st, 2, [0])
    assert not st["done"][0] and st["stable_count"][0] == 0
    sampler.eb_step(_peaked(4, 8, [1, 2, 3, 5])[None], 2, p, st, 2, [0])
    assert st["done"][0] and list(st["canvas"][0]) == [1, 2, 3, 5]


def test_mean_entropy_just_above_threshold_does_not_stop():
    # each row: two-point-like rows whose entropy is ~0.0051 nats; mean above 0.005
    v = 8
    z = np.full((4, v), -1e4)
    z[:, 0] = 0.0
    # choose a gap d with binary entropy 0.0051 at T = 0.8 (solve numerically)
    from scipy.optimize import brentq
    inv = float(sampler.inv_temperature_f32(1, 48))
    d = brentq(lambda g: sp_entropy([1 / (1 + np.exp(-g * inv)), 1 - 1 / (1 + np.exp(-g * inv))])
               - 0.0051, 1.0, 60.0)
    z[:, 1] = -d
    p = dict(P, entropy_bound=0.0)
    st = sampler.new_state(np.zeros((1, 4), dtype=np.int64))
    sampler.eb_step(z[None], 0, p, st, 2, [0])
    r = sampler.eb_step(z[None], 1, p, st, 2, [0])
    assert r["entropy"].mean() > 0.005 and not st["done"][0]


def test_stop_disabled_runs_to_last_step():
    p = dict(P, entropy_bound=0.0, stop_entropy=-1.0, max_steps=5)
    st = sampler.new_state(np.zeros((1, 4), dtype=np.int64))
    z = _peaked(4, 8, [1, 2, 3, 4])[None]
    for s in range(4):
        sampler.eb_step(z, s, p, st, 2, [0])
        assert not st["done"][0]
    sampler.eb_step(z, 4, p, st, 2, [0])
    assert st["done"][0]


def test_committed_positions_keep_tokens_and_frozen_canvas_never_changes():
    rng = np.random.default_rng(5)
    v, c = 64, 12
    st = sampler.new_state(sampler.init_canvas(2, [0, 1], c, v))
    p = dict(P, max_steps=8)
    for s in range(8):
        z = round_bf16(rng.standard_normal((2, c, v)) * (1 + 4 * s))
        before = copy.deepcopy(st)
        r = sampler.eb_step(z, s, p, st, 2, [0, 1])
        for b in range(2):
            if before["done"][b]:
                assert np.array_equal(st["canvas"][b], before["canvas"][b])
                continue
            keep = before["committed"][b]
            assert np.array_equal(st["canvas"][b][keep], before["canvas"][b][keep])
            assert not (r["commit_now"][b] & keep).any()
            if not r["finalised"][b]:
                assert r["entropy"][b][r["commit_now"][b]].sum() <= p["entropy_bound"]
    assert st["done"].all() and st["committed"].all()


def test_determinism_and_resume():
    rng = np.random.default_rng(6)
    v, c, steps = 32, 8, 8
    zs = [round_bf16(rng.standard_normal((1, c, v)) * (1 + s)) for s in range(steps)]
    p = dict(P, max_steps=steps)

    def run(seed, start_state=None, start=0):
        st = start_state or sampler.new_state(sampler.init_canvas(seed, [0], c, v))
        for s in range(start, steps):
            sampler.eb_step(zs[s], s, p, st, seed, [0])
        return st

    a, b = run(2), run(2)
    assert np.array_equal(a["canvas"], b["canvas"])
    st = sampler.new_state(sampler.init_canvas(2, [0], c, v))
    for s in range(4):
        sampler.eb_step(zs[s], s, p, st, 2, [0])
    resumed = run(2, copy.deepcopy(st), 4)
    assert all(np.array_equal(a[k], resumed[k]) for k in a)
    other = sampler.new_state(sampler.init_canvas(3, [0], c, v))
    assert not np.array_equal(other["canvas"], sampler.init_canvas(2, [0], c, v))


def test_init_canvas_is_uniform_tag():
    c0 = sampler.init_canvas(2, [0, 1], 256, 262144)
    assert c0.shape == (2, 256) and c0.min() >= 0 and c0.max() < 262144
    assert np.array_equal(c0[0], sampler.uniform_tokens(2, 0, 0xFFFFFFFF, np.arange(256), 262144))
