"""Pins of the oracle's selection rules (threshold with deadline, predict-and-
noise schedule, mock-autoregressive) against definitions written differently
from the oracle's counting form: subset enumeration, hand-derived closed forms,
multi-step invariants and reduction to the already pinned fixed-k rule."""
import itertools
import math

import numpy as np
import pytest

import oracle


def _spike_logits(confs, V=10):
    """Rows whose maximum softmax probability is exactly confs[i] (up to
    rounding): one logit delta above V-1 zeros, delta = ln(c (V-1) / (1-c))."""
    x = np.zeros((len(confs), V))
    for i, c in enumerate(confs):
        x[i, 3] = math.log(c * (V - 1) / (1.0 - c))
    return x


def _brute_threshold(conf, cand, gamma, d):
    """Smallest candidate set that holds every conf > gamma, has at least
    ceil(n/d) members, and precedes every left-out candidate in the order
    (conf descending, position ascending)."""
    n = len(cand)
    best = None
    for size in range(n + 1):
        for sub in itertools.combinations(cand, size):
            s = set(sub)
            if any(conf[p] > gamma and p not in s for p in cand):
                continue
            if size * d < n:
                continue
            ok = all(conf[i] > conf[j] or (conf[i] == conf[j] and i < j)
                     for i in s for j in cand if j not in s)
            if ok:
                assert best is None or len(best) == size
                if best is None:
                    best = s
        if best is not None:
            return best
    raise AssertionError("no valid set")


def test_threshold_against_subset_enumeration():
    rng = np.random.default_rng(31)
    for trial in range(300):
        L = int(rng.integers(1, 9))
        conf = np.round(rng.uniform(0, 1, L), 1)      # coarse values: many exact ties
        cand = sorted(rng.choice(L, int(rng.integers(0, L + 1)), replace=False).tolist())
        gamma = float(rng.choice([0.0, 0.35, 0.5, 0.8, 1.0, 2.0]))
        d = int(rng.integers(1, 6))
        chosen, gap, margin = oracle.select_step(conf, cand, L, oracle.THRESHOLD, gamma=gamma,
                                                 steps_left=d)
        assert set(chosen) == _brute_threshold(conf, cand, gamma, d), (conf, cand, gamma, d)
        assert len(chosen) == len(set(chosen))
        if cand:
            assert margin == min(abs(conf[p] - gamma) for p in cand)


def test_threshold_closed_form():
    # Confidences 0.95 0.9 0.81 0.79 0.5 0.3 0.85 0.2 at positions 0..7, gamma 0.8.
    confs = [0.95, 0.9, 0.81, 0.79, 0.5, 0.3, 0.85, 0.2]
    x = _spike_logits(confs)[None]
    mask = np.ones((1, 8), np.uint8)
    # d = 4: four are above 0.8, the deadline asks for ceil(8/4) = 2 -> 4, in rank order.
    r = oracle.unmask_step_select(x, mask, oracle.THRESHOLD, gamma=0.8, steps_left=4)
    assert r["order"][0] == [0, 1, 6, 2]
    assert r["n_commit"][0] == 4
    assert abs(r["margin"][0] - 0.01) < 1e-9
    # gamma 0.92: one above, deadline 2 -> the two most confident.
    r = oracle.unmask_step_select(x, mask, oracle.THRESHOLD, gamma=0.92, steps_left=4)
    assert r["order"][0] == [0, 1]
    # gamma 0.92 with 3 steps left: ceil(8/3) = 3.
    r = oracle.unmask_step_select(x, mask, oracle.THRESHOLD, gamma=0.92, steps_left=3)
    assert r["order"][0] == [0, 1, 6]
    # Last step (d = 1): everything still masked is committed.
    r = oracle.unmask_step_select(x, mask, oracle.THRESHOLD, gamma=0.99, steps_left=1)
    assert sorted(r["order"][0]) == list(range(8))
    # gamma 0: every confidence is positive, so everything is committed.
    r = oracle.unmask_step_select(x, mask, oracle.THRESHOLD, gamma=0.0, steps_left=8)
    assert sorted(r["order"][0]) == list(range(8))
    np.testing.assert_allclose(r["conf"][0], confs, rtol=1e-12)


def test_threshold_gamma_one_is_fixed_k_deadline():
    """conf <= 1, so with gamma >= 1 nothing is above it and the rule is the
    pinned fixed-k rule with k = ceil(n / d) per sequence."""
    rng = np.random.default_rng(32)
    B, L, V = 4, 12, 50
    x = rng.standard_normal((B, L, V)) * 2
    mask = (rng.uniform(size=(B, L)) < 0.7).astype(np.uint8)
    for d in (1, 2, 3, 5):
        r = oracle.unmask_step_select(x, mask, oracle.THRESHOLD, gamma=1.0, steps_left=d)
        for b in range(B):
            n = int(mask[b].sum())
            ref = oracle.unmask_step(x[b:b + 1], mask[b:b + 1], -(-n // d))
            assert r["order"][b] == ref["order"][0]
            assert np.array_equal(r["mask_out"][b], ref["mask_out"][0])


def test_threshold_finishes_within_deadline():
    """With d = T - r + 1 at step r, n_masked after step r is at most
    n_0 (T - r) / T, and the block is empty after T steps."""
    rng = np.random.default_rng(33)
    for T in (1, 2, 3, 4, 7):
        for gamma in (0.3, 0.8, 1.5):
            B, L, V = 3, 16, 40
            mask = np.ones((B, L), np.uint8)
            n0 = mask.sum(1)
            for r in range(1, T + 1):
                x = rng.standard_normal((B, L, V)) * 3
                out = oracle.unmask_step_select(x, mask, oracle.THRESHOLD, gamma=gamma,
                                                steps_left=T - r + 1)
                above = ((out["conf"] > gamma) & (mask != 0)).sum(1)
                assert np.all(out["n_commit"] >= above)
                mask = out["mask_out"]
                assert np.all(mask.sum(1) * T <= n0 * (T - r))
            assert mask.sum() == 0


def test_schedule_counts_closed_form():
    # L = 10, T = 4, fully masked: floor(10 * (4 - r) / 4) = 7, 5, 2, 0 stay masked,
    # so 3, 2, 3, 2 are committed.
    rng = np.random.default_rng(34)
    L, T = 10, 4
    mask = np.ones((1, L), np.uint8)
    got = []
    for r in range(1, T + 1):
        x = rng.standard_normal((1, L, 30))
        out = oracle.unmask_step_select(x, mask, oracle.SCHEDULE, step=r, n_steps=T)
        got.append(int(out["n_commit"][0]))
        mask = out["mask_out"]
    assert got == [3, 2, 3, 2]
    assert mask.sum() == 0
    # Off schedule: 3 masked at step 1 of 4 with L = 16 -> 12 may stay masked -> 0 committed.
    m = np.zeros((1, 16), np.uint8)
    m[0, [2, 5, 9]] = 1
    out = oracle.unmask_step_select(rng.standard_normal((1, 16, 30)), m, oracle.SCHEDULE,
                                    step=1, n_steps=4)
    assert out["n_commit"][0] == 0 and np.array_equal(out["mask_out"], m)


def test_schedule_remasks_least_confident():
    """The positions left masked are the `keep` lowest in the ascending order
    (conf ascending, position descending)."""
    rng = np.random.default_rng(35)
    for _ in range(100):
        L = int(rng.integers(1, 20))
        T = int(rng.integers(1, 6))
        r = int(rng.integers(1, T + 1))
        conf = np.round(rng.uniform(0, 1, L), 1)
        cand = sorted(rng.choice(L, int(rng.integers(0, L + 1)), replace=False).tolist())
        chosen, _, _ = oracle.select_step(conf, cand, L, oracle.SCHEDULE, step=r, n_steps=T)
        keep = (L * (T - r)) // T
        asc = sorted(cand, key=lambda p: (conf[p], -p))
        remasked = set(asc[:min(keep, len(cand))])
        assert set(chosen) == set(cand) - remasked


def test_schedule_on_schedule_equals_fixed_k():
    """From a fully masked block with T dividing L, every step commits L / T:
    the fixed-k rule with k = L / T."""
    rng = np.random.default_rng(36)
    B, L, T, V = 3, 16, 4, 25
    m1 = np.ones((B, L), np.uint8)
    m2 = m1.copy()
    for r in range(1, T + 1):
        x = rng.standard_normal((B, L, V))
        a = oracle.unmask_step_select(x, m1, oracle.SCHEDULE, step=r, n_steps=T)
        b = oracle.unmask_step(x, m2, L // T)
        assert a["order"] == b["order"]
        m1, m2 = a["mask_out"], b["mask_out"]


def test_leftmost_closed_form():
    # The leftmost masked position is the least confident one: it is still first.
    confs = [0.99, 0.2, 0.9, 0.95, 0.1, 0.5, 0.6]
    x = _spike_logits(confs)[None]
    mask = np.array([[0, 1, 1, 0, 1, 1, 1]], np.uint8)
    for k, want in ((1, [1]), (2, [1, 2]), (4, [1, 2, 4, 5]), (10, [1, 2, 4, 5, 6]), (0, [])):
        r = oracle.unmask_step_select(x, mask, oracle.LEFTMOST, k=k)
        assert r["order"][0] == want
        assert math.isinf(r["gap"][0])


def test_mock_ar_commits_left_to_right():
    rng = np.random.default_rng(37)
    L = 9
    mask = np.ones((2, L), np.uint8)
    for step in range(L):
        out = oracle.unmask_step_select(rng.standard_normal((2, L, 20)), mask, oracle.LEFTMOST, k=1)
        assert out["order"] == [[step], [step]]
        mask = out["mask_out"]
    assert mask.sum() == 0


def test_top_k_mode_is_unmask_step():
    rng = np.random.default_rng(38)
    x = rng.standard_normal((3, 10, 30))
    mask = (rng.uniform(size=(3, 10)) < 0.6).astype(np.uint8)
    for k in (0, 1, 3, 20):
        a = oracle.unmask_step_select(x, mask, oracle.TOP_K, k=k)
        b = oracle.unmask_step(x, mask, k)
        assert a["order"] == b["order"] and np.array_equal(a["mask_out"], b["mask_out"])
        np.testing.assert_array_equal(a["gap"], b["gap"])


@pytest.mark.parametrize("mode,params", [
    (oracle.THRESHOLD, dict(gamma=0.5, steps_left=0)),
    (oracle.THRESHOLD, dict(gamma=float("nan"), steps_left=2)),
    (oracle.SCHEDULE, dict(step=0, n_steps=4)),
    (oracle.SCHEDULE, dict(step=5, n_steps=4)),
    (oracle.LEFTMOST, dict(k=-1)),
    (7, dict(k=1)),
])
def test_invalid_selection_rejected(mode, params):
    with pytest.raises(ValueError):
        oracle.select_step(np.ones(3) * 0.5, [0, 1, 2], 3, mode, **params)
