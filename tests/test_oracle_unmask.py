"""Pins of the unmask oracle against things other than itself: library argmax
and logsumexp, closed forms, brute-force subset enumeration, an independent
selection-based top-k, and the commit invariants the sampler must satisfy."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from denoiser_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def test_vocab_stats_match_library():
    rng = np.random.default_rng(20)
    for V in (1, 2, 7, 1000, 4099):
        x = rng.standard_normal(V) * 3
        a, conf, lse = oracle.vocab_stats(x)
        assert a == int(np.argmax(x))
        assert abs(lse - scipy.special.logsumexp(x)) <= 1e-12 * max(1.0, abs(lse))
        assert abs(conf - scipy.special.softmax(x).max()) <= 1e-15
        assert abs(conf - math.exp(x.max() - lse)) <= 1e-14


def test_argmax_ties_lowest_id():
    x = np.zeros(50)
    x[[30, 12, 44]] = 5.0
    a, conf, _ = oracle.vocab_stats(x)
    assert a == 12 == int(np.argmax(x))
    assert abs(conf - 1.0 / (3 + 47 * math.exp(-5.0))) <= 1e-15


def test_golden_rows():
    with open(GOLDEN) as fh:
        rows = json.load(fh)["unmask_rows"]
    for r in rows:
        V = r["V"]
        if r["kind"] == "constant":
            x = np.full(V, r["value"])
        elif r["kind"] == "spike":
            x = np.full(V, r["base"])
            x[r["pos"]] += r["delta"]
        else:
            x = np.full(V, r["base"])
            x[r["pos"]] += r["delta"]
        a, conf, _ = oracle.vocab_stats(x)
        assert a == r["argmax"]
        assert abs(conf - r["conf"]) <= 1e-15


def brute_topk(conf, candidates, k):
    """Enumerate every size-min(k,n) subset; keep the one whose descending
    conf vector is largest, ties to the lexicographically smallest positions."""
    n = min(k, len(candidates))
    best = None
    for sub in itertools.combinations(sorted(candidates), n):
        key = (tuple(sorted((conf[p] for p in sub), reverse=True)), tuple(-p for p in sub))
        if best is None or key > best[0]:
            best = (key, sub)
    return sorted(best[1])


def select_topk(conf, candidates, k):
    """Second implementation: repeated arg-max with lowest-position ties."""
    left = sorted(candidates)
    chosen = []
    for _ in range(min(k, len(left))):
        best = left[0]
        for p in left[1:]:
            if conf[p] > conf[best]:
                best = p
        chosen.append(best)
        left.remove(best)
    return chosen


def test_topk_against_brute_force_and_selection():
    rng = np.random.default_rng(21)
    for trial in range(300):
        L = int(rng.integers(1, 9))
        conf = rng.choice([0.1, 0.2, 0.5, 0.9], size=L) if trial % 2 else rng.random(L)
        cand = [p for p in range(L) if rng.random() < 0.7]
        for k in range(0, L + 2):
            chosen, gap = oracle.topk_select(conf, cand, k)
            if cand:
                assert sorted(chosen) == brute_topk(conf, cand, k)
            assert chosen == select_topk(conf, cand, k)
            if 0 < k < len(cand):
                ranked = sorted(cand, key=lambda p: (-conf[p], p))
                assert gap == conf[ranked[k - 1]] - conf[ranked[k]]
            else:
                assert gap == math.inf


def _rows(rng, B, L, V):
    return rng.standard_normal((B, L, V)) * 2.0


def test_commit_invariants():
    rng = np.random.default_rng(22)
    B, L, V = 3, 12, 37
    x = _rows(rng, B, L, V)
    mask = (rng.random((B, L)) < 0.6).astype(np.uint8)
    for k in (0, 1, 3, 12, 20):
        r = oracle.unmask_step(x, mask, k)
        for b in range(B):
            n_masked = int(mask[b].sum())
            c = r["commit"][b]
            assert c.sum() == min(k, n_masked)
            assert not np.any(c & (mask[b] == 0))               # committed subset of masked
            if c.any() and (mask[b].astype(bool) & ~c).any():
                assert r["conf"][b][c].min() >= r["conf"][b][mask[b].astype(bool) & ~c].max()
            assert np.array_equal(r["mask_out"][b], (mask[b].astype(bool) & ~c).astype(np.uint8))
            assert np.all(r["pred"][b][mask[b] == 0] == -1)
            for ell in np.nonzero(mask[b])[0]:
                assert r["pred"][b, ell] == int(np.argmax(x[b, ell]))


def test_unmasked_logits_never_read():
    rng = np.random.default_rng(23)
    x = _rows(rng, 2, 6, 11)
    mask = np.array([[1, 0, 1, 0, 1, 1], [0, 0, 0, 1, 0, 0]], dtype=np.uint8)
    r1 = oracle.unmask_step(x, mask, 2)
    y = x.copy()
    y[mask == 0] = 1e3       # logits at committed positions must not matter
    r2 = oracle.unmask_step(y, mask, 2)
    assert np.array_equal(r1["commit"], r2["commit"])
    assert np.array_equal(r1["pred"], r2["pred"])


def test_k_equals_S_over_T_empties_block_in_T_steps():
    """Fixed k = S/T finishes the block within T steps (the sampler's deadline)."""
    rng = np.random.default_rng(24)
    cfg = synth.get_config("tiny_fp32")
    mask = synth.initial_mask(cfg)
    for step in range(cfg.steps):
        x = synth.logits(cfg, seed=0, step=step)
        n_before = int(mask.sum())
        r = oracle.unmask_step(x, mask, cfg.k)
        assert int(r["commit"].sum()) == min(cfg.k, n_before)
        mask = r["mask_out"]
    assert int(mask.sum()) == 0


def test_mock_ar_k1_commits_one_per_step():
    rng = np.random.default_rng(25)
    mask = np.ones((2, 5), dtype=np.uint8)
    for step in range(5):
        r = oracle.unmask_step(_rows(rng, 2, 5, 9), mask, 1)
        assert np.all(r["commit"].sum(1) == 1)
        mask = r["mask_out"]
    assert mask.sum() == 0


def test_identical_rows_commit_lower_position_first():
    rng = np.random.default_rng(26)
    x = _rows(rng, 1, 6, 40)
    x[0, 4] = x[0, 1]
    x[0, 1, 3] += 9.0        # make the duplicated row the most confident
    x[0, 4] = x[0, 1]
    r = oracle.unmask_step(x, np.ones((1, 6), np.uint8), 1)
    assert r["order"][0] == [1]
    r = oracle.unmask_step(x, np.ones((1, 6), np.uint8), 2)
    assert r["order"][0] == [1, 4]


def test_k_negative_rejected():
    with pytest.raises(ValueError):
        oracle.unmask_step(np.zeros((1, 2, 3)), np.ones((1, 2), np.uint8), -1)
