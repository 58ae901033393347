"""Pins of the LM-head + unmask oracle: logits against explicit loops,
closed forms with one-hot projection rows, rows that must never be read, and
the argmax-gap diagnostic against a direct sort."""
import math

import numpy as np
import pytest

import oracle


def test_logits_against_explicit_loops():
    rng = np.random.default_rng(50)
    B, L, d, V = 2, 3, 7, 5
    h = rng.standard_normal((B, L, d))
    w = rng.standard_normal((V, d))
    mask = np.array([[1, 0, 1], [1, 1, 0]], np.uint8)
    got = oracle.lmhead_logits(h, w, mask)
    for b in range(B):
        for l in range(L):
            for v in range(V):
                if mask[b, l]:
                    ref = math.fsum(h[b, l, i] * w[v, i] for i in range(d))
                    assert abs(got[b, l, v] - ref) <= 1e-13
                else:
                    assert math.isnan(got[b, l, v])


def test_one_hot_projection_closed_form():
    """W[v] = c * e_{v mod d}: logits[b, l, v] = c * hidden[b, l, v mod d], so
    the argmax is the lowest v with the largest hidden coordinate and the
    confidence has a closed form."""
    d, V, c = 4, 10, 2.0
    w = np.zeros((V, d))
    for v in range(V):
        w[v, v % d] = c
    h = np.array([[[0.5, 3.0, -1.0, 0.0]]])          # coordinate 1 is largest
    mask = np.ones((1, 1), np.uint8)
    r = oracle.lmhead_unmask_step(h, w, mask, oracle.TOP_K, k=1)
    # ids with coordinate 1: 1, 5, 9 -> lowest id 1; three ids tie at the max.
    assert r["pred"][0, 0] == 1
    x = np.array([c * h[0, 0, v % d] for v in range(V)])
    conf = 1.0 / np.exp(x - x.max()).sum()
    assert abs(r["conf"][0, 0] - conf) <= 1e-15
    assert abs(conf - 1.0 / (3 + 3 * math.exp(-5.0) + 2 * math.exp(-6.0) + 2 * math.exp(-8.0))) < 1e-15
    assert r["top2_gap"][0, 0] == 0.0
    assert r["commit"][0, 0]


def test_unmasked_hidden_rows_never_read():
    rng = np.random.default_rng(51)
    B, L, d, V = 2, 6, 8, 30
    h = rng.standard_normal((B, L, d))
    w = rng.standard_normal((V, d))
    mask = (rng.random((B, L)) < 0.5).astype(np.uint8)
    mask[0, 0] = 1
    a = oracle.lmhead_unmask_step(h, w, mask, oracle.THRESHOLD, gamma=0.5, steps_left=2)
    h2 = h.copy()
    h2[mask == 0] = np.nan
    b = oracle.lmhead_unmask_step(h2, w, mask, oracle.THRESHOLD, gamma=0.5, steps_left=2)
    assert a["order"] == b["order"] and np.array_equal(a["mask_out"], b["mask_out"])
    np.testing.assert_array_equal(a["conf"], b["conf"])
    with pytest.raises(ValueError):
        oracle.lmhead_unmask_step(h2, w, np.ones((B, L), np.uint8), oracle.TOP_K, k=1)


def test_equals_selection_on_materialised_logits_and_gap():
    rng = np.random.default_rng(52)
    B, L, d, V = 3, 5, 16, 40
    h = rng.standard_normal((B, L, d))
    w = rng.standard_normal((V, d)) * 0.5
    mask = np.ones((B, L), np.uint8)
    r = oracle.lmhead_unmask_step(h, w, mask, oracle.TOP_K, k=2)
    logits = np.einsum("bld,vd->blv", h, w)           # a second, library contraction
    ref = oracle.unmask_step(logits, mask, 2)
    assert r["order"] == ref["order"]
    np.testing.assert_allclose(r["conf"], ref["conf"], rtol=1e-12)
    srt = np.sort(logits, axis=2)
    np.testing.assert_allclose(r["top2_gap"], srt[..., -1] - srt[..., -2], atol=1e-12)
