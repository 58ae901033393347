"""Oracle for the confidence unmask step (test infrastructure only).

Definition followed: TwoTower paper §2.2 "Sampling" and Algorithm 2.  At each
step the denoiser predicts every still-masked position of the block in
parallel; the most confident predictions are committed and the rest stay
masked.  The paper commits the predictions above a threshold gamma while
guaranteeing that the block finishes within T steps (a deadline of T-r+1
remaining steps).  This oracle implements the fixed-k form: with the
threshold switched off the deadline alone commits ceil(n / (T-r+1))
positions, which is a fixed k = S/T when T divides S.

Readings where the pages are silent:
* Confidence of a position = the largest probability of the denoiser's
  distribution at temperature 1, i.e. 1 / sum_v exp(x_v - max_v x_v).
* The committed token is the argmax (greedy); ties go to the lowest id.
* Top-k order: confidence descending, then position ascending.
* Committed positions are never re-read: their logits are ignored and their
  token and mask are unchanged.
* k = 0 commits nothing; k >= n_masked commits every masked position.

Selection rules (``unmask_step_select``), all over the same per-position
statistics and all committing a prefix of one ranking:
* TOP_K      the fixed-k form above.
* THRESHOLD  ConfidenceSample of Algorithm 2 with threshold gamma and a
             deadline of d = T-r+1 remaining steps: every masked position
             with conf > gamma (strict), and at least ceil(n / d) of them,
             so that n masked positions are gone after d steps.  Because the
             positions above gamma rank ahead of all others, the union is the
             first max(#{conf > gamma}, ceil(n / d)) positions of the ranking.
* SCHEDULE   the predict-and-noise sampler of §2.2 with the linear schedule
             alpha_t = 1 - t: step r of T leaves floor(L * (T - r) / T)
             positions masked (the expected masked count L * (1 - alpha_s)
             at the next noise level s = (T - r) / T, floored), re-masking the
             least confident predictions; it commits max(0, n - that).
* LEFTMOST   the mock-autoregressive mode: the k masked positions with the
             lowest index (left to right), whatever their confidence.
"""
from __future__ import annotations

import math

import numpy as np


def vocab_stats(row) -> tuple[int, float, float]:
    """(argmax id, confidence, logsumexp) of one logit row, in float64.

    argmax: ids sorted by value descending with a stable sort, so that the
    first id is the lowest id among the maxima.
    confidence: 1 / fsum_v exp(x_v - max), the maximum softmax probability.
    """
    x = np.asarray(row, dtype=np.float64)
    if x.ndim != 1 or x.size == 0:
        raise ValueError("vocab row must be a non-empty vector")
    if not np.isfinite(x).all():
        raise ValueError("non-finite logit")
    order = np.argsort(-x, kind="stable")
    a = int(order[0])
    m = x[a]
    total = math.fsum(np.exp(x - m).tolist())
    return a, 1.0 / total, m + math.log(total)


def topk_select(conf, candidates, k: int) -> tuple[list[int], float]:
    """Pick min(k, n) candidate positions by (confidence desc, position asc).

    Returns (chosen positions in rank order, gap) where gap is
    conf of the k-th minus conf of the (k+1)-th candidate in that order
    (+inf when every candidate is chosen or k == 0)."""
    cand = [int(c) for c in candidates]
    # Sort key (-conf, position): a stable sort of positions already in
    # ascending order by descending confidence.
    cand.sort()
    ranked = sorted(cand, key=lambda p: -conf[p])
    n_take = min(max(k, 0), len(ranked))
    chosen = ranked[:n_take]
    if 0 < n_take < len(ranked):
        gap = float(conf[ranked[n_take - 1]] - conf[ranked[n_take]])
    else:
        gap = math.inf
    return chosen, gap


def unmask_step(logits, mask_state, k: int) -> dict:
    """One fixed-k confidence-unmasking step over a batch of blocks.

    logits [B, L, V] float, mask_state [B, L] (nonzero = still [MASK]).
    Returns a dict of numpy arrays:
      commit [B,L] bool   positions committed by this step
      pred   [B,L] int64  argmax at masked positions, -1 elsewhere
      conf   [B,L] f64    confidence at masked positions, NaN elsewhere
      lse    [B,L] f64    logsumexp at masked positions, NaN elsewhere
      mask_out [B,L] u8   mask after the step
      gap    [B]   f64    k-th minus (k+1)-th confidence (+inf if none)
      order  list of per-sequence committed positions in rank order
    """
    if k < 0:
        raise ValueError("k must be >= 0")
    x = np.asarray(logits)
    mask = np.asarray(mask_state) != 0
    B, L, V = x.shape
    if mask.shape != (B, L):
        raise ValueError("mask shape mismatch")
    pred = np.full((B, L), -1, dtype=np.int64)
    conf = np.full((B, L), np.nan, dtype=np.float64)
    lse = np.full((B, L), np.nan, dtype=np.float64)
    commit = np.zeros((B, L), dtype=bool)
    gap = np.full(B, np.inf, dtype=np.float64)
    order = []
    for b in range(B):
        masked = [ell for ell in range(L) if mask[b, ell]]
        for ell in masked:
            a, c, s = vocab_stats(x[b, ell])
            pred[b, ell], conf[b, ell], lse[b, ell] = a, c, s
        chosen, gap[b] = topk_select(conf[b], masked, k)
        commit[b, chosen] = True
        order.append(chosen)
    mask_out = (mask & ~commit).astype(np.uint8)
    return dict(commit=commit, pred=pred, conf=conf, lse=lse, mask_out=mask_out, gap=gap,
                order=order)


# Selection rules of one sampling step.
TOP_K, THRESHOLD, SCHEDULE, LEFTMOST = 0, 1, 2, 3


def commit_count(mode: int, conf, candidates, block_len: int, *, k: int = 0, gamma: float = 1.0,
                 steps_left: int = 1, step: int = 1, n_steps: int = 1) -> int:
    """Number of masked positions one step commits under `mode`."""
    n = len(candidates)
    if mode in (TOP_K, LEFTMOST):
        if k < 0:
            raise ValueError("k must be >= 0")
        return min(k, n)
    if mode == THRESHOLD:
        if steps_left < 1 or not math.isfinite(gamma):
            raise ValueError("threshold needs steps_left >= 1 and a finite gamma")
        above = sum(1 for p in candidates if conf[p] > gamma)
        deadline = -(-n // steps_left)          # ceil(n / d)
        return min(n, max(above, deadline))
    if mode == SCHEDULE:
        if not 1 <= step <= n_steps:
            raise ValueError("schedule needs 1 <= step <= n_steps")
        keep = (block_len * (n_steps - step)) // n_steps
        return max(0, n - keep)
    raise ValueError(f"unknown selection mode {mode}")


def select_step(conf, candidates, block_len: int, mode: int, **params):
    """Rank the candidates and take the first commit_count(...) of them.

    Ranking: (conf descending, position ascending), or position ascending for
    LEFTMOST.  Returns (chosen in rank order, gap, margin): gap = conf of the
    last chosen minus conf of the first unchosen candidate (+inf when all or
    none are chosen, and for LEFTMOST); margin = min |conf - gamma| over the
    candidates for THRESHOLD (+inf otherwise)."""
    cand = sorted(int(c) for c in candidates)
    ranked = cand if mode == LEFTMOST else sorted(cand, key=lambda p: -conf[p])
    n_take = commit_count(mode, conf, cand, block_len, **params)
    chosen = ranked[:n_take]
    gap = math.inf
    if mode != LEFTMOST and 0 < n_take < len(ranked):
        gap = float(conf[ranked[n_take - 1]] - conf[ranked[n_take]])
    margin = math.inf
    if mode == THRESHOLD and cand:
        margin = min(abs(float(conf[p]) - params["gamma"]) for p in cand)
    return chosen, gap, margin


def unmask_step_select(logits, mask_state, mode: int, **params) -> dict:
    """One unmasking step under any selection rule (see the module notes).

    Same outputs as unmask_step, plus margin [B] (THRESHOLD: distance of the
    nearest masked confidence to gamma) and n_commit [B]."""
    x = np.asarray(logits)
    mask = np.asarray(mask_state) != 0
    B, L, V = x.shape
    if mask.shape != (B, L):
        raise ValueError("mask shape mismatch")
    pred = np.full((B, L), -1, dtype=np.int64)
    conf = np.full((B, L), np.nan, dtype=np.float64)
    lse = np.full((B, L), np.nan, dtype=np.float64)
    commit = np.zeros((B, L), dtype=bool)
    gap = np.full(B, np.inf, dtype=np.float64)
    margin = np.full(B, np.inf, dtype=np.float64)
    n_commit = np.zeros(B, dtype=np.int64)
    order = []
    for b in range(B):
        masked = [ell for ell in range(L) if mask[b, ell]]
        for ell in masked:
            a, c, s = vocab_stats(x[b, ell])
            pred[b, ell], conf[b, ell], lse[b, ell] = a, c, s
        chosen, gap[b], margin[b] = select_step(conf[b], masked, L, mode, **params)
        commit[b, chosen] = True
        n_commit[b] = len(chosen)
        order.append(chosen)
    mask_out = (mask & ~commit).astype(np.uint8)
    return dict(commit=commit, pred=pred, conf=conf, lse=lse, mask_out=mask_out, gap=gap,
                margin=margin, n_commit=n_commit, order=order)
