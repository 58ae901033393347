"""Oracle for the fused vocabulary projection + unmask step (test
infrastructure only).

Definition followed: the denoiser's distribution p_theta at a masked
position (TwoTower paper §2.2 "Sampling", Algorithm 2, DenoiserTower) is the
softmax of the logits its LM head produces from the position's final hidden
state: logits[b, l, v] = sum_i hidden[b, l, i] * W[v, i] (W is the
[vocab, d_model] projection).  The unmask step then treats those logits as
``unmask_step_select`` does.  Only still-masked positions are projected; the
hidden rows of committed positions are never read.

Method: upcast the (bf16) hidden rows and weights to float64, one matrix
product per masked row set, then the selection oracle on the full logit rows.
Also returned: the gap between the largest and second-largest logit of each
masked row (how close its argmax is to a tie).
"""
from __future__ import annotations

import numpy as np

from .unmask import unmask_step_select


def lmhead_logits(hidden, weight, mask_state) -> np.ndarray:
    """[B, L, V] float64 logits at masked positions, NaN elsewhere."""
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    mask = np.asarray(mask_state) != 0
    B, L, d = h.shape
    V = w.shape[0]
    if w.shape != (V, d):
        raise ValueError("weight must be [vocab, d_model]")
    out = np.full((B, L, V), np.nan, dtype=np.float64)
    rows = h[mask]                                     # masked rows only
    if not np.isfinite(rows).all() or not np.isfinite(w).all():
        raise ValueError("non-finite hidden state or weight")
    out[mask] = rows @ w.T
    return out


def lmhead_unmask_step(hidden, weight, mask_state, mode: int, **params) -> dict:
    """unmask_step_select over the LM-head logits of the masked positions.
    Adds ``top2_gap`` [B, L]: largest minus second-largest logit at masked
    positions (+inf for a one-word vocabulary), NaN elsewhere."""
    logits = lmhead_logits(hidden, weight, mask_state)
    mask = np.asarray(mask_state) != 0
    filled = np.where(mask[..., None], logits, 0.0)   # unmasked rows are never read
    res = unmask_step_select(filled, mask_state, mode, **params)
    gap = np.full(mask.shape, np.nan)
    V = logits.shape[2]
    for b, l in zip(*np.nonzero(mask)):
        if V == 1:
            gap[b, l] = np.inf
        else:
            top = np.partition(logits[b, l], V - 2)[V - 2:]
            gap[b, l] = top[1] - top[0]
    res["top2_gap"] = gap
    res["logits"] = logits
    return res
