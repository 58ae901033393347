"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP
path through the binding, run the oracle on the same inputs, compare."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
from denoiser_attention_amd import synth

# Tolerances against the fp64 oracle.
BF16_MAX_ABS = 1e-2      # bf16 inputs, fp32 accumulation
BF16_MEAN_ABS = 1e-3
FP32_MAX_ABS = 1e-5      # fp32 inputs end to end
CONF_MAX_ABS = 1e-5      # confidence from fp32 logits (fp32 sum of <= 2^17 terms)
GAP_EXEMPT = 1e-4        # commit sets may differ where the k-th/(k+1)-th gap is below this


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, dev) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def as_f64(arr: np.ndarray) -> np.ndarray:
    return oracle.decode_bf16(arr) if arr.dtype == np.uint16 else arr.astype(np.float64)


def gpu_attn(inp: dict, dev, **kw) -> np.ndarray:
    from denoiser_attention_amd import block_attn
    t = {n: to_dev(inp[n], dev) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}
    kc, vc = (t["k_ctx"], t["v_ctx"]) if inp["prefix_cap"] > 0 else (None, None)
    out = block_attn(t["q"], kc, vc, inp["prefix_len"], t["k_blk"], t["v_blk"], inp["scale"], **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def oracle_attn(inp: dict, heads=None, batches=None) -> np.ndarray:
    """Oracle output; optionally only for some (batch, query head) pairs, by
    slicing the inputs to single-head problems."""
    q, kc, vc = as_f64(inp["q"]), as_f64(inp["k_ctx"]), as_f64(inp["v_ctx"])
    kb, vb = as_f64(inp["k_blk"]), as_f64(inp["v_blk"])
    if heads is None:
        out, _ = oracle.block_attn(q, kc, vc, inp["prefix_len"], kb, vb, inp["scale"])
        return out
    G = q.shape[1] // kb.shape[1]
    res = {}
    for b in batches:
        for h in heads:
            g = h // G
            o, _ = oracle.block_attn(q[b:b + 1, h:h + 1], kc[b:b + 1, g:g + 1], vc[b:b + 1, g:g + 1],
                                     inp["prefix_len"], kb[b:b + 1, g:g + 1], vb[b:b + 1, g:g + 1],
                                     inp["scale"])
            res[(b, h)] = o[0, 0]
    return res


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |x| (the rounding of an exact result to bf16)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    e = np.floor(np.log2(ax))
    return 2.0 ** (e - 8)


def check_attn(got: np.ndarray, ref: np.ndarray, in_dtype: str, out_bf16: bool, what: str):
    err = np.abs(got - ref)
    if in_dtype == "fp32":
        say(f"{what}: max_abs={err.max():.3e}")
        assert err.max() <= FP32_MAX_ABS, f"{what}: max abs {err.max()}"
        return
    # bf16 inputs: the arithmetic bar, plus half a bf16 ulp of the result when
    # the output itself is rounded to bf16.
    bound = BF16_MAX_ABS + (bf16_half_ulp(ref) if out_bf16 else 0.0)
    say(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} "
        f"worst_excess={(err - bound).max():.3e}")
    assert np.all(err <= bound), f"{what}: max abs {err.max()} over bound"
    assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean abs {err.mean()}"


def gpu_unmask(logits_dev, mask: np.ndarray, k: int, tokens0: np.ndarray, dev, alias=False):
    from denoiser_attention_amd import unmask_step
    B, L = mask.shape
    m = torch.from_numpy(mask).to(dev)
    tok = torch.from_numpy(tokens0.astype(np.int32)).to(dev)
    conf = torch.full((B, L), 7.0, device=dev)
    pred = torch.full((B, L), 12345, dtype=torch.int32, device=dev)
    mo = m if alias else torch.full((B, L), 9, dtype=torch.uint8, device=dev)
    unmask_step(logits_dev, m, k, tok, mask_out=mo, conf_out=conf, pred_out=pred)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), mask_out=mo.cpu().numpy(), conf=conf.cpu().numpy(),
                pred=pred.cpu().numpy())


def check_unmask(got: dict, ref: dict, mask: np.ndarray, k: int, tokens0: np.ndarray, what: str,
                 seqs=None) -> list:
    """Compare one GPU unmask step with the oracle.  Returns the sequences
    exempted by the near-tie rule (gap < GAP_EXEMPT)."""
    B, L = mask.shape
    seqs = range(B) if seqs is None else seqs
    exempt = []
    worst_conf = 0.0
    for b in seqs:
        mb = mask[b] != 0
        # predictions at every masked position: exact ids
        assert np.array_equal(got["pred"][b][mb], ref["pred"][b][mb]), f"{what}: pred b={b}"
        assert np.all(got["pred"][b][~mb] == -1), f"{what}: pred outside mask b={b}"
        assert np.all(got["conf"][b][~mb] == -1.0)
        if mb.any():
            dc = np.abs(got["conf"][b][mb] - ref["conf"][b][mb]).max()
            worst_conf = max(worst_conf, dc)
            assert dc <= CONF_MAX_ABS, f"{what}: conf b={b} err {dc}"
        committed = (mb & (got["mask_out"][b] == 0))
        assert np.all(np.isin(got["mask_out"][b], (0, 1))), f"{what}: mask_out values"
        assert np.all(got["mask_out"][b][~mb] == 0)
        n_exp = min(k, int(mb.sum()))
        assert int(committed.sum()) == n_exp, f"{what}: count b={b}"
        # committed ids are the predictions; others keep their token
        assert np.array_equal(got["tokens"][b][committed], ref["pred"][b][committed])
        assert np.array_equal(got["tokens"][b][~committed], tokens0[b][~committed])
        if not np.array_equal(committed, ref["commit"][b]):
            assert ref["gap"][b] < GAP_EXEMPT, f"{what}: commit set b={b} (gap {ref['gap'][b]})"
            exempt.append(b)
            # still a valid top-k: every committed conf >= every uncommitted one (within eps)
            c = ref["conf"][b]
            left = mb & ~committed
            if committed.any() and left.any():
                assert c[committed].min() >= c[left].max() - GAP_EXEMPT
    say(f"{what}: conf max_abs={worst_conf:.3e} exempt={exempt}")
    return exempt


def expected_commit_count(mode: str, n: int, L: int, gpu_conf_masked=None, **params) -> int:
    """Committed count of one step under a selection rule (TwoTower paper
    §2.2 "Sampling", Algorithm 2), from the rule's own arithmetic: exact for
    top-k, leftmost and the schedule; for the threshold rule it is taken from
    the GPU's own fp32 confidences (the kernel compares those with gamma)."""
    if mode in ("top_k", "leftmost"):
        return min(int(params["k"]), n)
    if mode == "schedule":
        T, r = int(params["n_steps"]), int(params["step"])
        return max(0, n - (L * (T - r)) // T)
    if mode == "threshold":
        d = int(params["steps_left"])
        above = int((np.asarray(gpu_conf_masked, np.float32) > np.float32(params["gamma"])).sum())
        return min(n, max(-(-n // d), above))
    raise ValueError(mode)


def check_commit_valid(what: str, mode: str, mb: np.ndarray, committed: np.ndarray,
                       gpu_conf: np.ndarray, ref_conf: np.ndarray, ref_commit: np.ndarray,
                       tol: np.ndarray, exempt_slack: float, **params) -> bool:
    """Validity of one sequence's commit set where floating point may decide it.

    mb          masked positions (bool [L])
    committed   positions the GPU committed (bool [L])
    gpu_conf    the GPU's own fp32 confidences (conf_out)
    ref_conf    the oracle's float64 confidences
    ref_commit  the oracle's commit set
    tol         per-position bound on |gpu_conf - ref_conf| (already asserted)
    exempt_slack  a swapped pair (a, b) is accepted only when the oracle ranks
                b above a by at most tol_a + tol_b + exempt_slack

    Asserts: the count (exact; for the threshold rule equal to the count the
    GPU's own confidences give, and inside the range the oracle's
    confidences +- tol allow); the set is the first `count` positions of the
    GPU's own ranking (conf desc, position asc; position asc for leftmost);
    and, against the oracle, equality unless the boundary is a near tie by the
    per-position tolerances (or, for the threshold rule, a confidence lies
    within tol + exempt_slack of gamma).  Returns True if exempted."""
    L = mb.shape[0]
    pos = np.nonzero(mb)[0]
    n = pos.size
    n_got = int(committed.sum())
    n_exp = expected_commit_count(mode, n, L, gpu_conf[pos], **params)
    assert n_got == n_exp, f"{what}: count {n_got} != {n_exp}"
    if mode == "threshold" and n:
        d = int(params["steps_left"])
        g = float(params["gamma"])
        floor_n = -(-n // d)
        lo = min(n, max(floor_n, int((ref_conf[pos] - tol[pos] > g).sum())))
        hi = min(n, max(floor_n, int((ref_conf[pos] + tol[pos] > g).sum())))
        assert lo <= n_got <= hi, f"{what}: threshold count {n_got} outside [{lo}, {hi}]"
    # The committed set is a prefix of the GPU's own ranking.
    if mode == "leftmost":
        own = list(pos[:n_exp])
    else:
        own = sorted(pos.tolist(), key=lambda p: (-float(gpu_conf[p]), p))[:n_exp]
    assert set(np.nonzero(committed)[0].tolist()) == set(int(p) for p in own), \
        f"{what}: commit set is not a prefix of the GPU's own ranking"
    if np.array_equal(committed, ref_commit):
        return False
    assert mode != "leftmost", f"{what}: leftmost set differs"
    # Exempt only a near tie: every pair the two sets order differently is
    # within the per-position tolerances of each other in the oracle.
    extra = np.nonzero(committed & ~ref_commit)[0]
    missing = np.nonzero(ref_commit & ~committed & mb)[0]
    for a in extra:
        for b in missing:
            assert ref_conf[b] - ref_conf[a] <= tol[a] + tol[b] + exempt_slack, \
                f"{what}: swapped pair ({a}, {b}) is not a near tie"
    return True
