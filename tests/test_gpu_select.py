"""GPU parity of the unmask step's selection rules (tt_unmask_step_ex /
tt_unmask_commit_ex) against the oracle's unmask_step_select: exact argmax ids,
confidences within 1e-5, exact commit counts and sets.  Floating point decides
two things here: the ranking (exempt where the oracle's last-chosen /
first-left gap is below 1e-4) and, for the threshold rule, which confidences
exceed gamma (exempt where a masked confidence lies within 1e-4 of gamma).  An
exempt sequence must still commit a valid prefix of the ranking."""
import numpy as np
import pytest
import torch

import oracle
from denoiser_attention_amd import synth
from helpers import CONF_MAX_ABS, GAP_EXEMPT, check_commit_valid, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MASK_ID = -7
MODES = {"top_k": oracle.TOP_K, "threshold": oracle.THRESHOLD, "schedule": oracle.SCHEDULE,
         "leftmost": oracle.LEFTMOST}


def varied_logits(rng, B, L, V, spread=(-2.0, 10.0)):
    """N(0, 2) logits with one peak per row set to (row max + delta), delta
    uniform in `spread`: confidences from near 0 to near 1."""
    x = (rng.standard_normal((B, L, V)) * 2).astype(np.float32)
    ids = rng.integers(0, V, size=(B, L))
    delta = rng.uniform(*spread, size=(B, L)).astype(np.float32)
    for b in range(B):
        for ell in range(L):
            x[b, ell, ids[b, ell]] = x[b, ell].max() + delta[b, ell]
    return x


def gpu_step(x, mask, tokens0, mode, split=False, **params):
    import denoiser_attention_amd as tt
    B, L = mask.shape
    sel = tt.select_rule(mode, **params)
    xd = torch.from_numpy(x).to(DEV)
    m = torch.from_numpy(mask).to(DEV)
    tok = torch.from_numpy(tokens0.astype(np.int32)).to(DEV)
    conf = torch.full((B, L), 7.0, device=DEV)
    pred = torch.full((B, L), 12345, dtype=torch.int32, device=DEV)
    mo = torch.full((B, L), 9, dtype=torch.uint8, device=DEV)
    if split:
        ws = torch.empty(tt.unmask_workspace_bytes(B, L, x.shape[2]), dtype=torch.uint8, device=DEV)
        tt.unmask_reduce(xd, m, ws)
        tt.unmask_commit_ex(m, sel, tok, mo, x.shape[2], ws, conf_out=conf, pred_out=pred)
    else:
        tt.unmask_step_ex(xd, m, sel, tok, mask_out=mo, conf_out=conf, pred_out=pred)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), mask_out=mo.cpu().numpy(), conf=conf.cpu().numpy(),
                pred=pred.cpu().numpy())


def check_select(got, ref, mask, tokens0, mode, what, **params):
    """Returns the exempted sequences.  Every sequence's count is asserted
    exactly (threshold: the count the GPU's own fp32 confidences give, inside
    the range the oracle's confidences +- 1e-5 allow), its set must be a prefix
    of the GPU's own ranking, and it equals the oracle's set unless the
    boundary gap, or a confidence's distance to gamma, is below 1e-4."""
    B, L = mask.shape
    exempt = []
    worst = 0.0
    for b in range(B):
        mb = mask[b] != 0
        assert np.array_equal(got["pred"][b][mb], ref["pred"][b][mb]), f"{what}: pred b={b}"
        assert np.all(got["pred"][b][~mb] == -1) and np.all(got["conf"][b][~mb] == -1.0)
        if mb.any():
            dc = float(np.abs(got["conf"][b][mb] - ref["conf"][b][mb]).max())
            worst = max(worst, dc)
            assert dc <= CONF_MAX_ABS, f"{what}: conf b={b} err {dc}"
        assert np.all(np.isin(got["mask_out"][b], (0, 1))) and np.all(got["mask_out"][b][~mb] == 0)
        committed = mb & (got["mask_out"][b] == 0)
        assert np.array_equal(got["tokens"][b][committed], ref["pred"][b][committed])
        assert np.array_equal(got["tokens"][b][~committed], tokens0[b][~committed])
        tol = np.where(mb, CONF_MAX_ABS, 0.0)
        if check_commit_valid(f"{what} b={b}", mode, mb, committed, got["conf"][b],
                              ref["conf"][b], ref["commit"][b], tol, GAP_EXEMPT, **params):
            assert ref["margin"][b] < GAP_EXEMPT or ref["gap"][b] < GAP_EXEMPT, \
                f"{what}: commit set b={b} (gap {ref['gap'][b]}, margin {ref['margin'][b]})"
            exempt.append(b)
        else:
            assert int(committed.sum()) == int(ref["n_commit"][b]), f"{what}: count b={b}"
    say(f"{what}: conf max_abs={worst:.3e} exempt={exempt}")
    return exempt


def run(x, mask, mode, what, split=False, tokens0=None, **params):
    B, L = mask.shape
    tokens0 = np.full((B, L), MASK_ID, np.int32) if tokens0 is None else tokens0
    got = gpu_step(x, mask, tokens0, mode, split=split, **params)
    ref = oracle.unmask_step_select(x.astype(np.float64), mask, MODES[mode], **params)
    check_select(got, ref, mask, tokens0, mode, what, **params)
    return got, ref


@pytest.mark.parametrize("L,T", [(16, 4), (32, 4), (16, 16)])
def test_threshold_sampler_teacher_forced(L, T):
    """The paper's default sampler (gamma 0.8, block 16) over T steps with the
    T-r+1 deadline; every GPU step starts from the oracle's mask."""
    rng = np.random.default_rng(100 + L + T)
    B, V = 8, 32768
    mask = np.ones((B, L), np.uint8)
    tokens = np.full((B, L), MASK_ID, np.int32)
    for r in range(1, T + 1):
        x = varied_logits(rng, B, L, V)
        got, ref = run(x, mask, "threshold", f"L{L} T{T} step {r}", tokens0=tokens, gamma=0.8,
                       steps_left=T - r + 1)
        tokens = got["tokens"]
        mask = ref["mask_out"]
    assert mask.sum() == 0


@pytest.mark.parametrize("gamma", [0.0, 0.3, 0.9, 0.999, 1.0, 2.5])
@pytest.mark.parametrize("steps_left", [1, 2, 5])
def test_threshold_gamma_and_deadline(gamma, steps_left):
    rng = np.random.default_rng(int(gamma * 1000) + steps_left)
    B, L, V = 5, 24, 3000
    x = varied_logits(rng, B, L, V)
    mask = (rng.random((B, L)) < 0.75).astype(np.uint8)
    mask[0] = 0          # a sequence with nothing masked
    mask[1] = 1          # and one fully masked
    run(x, mask, "threshold", f"gamma={gamma} d={steps_left}", gamma=gamma, steps_left=steps_left)


def test_threshold_on_planted_workload():
    """Decode-shaped workload (V = 131072, half the positions planted with a
    confident peak): gamma 0.8 commits the planted ones, the deadline the rest."""
    cfg = synth.get_config("decode_b8_p2048_l32")
    mask = synth.initial_mask(cfg)
    tokens = np.full(mask.shape, MASK_ID, np.int32)
    for r in range(1, cfg.steps + 1):
        x = synth.logits(cfg, seed=0, step=r - 1)
        got, ref = run(x, mask, "threshold", f"decode planted step {r}", tokens0=tokens,
                       gamma=0.8, steps_left=cfg.steps - r + 1)
        tokens, mask = got["tokens"], ref["mask_out"]
        del x
    assert mask.sum() == 0


@pytest.mark.parametrize("L,T", [(32, 4), (10, 4), (7, 3), (1, 1)])
def test_schedule_sampler_teacher_forced(L, T):
    rng = np.random.default_rng(200 + L * T)
    B, V = 6, 5000
    mask = np.ones((B, L), np.uint8)
    counts = []
    for r in range(1, T + 1):
        x = varied_logits(rng, B, L, V)
        got, ref = run(x, mask, "schedule", f"schedule L{L} T{T} step {r}", step=r, n_steps=T)
        counts.append(int(ref["n_commit"][0]))
        mask = ref["mask_out"]
    assert mask.sum() == 0
    say(f"schedule L{L} T{T} counts {counts}")


def test_schedule_off_schedule_masks():
    rng = np.random.default_rng(201)
    B, L, V = 6, 40, 2000
    x = varied_logits(rng, B, L, V)
    mask = (rng.random((B, L)) < 0.5).astype(np.uint8)
    for r, T in ((1, 4), (2, 4), (3, 4), (4, 4), (1, 1), (3, 7)):
        run(x, mask, "schedule", f"off-schedule r{r} T{T}", step=r, n_steps=T)


@pytest.mark.parametrize("k", [0, 1, 3, 50])
def test_leftmost_random_masks(k):
    rng = np.random.default_rng(300 + k)
    B, L, V = 7, 33, 1000
    x = varied_logits(rng, B, L, V)
    mask = (rng.random((B, L)) < 0.6).astype(np.uint8)
    run(x, mask, "leftmost", f"leftmost k={k}", k=k)


def test_mock_ar_full_block():
    """k = 1 left to right: step s commits position s, every sequence."""
    rng = np.random.default_rng(301)
    B, L, V = 3, 12, 700
    mask = np.ones((B, L), np.uint8)
    tokens = np.full((B, L), MASK_ID, np.int32)
    for s in range(L):
        x = varied_logits(rng, B, L, V)
        got, ref = run(x, mask, "leftmost", f"mock-AR step {s}", tokens0=tokens, k=1)
        assert np.all(got["mask_out"][:, s] == 0) and np.all(got["mask_out"][:, s + 1:] == 1)
        tokens, mask = got["tokens"], got["mask_out"]
    assert mask.sum() == 0


def test_top_k_mode_matches_unmask_step_bitwise():
    import denoiser_attention_amd as tt
    rng = np.random.default_rng(400)
    B, L, V = 4, 40, 9000
    x = varied_logits(rng, B, L, V)
    mask = (rng.random((B, L)) < 0.8).astype(np.uint8)
    a = gpu_step(x, mask, np.zeros((B, L), np.int32), "top_k", k=6)
    xd, m = torch.from_numpy(x).to(DEV), torch.from_numpy(mask).to(DEV)
    tok = torch.zeros((B, L), dtype=torch.int32, device=DEV)
    conf = torch.empty((B, L), device=DEV)
    tt.unmask_step(xd, m, 6, tok, conf_out=conf)
    torch.cuda.synchronize()
    assert np.array_equal(a["tokens"], tok.cpu().numpy())
    assert np.array_equal(a["conf"].view(np.uint32), conf.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("mode,params", [("threshold", dict(gamma=0.6, steps_left=3)),
                                         ("schedule", dict(step=2, n_steps=5)),
                                         ("leftmost", dict(k=4))])
def test_split_halves_equal_step(mode, params):
    rng = np.random.default_rng(500)
    B, L, V = 3, 20, 17000
    x = varied_logits(rng, B, L, V)
    mask = (rng.random((B, L)) < 0.7).astype(np.uint8)
    t0 = np.zeros((B, L), np.int32)
    a = gpu_step(x, mask, t0, mode, **params)
    b = gpu_step(x, mask, t0, mode, split=True, **params)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("mode,params", [("threshold", dict(gamma=0.5, steps_left=7)),
                                         ("leftmost", dict(k=300))])
def test_max_block_len(mode, params):
    rng = np.random.default_rng(600)
    B, L, V = 2, 1024, 64
    x = varied_logits(rng, B, L, V, spread=(-1.0, 6.0))
    mask = (rng.random((B, L)) < 0.9).astype(np.uint8)
    run(x, mask, mode, f"L=1024 {mode}", **params)
