"""GPU parity of the fused LM-head + unmask step (tt_lmhead_unmask_step)
against the oracle (float64 logits of the same bf16 hidden states and
weights).

The GPU forms each logit as an fp32 sum of d_model exact bf16 products, so a
logit can differ from the exact one by at most tau = d_model * 2^-24 *
sum_i |h_i w_i| (the standard bound for d_model roundings).  The bar, per
masked position: the argmax id is exact wherever the oracle's top-two logit
gap exceeds 2 tau (else the id must be one whose logit is within 2 tau of the
maximum); the confidence is within conf * (e^(2 tau) - 1) + 1e-5; commit sets
are exact per sequence except where the oracle's confidence gap at the
selection boundary (or a confidence's distance to gamma) is below the two
positions' confidence bounds plus 1e-4.  Every committed count is asserted
exactly: min(k, n) for top-k and leftmost, the schedule's count, and for the
threshold rule the count the GPU's own fp32 confidences give (which must lie
in the range the oracle's confidences, within their bounds, allow); the set
must be a prefix of the GPU's own ranking."""
import numpy as np
import pytest
import torch

import oracle
from denoiser_attention_amd import synth
from helpers import check_commit_valid, say, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MASK_ID = -7
MODES = {"top_k": oracle.TOP_K, "threshold": oracle.THRESHOLD, "schedule": oracle.SCHEDULE,
         "leftmost": oracle.LEFTMOST}


def cfg_v(V=None):
    c = synth.get_config("decode_b8_p2048_l32")
    return c if V is None else c.with_(vocab=V)


def tau_bound(h, w, mask):
    """Per masked position: d * 2^-24 * max_v sum_i |h_i w_vi| (float64)."""
    d = h.shape[2]
    tau = np.zeros(mask.shape)
    idx = np.nonzero(mask)
    if idx[0].size:
        rows = np.abs(h[idx])
        absw = np.abs(w)
        for s in range(0, rows.shape[0], 256):
            tau[idx[0][s:s + 256], idx[1][s:s + 256]] = \
                d * 2.0 ** -24 * (rows[s:s + 256] @ absw.T).max(axis=1)
    return tau


def gpu_lmhead(inp, mask, mode, tokens0=None, **params):
    import denoiser_attention_amd as tt
    B, L = mask.shape
    tokens0 = np.full((B, L), MASK_ID, np.int32) if tokens0 is None else tokens0
    hd, wd = to_dev(inp["hidden"], DEV), to_dev(inp["weight"], DEV)
    m = torch.from_numpy(mask).to(DEV)
    tok = torch.from_numpy(tokens0.astype(np.int32)).to(DEV)
    conf = torch.full((B, L), 7.0, device=DEV)
    pred = torch.full((B, L), 12345, dtype=torch.int32, device=DEV)
    mo = torch.full((B, L), 9, dtype=torch.uint8, device=DEV)
    tt.lmhead_unmask_step(hd, wd, m, tt.select_rule(mode, **params), tok, mask_out=mo,
                          conf_out=conf, pred_out=pred)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), mask_out=mo.cpu().numpy(), conf=conf.cpu().numpy(),
                pred=pred.cpu().numpy()), tokens0


def check(inp, mask, mode, what, seqs=None, tokens0=None, **params):
    B, L = mask.shape
    seqs = list(range(B)) if seqs is None else list(seqs)
    got, tokens0 = gpu_lmhead(inp, mask, mode, tokens0=tokens0, **params)
    h = oracle.decode_bf16(inp["hidden"][seqs])
    w = oracle.decode_bf16(inp["weight"])
    ms = mask[seqs]
    ref = oracle.lmhead_unmask_step(h, w, ms, MODES[mode], **params)
    tau = tau_bound(h, w, ms)
    worst_conf, worst_tau, worst_tol, exempt = 0.0, float(tau.max()) if tau.size else 0.0, 0.0, []
    for i, b in enumerate(seqs):
        mb = ms[i] != 0
        assert np.all(got["pred"][b][~mb] == -1) and np.all(got["conf"][b][~mb] == -1.0)
        assert np.all(got["mask_out"][b][~mb] == 0)
        conf_tol = np.zeros(L)
        for l in np.nonzero(mb)[0]:
            g, r = int(got["pred"][b, l]), int(ref["pred"][i, l])
            if ref["top2_gap"][i, l] > 2 * tau[i, l]:
                assert g == r, f"{what}: pred b={b} l={l} {g} != {r}"
            else:
                lg = ref["logits"][i, l]
                assert lg[g] >= lg.max() - 2 * tau[i, l], f"{what}: ambiguous pred b={b} l={l}"
            c = ref["conf"][i, l]
            conf_tol[l] = c * np.expm1(2 * tau[i, l]) + 1e-5
            err = abs(float(got["conf"][b, l]) - c)
            worst_conf = max(worst_conf, err)
            assert err <= conf_tol[l], f"{what}: conf b={b} l={l} err {err} tol {conf_tol[l]}"
        committed = mb & (got["mask_out"][b] == 0)
        assert np.array_equal(got["tokens"][b][committed], got["pred"][b][committed])
        assert np.array_equal(got["tokens"][b][~committed], tokens0[b][~committed])
        if check_commit_valid(f"{what} b={b}", mode, mb, committed, got["conf"][b],
                              ref["conf"][i], ref["commit"][i], conf_tol, 1e-4, **params):
            # exempt only at a near tie by the per-position tolerances: the
            # oracle's boundary pair, or (threshold) a confidence near gamma
            c = ref["conf"][i]
            pos = np.nonzero(mb)[0]
            ranked = sorted(pos.tolist(), key=lambda p: (-c[p], p))
            n_ref = int(ref["n_commit"][i])
            near = False
            if 0 < n_ref < len(ranked):
                a, bb = ranked[n_ref - 1], ranked[n_ref]
                near = c[a] - c[bb] < conf_tol[a] + conf_tol[bb] + 1e-4
            if mode == "threshold":
                near |= bool(np.any(np.abs(c[pos] - params["gamma"]) < conf_tol[pos] + 1e-4))
            assert near, f"{what}: commit set b={b} differs away from a near tie"
            exempt.append(b)
        else:
            assert int(committed.sum()) == int(ref["n_commit"][i]), f"{what}: count b={b}"
        worst_tol = max(worst_tol, float(conf_tol.max()))
    say(f"{what}: tau<={worst_tau:.2e} conf max_abs={worst_conf:.2e} "
        f"(bound up to {worst_tol:.2e}) exempt={exempt}")
    return got, ref


@pytest.mark.parametrize("V,d", [(1000, 96), (256, 64), (257, 32), (1, 64), (3000, 256)])
def test_small_vocab_and_width(V, d):
    inp = synth.lmhead_inputs(cfg_v(V), d_model=d, seed=V + d, batch=3, block_len=17)
    rng = np.random.default_rng(V)
    mask = (rng.random((3, 17)) < 0.7).astype(np.uint8)
    mask[0] = 0
    mask[1] = 1
    check(inp, mask, "top_k", f"V={V} d={d}", k=4)


def test_one_ragged_row_tile():
    """200 masked rows: one 256-row tile, ragged."""
    inp = synth.lmhead_inputs(cfg_v(5000), d_model=128, seed=61, batch=5, block_len=40)
    mask = np.ones((5, 40), np.uint8)
    check(inp, mask, "top_k", "200 rows", k=7)


def test_three_row_tiles_full_oracle():
    """About 614 masked rows scattered over 16 x 64 positions (density 0.6):
    three 256-row tiles, the last ragged, every position checked."""
    inp = synth.lmhead_inputs(cfg_v(5000), d_model=128, seed=68, batch=16, block_len=64)
    rng = np.random.default_rng(68)
    mask = (rng.random((16, 64)) < 0.6).astype(np.uint8)
    say(f"three row tiles: {int(mask.sum())} masked rows")
    assert int(mask.sum()) > 512
    check(inp, mask, "top_k", "614 rows", k=9)
    check(inp, mask, "threshold", "614 rows threshold", gamma=0.5, steps_left=3)


def test_highbatch_4096_rows_sampled():
    """The high-batch geometry: 64 x 64 positions all masked (16 row tiles of
    256), vocabulary 131072, d_model 2688; the oracle checks sequences in the
    first, a middle and the last row tile."""
    cfg = synth.get_config("highbatch_b64_p4096_l64")
    inp = synth.lmhead_inputs(cfg, seed=69)
    mask = synth.initial_mask(cfg)
    say("4096-row LM head: oracle on sequences 0, 31 and 63")
    check(inp, mask, "top_k", "4096 rows", seqs=[0, 31, 63], k=cfg.k)


def test_unmasked_rows_never_read():
    inp = synth.lmhead_inputs(cfg_v(2000), d_model=160, seed=62, batch=4, block_len=33)
    rng = np.random.default_rng(62)
    mask = (rng.random((4, 33)) < 0.4).astype(np.uint8)
    nan_bits = np.uint16(0x7FC0)
    inp["hidden"][mask == 0] = nan_bits
    check(inp, mask, "threshold", "NaN in unmasked rows", gamma=0.5, steps_left=3)


@pytest.mark.parametrize("mode,params", [("threshold", dict(gamma=0.8, steps_left=2)),
                                         ("schedule", dict(step=2, n_steps=4)),
                                         ("leftmost", dict(k=3))])
def test_selection_rules(mode, params):
    inp = synth.lmhead_inputs(cfg_v(4096), d_model=192, seed=63, batch=4, block_len=32)
    rng = np.random.default_rng(63)
    mask = (rng.random((4, 32)) < 0.8).astype(np.uint8)
    check(inp, mask, mode, f"{mode}", **params)


def test_threshold_multi_step_teacher_forced():
    """gamma 0.8 over 4 steps of a 32-position block; each GPU step starts from
    the oracle's mask."""
    cfg = cfg_v(8192)
    mask = np.ones((3, 32), np.uint8)
    tokens = np.full((3, 32), MASK_ID, np.int32)
    for r in range(1, 5):
        inp = synth.lmhead_inputs(cfg, d_model=256, seed=64, step=r, batch=3, block_len=32)
        got, ref = check(inp, mask, "threshold", f"step {r}", tokens0=tokens, gamma=0.8,
                         steps_left=5 - r)
        tokens, mask = got["tokens"], ref["mask_out"]
    assert mask.sum() == 0


def test_deterministic():
    import denoiser_attention_amd as tt
    inp = synth.lmhead_inputs(cfg_v(3000), d_model=128, seed=65, batch=2, block_len=32)
    mask = np.ones((2, 32), np.uint8)
    a, _ = gpu_lmhead(inp, mask, "top_k", k=5)
    b, _ = gpu_lmhead(inp, mask, "top_k", k=5)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_full_size_decode_sampled():
    """Decode-shaped step: 8 x 32 positions, vocabulary 131072, d_model 2688;
    the oracle checks two sequences."""
    cfg = cfg_v()
    inp = synth.lmhead_inputs(cfg, seed=66)
    mask = synth.initial_mask(cfg)
    say("full-size LM head: oracle on sequences 0 and 5")
    check(inp, mask, "top_k", "decode full size", seqs=[0, 5], k=cfg.k)


def test_full_vocab_odd_width_sampled():
    """Vocabulary 131072 with d_model 2720 (an odd multiple of 32, so the last
    column stage holds 32 columns) over 2 x 40 positions (a ragged row tile);
    the oracle checks one sequence."""
    cfg = cfg_v()
    inp = synth.lmhead_inputs(cfg, d_model=2720, seed=67, batch=2, block_len=40)
    rng = np.random.default_rng(67)
    mask = (rng.random((2, 40)) < 0.8).astype(np.uint8)
    say("full-vocabulary LM head at d_model 2720: oracle on sequence 1")
    check(inp, mask, "top_k", "V=131072 d=2720", seqs=[1], k=6)
