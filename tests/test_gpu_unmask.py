"""GPU parity of tt_unmask_step against the fp64 oracle: exact argmax ids and
commit counts, exact commit sets except where the oracle's k-th/(k+1)-th
confidence gap is below 1e-4, confidence within 1e-5; multi-step runs
teacher-forced (each GPU step starts from the oracle's mask) and free-running."""
import numpy as np
import pytest
import torch

import oracle
from denoiser_attention_amd import synth
from helpers import check_unmask, gpu_unmask, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MASK_ID = -7


def run_steps(cfg, batch=None, seqs=None, seed=0, teacher=True):
    """Run cfg.steps unmask steps.  Teacher-forced: every GPU step starts from
    the oracle's mask of the previous step (so an exempted near-tie cannot
    cascade).  Free-running: the GPU's own mask feeds the next step, until the
    first exempted near-tie."""
    B = cfg.batch if batch is None else batch
    sel = list(range(B)) if seqs is None else list(seqs)
    mask = synth.initial_mask(cfg, batch=B)
    tokens = np.full((B, cfg.block_len), MASK_ID, dtype=np.int32)
    for step in range(cfg.steps):
        x = synth.logits(cfg, seed=seed, step=step, batch=B)
        ref_full = oracle.unmask_step(x[sel], mask[sel], cfg.k)
        ref = {key: _scatter(ref_full[key], sel, B, key) for key in ("pred", "conf", "commit")}
        ref["gap"] = np.full(B, np.inf)
        ref["gap"][sel] = ref_full["gap"]
        got = gpu_unmask(torch.from_numpy(x).to(DEV), mask, cfg.k, tokens, DEV)
        exempt = check_unmask(got, ref, mask, cfg.k, tokens, f"{cfg.name} step {step}", seqs=sel)
        tokens = got["tokens"]
        if teacher:
            mask = got["mask_out"].copy()
            mask[sel] = ref_full["mask_out"]
        else:
            if exempt:
                say(f"free-running stops at step {step}: near-tie in {exempt}")
                return
            mask = got["mask_out"]
    assert int(mask.sum()) == 0, "block must be empty after steps = L / k"


def _scatter(arr, sel, B, key):
    shape = (B,) + arr.shape[1:]
    fill = {"pred": -1, "conf": np.nan, "commit": False}[key]
    out = np.full(shape, fill, dtype=arr.dtype)
    out[sel] = arr
    return out


def test_tiny_teacher_forced():
    run_steps(synth.get_config("tiny_fp32"))


def test_tiny_free_running():
    run_steps(synth.get_config("tiny_fp32"), teacher=False)


def test_decode_full_batch_teacher_forced():
    run_steps(synth.get_config("decode_b8_p2048_l32"))


def test_decode_free_running_two_seqs():
    run_steps(synth.get_config("decode_b8_p2048_l32"), batch=2, teacher=False)


@pytest.mark.parametrize("name,seqs", [
    ("highbatch_b64_p4096_l64", [0, 41]),
    ("block256_b16_p1024", [9]),
    ("gen8k_b4_l256", [2]),
])
def test_full_size_sampled_sequences(name, seqs):
    cfg = synth.get_config(name)
    say(f"full-size unmask {name}, oracle on sequences {seqs}")
    # steps 0 and the last one: all masked, and only k left
    B, L = cfg.batch, cfg.block_len
    for step, n_left in ((0, L), (cfg.steps - 1, cfg.k)):
        x = synth.logits(cfg, seed=0, step=step)
        rng = np.random.default_rng(step)
        mask = np.zeros((B, L), np.uint8)
        for b in range(B):
            mask[b, rng.choice(L, n_left, replace=False)] = 1
        tokens = np.full((B, L), MASK_ID, np.int32)
        got = gpu_unmask(torch.from_numpy(x).to(DEV), mask, cfg.k, tokens, DEV)
        ref_full = oracle.unmask_step(x[seqs], mask[seqs], cfg.k)
        ref = {key: _scatter(ref_full[key], seqs, B, key) for key in ("pred", "conf", "commit")}
        ref["gap"] = np.full(B, np.inf)
        ref["gap"][seqs] = ref_full["gap"]
        check_unmask(got, ref, mask, cfg.k, tokens, f"{name} step {step}", seqs=seqs)
        # every sequence commits exactly min(k, n_masked)
        assert np.all(((mask != 0) & (got["mask_out"] == 0)).sum(1) == min(cfg.k, n_left))
        del x


def _single(x, mask, k, tokens=None, alias=False):
    B, L, V = x.shape
    tokens = np.full((B, L), MASK_ID, np.int32) if tokens is None else tokens
    got = gpu_unmask(torch.from_numpy(x.astype(np.float32)).to(DEV), mask, k, tokens, DEV,
                     alias=alias)
    ref = oracle.unmask_step(x, mask, k)
    check_unmask(got, ref, mask, k, tokens, f"V={V} k={k}")
    return got, ref


@pytest.mark.parametrize("V", [1, 3, 4, 1000, 8191, 8192, 8193, 20000, 131072])
def test_vocab_sizes_and_tails(V):
    rng = np.random.default_rng(V)
    x = (rng.standard_normal((2, 9, V)) * 3).astype(np.float32)
    mask = (rng.random((2, 9)) < 0.7).astype(np.uint8)
    _single(x, mask, 3)


@pytest.mark.parametrize("V", [(1 << 20) + 4100, (1 << 20) + 4099])
def test_large_vocab(V):
    """A vocabulary past 2^20 (129 chunks, a ragged last chunk; 16-byte rows
    and, with V odd, the scalar-load form), with the argmax planted in the last
    chunk for one row and duplicated across the first and last chunk for
    another (lowest id wins)."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((1, 4, V)) * 3).astype(np.float32)
    x[0, 1, V - 2] = 40.0
    x[0, 2, 17] = 40.0
    x[0, 2, V - 1] = 40.0
    mask = np.ones((1, 4), np.uint8)
    got, _ = _single(x, mask, 2)
    assert got["pred"][0, 1] == V - 2 and got["pred"][0, 2] == 17


def test_k_edge_cases():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((3, 12, 5000)) * 2).astype(np.float32)
    mask = np.ones((3, 12), np.uint8)
    mask[1, ::2] = 0
    mask[2] = 0                                   # empty sequence
    for k in (0, 1, 5, 12, 100):
        got, _ = _single(x, mask, k)
        if k == 0:
            assert np.array_equal(got["mask_out"], mask)
            assert np.all(got["tokens"] == MASK_ID)


def test_mask_out_aliases_mask_state():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((4, 32, 3000)) * 3).astype(np.float32)
    mask = (rng.random((4, 32)) < 0.8).astype(np.uint8)
    _single(x, mask, 4, alias=True)


def test_ties_across_chunks_and_duplicate_rows():
    V = 3 * 8192 + 100
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((1, 8, V)) * 2).astype(np.float32)
    for ell, ids in enumerate([(20000, 100), (8192, 8191), (24675, 0), (16384, 16385)]):
        x[0, ell, list(ids)] = 50.0               # equal maxima in different chunks
    x[0, 6] = x[0, 5]                             # identical rows: lower position first
    x[0, 5, 77] = x[0, 6, 77] = 60.0
    got, ref = _single(x, np.ones((1, 8), np.uint8), 1)
    assert list(np.nonzero(got["mask_out"][0] == 0)[0]) == [5]
    assert got["pred"][0, 0] == 100 and got["pred"][0, 1] == 8191
    assert got["pred"][0, 2] == 0 and got["pred"][0, 3] == 16384


def test_max_block_len():
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((1, 1024, 64)) * 2).astype(np.float32)
    _single(x, np.ones((1, 1024), np.uint8), 100)


def test_unmasked_rows_never_read():
    """Rows of committed positions hold NaN: the result must not change."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((2, 16, 4096)) * 2).astype(np.float32)
    mask = (rng.random((2, 16)) < 0.5).astype(np.uint8)
    got1, _ = _single(x, mask, 3)
    y = x.copy()
    y[mask == 0] = np.nan
    tokens = np.full((2, 16), MASK_ID, np.int32)
    got2 = gpu_unmask(torch.from_numpy(y).to(DEV), mask, 3, tokens, DEV)
    for key in ("tokens", "mask_out", "pred"):
        assert np.array_equal(got1[key], got2[key])


def test_deterministic():
    rng = np.random.default_rng(12)
    x = torch.from_numpy((rng.standard_normal((4, 64, 50000)) * 3).astype(np.float32)).to(DEV)
    mask = np.ones((4, 64), np.uint8)
    tokens = np.full((4, 64), MASK_ID, np.int32)
    a = gpu_unmask(x, mask, 16, tokens, DEV)
    b = gpu_unmask(x, mask, 16, tokens, DEV)
    for key in a:
        assert np.array_equal(a[key], b[key])


@pytest.mark.parametrize("shift", [1, 2, 3])
def test_logits_base_not_16_byte_aligned(shift):
    """Logits that start 4, 8 or 12 bytes past a 16-byte boundary (a
    contiguous view into a larger buffer), with V a multiple of 4: the rows are
    not 16-byte aligned, so the vocabulary pass takes its scalar-load form and
    still gives the oracle's ids, confidences and commits."""
    B, L, V, k = 2, 12, 8192 + 4, 3
    rng = np.random.default_rng(90 + shift)
    x = (rng.standard_normal((B, L, V)) * 3).astype(np.float32)
    mask = (rng.random((B, L)) < 0.75).astype(np.uint8)
    buf = torch.empty(B * L * V + shift, dtype=torch.float32, device=DEV)
    view = buf[shift:].view(B, L, V)
    assert view.data_ptr() % 16 == 4 * shift
    view.copy_(torch.from_numpy(x))
    tokens = np.full((B, L), MASK_ID, np.int32)
    got = gpu_unmask(view, mask, k, tokens, DEV)
    check_unmask(got, oracle.unmask_step(x, mask, k), mask, k, tokens, f"base+{4 * shift}B")
