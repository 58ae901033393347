"""GPU check of tt_unmask_step_noalloc, the allocation-free variant of
tt_unmask_step (its vocabulary partials live in the library's static device
array): on the same inputs both entry points, called through the C ABI, give
identical tokens, masks, confidences and predictions, bit for bit.  Two
calls in a row, the second with a smaller input, so that the second call runs
on the array the first left behind."""
import ctypes

import numpy as np
import pytest
import torch

import denoiser_attention_amd as tt
from denoiser_attention_amd import _binding as B
from denoiser_attention_amd import synth
from helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_entry(noalloc, x, mask, k, tokens0, fill):
    lib = tt.lib()
    Bn, L, V = x.shape
    xd = torch.from_numpy(x).to(DEV)
    m = torch.from_numpy(mask).to(DEV)
    tok = torch.from_numpy(tokens0).to(DEV)
    mo = torch.full((Bn, L), fill, dtype=torch.uint8, device=DEV)
    conf = torch.full((Bn, L), float(fill), device=DEV)
    pred = torch.full((Bn, L), fill, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    if noalloc:
        st = lib.tt_unmask_step_noalloc(xd.data_ptr(), m.data_ptr(), k, tok.data_ptr(),
                                        mo.data_ptr(), Bn, L, V, conf.data_ptr(),
                                        pred.data_ptr(), None)
    else:
        n = lib.tt_unmask_workspace_bytes(Bn, L, V)
        ws = torch.empty(n, dtype=torch.uint8, device=DEV)
        torch.cuda.synchronize()
        st = lib.tt_unmask_step(xd.data_ptr(), m.data_ptr(), k, tok.data_ptr(), mo.data_ptr(),
                                Bn, L, V, conf.data_ptr(), pred.data_ptr(), ws.data_ptr(), n,
                                None)
    assert st == B.TT_OK, B.status_string(st)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), mask_out=mo.cpu().numpy(),
                conf=conf.cpu().numpy().view(np.uint32), pred=pred.cpu().numpy())


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    cfg = synth.get_config("highbatch_b64_p4096_l64")
    cases = [
        # 1024 positions (16 KB vocabulary chunks: 32 per row, 512 KB of partials), ties
        dict(batch=16, block_len=64, vocab=131072, k=16, seed=11),
        # then a smaller call: 4 x 40 positions, 32 KB chunks, a ragged last chunk
        dict(batch=4, block_len=40, vocab=50001, k=5, seed=12),
    ]
    lib = tt.lib()
    for c in cases:
        rng = np.random.default_rng(c["seed"])
        x = synth.logits(cfg, seed=c["seed"], batch=c["batch"], block_len=c["block_len"],
                         vocab=c["vocab"])
        mask = (rng.random((c["batch"], c["block_len"])) < 0.8).astype(np.uint8)
        mask[0] = 1
        tokens0 = rng.integers(-5, 0, size=mask.shape).astype(np.int32)
        need = lib.tt_unmask_workspace_bytes(c["batch"], c["block_len"], c["vocab"])
        say(f"noalloc case {c}: partials {need} B of {B.NOALLOC_SCRATCH_BYTES}")
        assert 0 < need <= B.NOALLOC_SCRATCH_BYTES
        a = run_entry(False, x, mask, c["k"], tokens0, 7)
        b = run_entry(True, x, mask, c["k"], tokens0, 9)
        for key in a:
            assert np.array_equal(a[key], b[key]), f"{key} differs for {c}"
        n_commit = int(((mask != 0) & (b["mask_out"] == 0)).sum())
        assert n_commit == sum(min(c["k"], int(r.sum())) for r in mask)
        del x


def test_noalloc_binding_and_size_limit():
    cfg = synth.get_config("decode_b8_p2048_l32")
    x = torch.from_numpy(synth.logits(cfg, seed=3, batch=2)).to(DEV)
    m = torch.ones((2, cfg.block_len), dtype=torch.uint8, device=DEV)
    t1 = torch.zeros((2, cfg.block_len), dtype=torch.int32, device=DEV)
    t2 = torch.zeros_like(t1)
    tt.unmask_step(x, m, cfg.k, t1)
    tt.unmask_step_noalloc(x, m, cfg.k, t2)
    torch.cuda.synchronize()
    assert torch.equal(t1, t2)
    # 64 x 1024 positions of 131072 ids need 32 MiB of partials: refused
    # before anything is enqueued.
    st = tt.lib().tt_unmask_step_noalloc(x.data_ptr(), m.data_ptr(), 4, t1.data_ptr(),
                                         m.data_ptr(), 64, 1024, 131072, None, None, None)
    assert st == B.TT_EUNSUPPORTED
