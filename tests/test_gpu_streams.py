"""Calls on different streams at the same time: each call's result depends
only on its own arguments (the library keeps no state between calls apart
from the allocation-free entry point's documented scratch), so calls that
overlap on two streams, each with its own workspace, give the bits the same
calls give one after the other."""
import numpy as np
import pytest
import torch

import denoiser_attention_amd as tt
from denoiser_attention_amd import synth
from helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bf16(a):
    return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)


def test_overlapping_calls_on_two_streams():
    cfg = synth.get_config("decode_b8_p2048_l32").with_(batch=4, prefix_len=900, vocab=9000)
    B, Hq, Hkv, L, P, D, V = 4, 32, 2, 32, 900, 128, 9000
    li_cfg = cfg.with_(vocab=3000)
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    work = []
    for j, s in enumerate((s1, s2)):
        inp = synth.attn_inputs(cfg, seed=70 + j, prefix_cap=P)
        t = {n: _bf16(inp[n]) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}
        x = torch.from_numpy(synth.logits(cfg, seed=70 + j)).to(DEV)
        li = synth.lmhead_inputs(li_cfg, d_model=256, seed=70 + j)
        h, w = _bf16(li["hidden"]), _bf16(li["weight"])
        mask = torch.ones((B, L), dtype=torch.uint8, device=DEV)
        bufs = dict(out=torch.empty_like(t["q"]),
                    tok=torch.zeros((B, L), dtype=torch.int32, device=DEV),
                    mo=torch.empty_like(mask),
                    tok_lm=torch.zeros((B, L), dtype=torch.int32, device=DEV),
                    mo_lm=torch.empty_like(mask))
        ws_a = torch.empty(tt.attn_workspace_bytes(B, P, L, Hq, Hkv, D, torch.bfloat16),
                           dtype=torch.uint8, device=DEV)
        ws_u = torch.empty(tt.unmask_workspace_bytes(B, L, V), dtype=torch.uint8, device=DEV)
        ws_l = torch.empty(tt.lmhead_unmask_workspace_bytes(B, L, 3000, 256), dtype=torch.uint8,
                           device=DEV)
        with torch.cuda.stream(s):
            calls = [
                tt.prepare_block_attn(t["q"], t["k_ctx"], t["v_ctx"], P, t["k_blk"], t["v_blk"],
                                      inp["scale"], bufs["out"], workspace=ws_a, stream=s),
                tt.prepare_unmask_reduce(x, mask, ws_u, stream=s),
                tt.prepare_unmask_commit(mask, 8, bufs["tok"], bufs["mo"], V, ws_u, stream=s),
                tt.prepare_lmhead_unmask_step(h, w, mask, tt.select_rule("top_k", k=5),
                                              bufs["tok_lm"], bufs["mo_lm"], workspace=ws_l,
                                              stream=s),
            ]
        work.append((s, calls, bufs, (t, x, h, w, mask, ws_a, ws_u, ws_l)))
    torch.cuda.synchronize()

    def reset(bufs):
        bufs["out"].fill_(0)
        for key in ("tok", "tok_lm"):
            bufs[key].fill_(-1)
        for key in ("mo", "mo_lm"):
            bufs[key].fill_(9)

    # One after the other.
    ref = []
    for s, calls, bufs, _ in work:
        with torch.cuda.stream(s):
            reset(bufs)
            for c in calls:
                c()
        torch.cuda.synchronize()
        ref.append({k: v.clone() for k, v in bufs.items()})
    # Interleaved on two streams, several rounds.
    for r in range(3):
        say(f"two-stream round {r}")
        for s, _, bufs, _ in work:
            with torch.cuda.stream(s):
                reset(bufs)
        torch.cuda.synchronize()
        for i in range(4):
            for s, calls, _, _ in work:
                with torch.cuda.stream(s):
                    calls[i]()
        torch.cuda.synchronize()
        for (_, _, bufs, _), rb in zip(work, ref):
            for key, v in bufs.items():
                a, b = v, rb[key]
                if a.dtype == torch.bfloat16:
                    a, b = a.view(torch.int16), b.view(torch.int16)
                assert torch.equal(a, b), (r, key)
