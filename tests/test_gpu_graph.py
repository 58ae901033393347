"""HIP-graph capture of the library's calls: a captured step replays bit for
bit like the eager calls, replay after replay, with other eager work on the
same workspaces (and on the allocation-free entry point's shared scratch)
and synchronisations in between.  The library enqueues kernels only (no
memset, copy or allocation), so every call can be captured."""
import numpy as np
import pytest
import torch

import denoiser_attention_amd as tt
from denoiser_attention_amd import synth
from helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def _bf16(a):
    return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)


def _attn_set(cfg, seed, P):
    inp = synth.attn_inputs(cfg, seed=seed, prefix_cap=P)
    return {n: _bf16(inp[n]) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}, inp["scale"]


def _same(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def test_captured_step_replays_like_eager():
    """Attention with key splits (partials in the workspace, merged by a
    second kernel), then the vocabulary pass and the commit."""
    B, Hq, Hkv, L, P, D, V, k = 2, 32, 2, 32, 600, 128, 5000, 8
    cfg = synth.get_config("decode_b8_p2048_l32").with_(batch=B, prefix_len=P, vocab=V)
    stream = torch.cuda.Stream(DEV)
    t, scale = _attn_set(cfg, 31, P)
    t2, _ = _attn_set(cfg, 32, P)
    x = torch.from_numpy(synth.logits(cfg, seed=31)).to(DEV)
    x2 = torch.from_numpy(synth.logits(cfg, seed=32)).to(DEV)
    mask = torch.from_numpy((np.random.default_rng(31).random((B, L)) < 0.8).astype(np.uint8)).to(DEV)
    out = torch.empty_like(t["q"])
    out2 = torch.empty_like(t["q"])
    tokens = torch.empty((B, L), dtype=torch.int32, device=DEV)
    mask_out = torch.empty_like(mask)
    conf = torch.empty((B, L), dtype=torch.float32, device=DEV)
    pred = torch.empty((B, L), dtype=torch.int32, device=DEV)
    ws_a = torch.empty(tt.attn_workspace_bytes(B, P, L, Hq, Hkv, D, torch.bfloat16),
                       dtype=torch.uint8, device=DEV)
    assert ws_a.numel() > 0, "the shape should plan key splits"
    ws_u = torch.empty(tt.unmask_workspace_bytes(B, L, V), dtype=torch.uint8, device=DEV)
    with torch.cuda.stream(stream):
        attn = tt.prepare_block_attn(t["q"], t["k_ctx"], t["v_ctx"], P, t["k_blk"], t["v_blk"],
                                     scale, out, workspace=ws_a, stream=stream)
        other = tt.prepare_block_attn(t2["q"], t2["k_ctx"], t2["v_ctx"], P, t2["k_blk"],
                                      t2["v_blk"], scale, out2, workspace=ws_a, stream=stream)
        red = tt.prepare_unmask_reduce(x, mask, ws_u, stream=stream)
        red2 = tt.prepare_unmask_reduce(x2, mask, ws_u, stream=stream)
        com = tt.prepare_unmask_commit(mask, k, tokens, mask_out, V, ws_u, conf_out=conf,
                                       pred_out=pred, stream=stream)

    def reset():
        out.fill_(0)
        tokens.fill_(7)
        mask_out.fill_(9)
        conf.fill_(5.0)
        pred.fill_(-5)

    def step():
        attn()
        red()
        com()

    with torch.cuda.stream(stream):
        reset()
        step()
    torch.cuda.synchronize()
    ref = [a.clone() for a in (out, tokens, mask_out, conf, pred)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        say(f"graph replay {r}")
        with torch.cuda.stream(stream):
            # Other eager work over the same workspaces, then fresh outputs.
            other()
            red2()
            reset()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, tokens, mask_out, conf, pred), ref):
            assert _same(a, b), f"replay {r}"


def test_captured_noalloc_step_replays_like_eager():
    """The allocation-free unmask step inside a graph, with eager calls of the
    same entry point (which share its static scratch) between replays."""
    B, L, V, k = 4, 32, 20000, 5
    cfg = synth.get_config("decode_b8_p2048_l32").with_(batch=B, vocab=V)
    stream = torch.cuda.Stream(DEV)
    x = torch.from_numpy(synth.logits(cfg, seed=41)).to(DEV)
    x2 = torch.from_numpy(synth.logits(cfg, seed=42, batch=2)).to(DEV)
    mask = torch.from_numpy((np.random.default_rng(41).random((B, L)) < 0.7).astype(np.uint8)).to(DEV)
    mask2 = torch.ones((2, L), dtype=torch.uint8, device=DEV)
    tokens, tokens2 = (torch.empty((n, L), dtype=torch.int32, device=DEV) for n in (B, 2))
    mask_out, mask_out2 = torch.empty_like(mask), torch.empty_like(mask2)
    conf = torch.empty((B, L), dtype=torch.float32, device=DEV)

    def reset():
        tokens.fill_(3)
        mask_out.fill_(9)
        conf.fill_(5.0)

    def step():
        tt.unmask_step_noalloc(x, mask, k, tokens, mask_out=mask_out, conf_out=conf, stream=stream)

    with torch.cuda.stream(stream):
        reset()
        step()
    torch.cuda.synchronize()
    ref = [a.clone() for a in (tokens, mask_out, conf)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        say(f"noalloc graph replay {r}")
        with torch.cuda.stream(stream):
            tt.unmask_step_noalloc(x2, mask2, 2, tokens2, mask_out=mask_out2, stream=stream)
            reset()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for a, b in zip((tokens, mask_out, conf), ref):
            assert _same(a, b), f"replay {r}"


@pytest.mark.parametrize("d_model", [384, 160])
def test_captured_lmhead_step_replays_like_eager(d_model):
    """The fused LM head + unmask (row compaction, statistics, slice merge,
    commit) inside a graph; d_model 384 takes the persistent hand-over path,
    160 one workgroup per item with a 32-column last stage."""
    B, L, V = 2, 32, 5000
    cfg = synth.get_config("decode_b8_p2048_l32").with_(batch=B, vocab=V)
    stream = torch.cuda.Stream(DEV)
    li = synth.lmhead_inputs(cfg, d_model=d_model, seed=51)
    li2 = synth.lmhead_inputs(cfg, d_model=d_model, seed=52)
    h, w = _bf16(li["hidden"]), _bf16(li["weight"])
    h2, w2 = _bf16(li2["hidden"]), _bf16(li2["weight"])
    mask = torch.from_numpy((np.random.default_rng(51).random((B, L)) < 0.8).astype(np.uint8)).to(DEV)
    sel = tt.select_rule("top_k", k=6)
    tokens, tokens2 = (torch.empty((B, L), dtype=torch.int32, device=DEV) for _ in range(2))
    mask_out, mask_out2 = torch.empty_like(mask), torch.empty_like(mask)
    conf = torch.empty((B, L), dtype=torch.float32, device=DEV)
    ws = torch.empty(tt.lmhead_unmask_workspace_bytes(B, L, V, d_model), dtype=torch.uint8,
                     device=DEV)
    with torch.cuda.stream(stream):
        call = tt.prepare_lmhead_unmask_step(h, w, mask, sel, tokens, mask_out, conf_out=conf,
                                             workspace=ws, stream=stream)
        other = tt.prepare_lmhead_unmask_step(h2, w2, mask, sel, tokens2, mask_out2,
                                              workspace=ws, stream=stream)

    def reset():
        tokens.fill_(3)
        mask_out.fill_(9)
        conf.fill_(5.0)

    with torch.cuda.stream(stream):
        reset()
        call()
    torch.cuda.synchronize()
    ref = [a.clone() for a in (tokens, mask_out, conf)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        say(f"lmhead graph replay {r} d_model={d_model}")
        with torch.cuda.stream(stream):
            other()
            reset()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for a, b in zip((tokens, mask_out, conf), ref):
            assert _same(a, b), f"replay {r}"
