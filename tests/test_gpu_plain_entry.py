"""GPU parity of the two entry points the path is named by, called through
ctypes exactly as a C caller would: tt_block_attn (no options struct, the
library's own launch plan) and tt_unmask_step with NULL conf_out / pred_out.
Also: binding calls that pass a side stream without making it current.

Block attention: TwoTower paper §2.1 "Bidirectional Attention", Eq. (1).
Unmask: §2.2 "Sampling", Algorithm 2 (fixed-k form)."""
import numpy as np
import pytest
import torch

import oracle
import denoiser_attention_amd as tt
from denoiser_attention_amd import _binding as B
from denoiser_attention_amd import synth
from helpers import check_attn, check_unmask, oracle_attn, say, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def plain_block_attn(inp, out_dtype=None):
    """tt_block_attn through ctypes: device buffers from torch, the workspace
    sized by tt_block_attn_workspace_bytes with no options, the null stream."""
    t = {n: to_dev(inp[n], DEV) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}
    q = t["q"]
    Bn, Hq, L, D = q.shape
    Hkv, Pcap = t["k_ctx"].shape[1], t["k_ctx"].shape[2]
    dt = B.TT_BF16 if q.dtype == torch.bfloat16 else B.TT_FP32
    odt = dt if out_dtype is None else out_dtype
    out = torch.empty(q.shape, dtype=torch.float32 if odt == B.TT_FP32 else torch.bfloat16,
                      device=DEV)
    lib = tt.lib()
    ws_n = lib.tt_block_attn_workspace_bytes(Bn, inp["prefix_len"], L, Hq, Hkv, D, dt, None)
    assert ws_n != B.SIZE_MAX
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    st = lib.tt_block_attn(q.data_ptr(), t["k_ctx"].data_ptr(), t["v_ctx"].data_ptr(),
                           inp["prefix_len"], t["k_blk"].data_ptr(), t["v_blk"].data_ptr(), L,
                           Hq, Hkv, D, float(inp["scale"]), out.data_ptr(), Bn, Pcap, dt, odt,
                           ws.data_ptr() if ws_n else None, ws_n, None)
    assert st == B.TT_OK, B.status_string(st)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), ws_n


def test_plain_block_attn_tiny_fp32():
    cfg = synth.get_config("tiny_fp32")
    inp = synth.attn_inputs(cfg, seed=0)
    got, _ = plain_block_attn(inp)
    check_attn(got, oracle_attn(inp), "fp32", False, "plain tt_block_attn tiny_fp32")


def test_plain_block_attn_decode_sampled():
    """The decode-shaped workload (B8 P2048 L32, 32/2 heads, D128, bf16) in
    the library's own plan (key splits and their merge); the oracle checks
    three (batch, head) pairs element by element."""
    cfg = synth.get_config("decode_b8_p2048_l32")
    inp = synth.attn_inputs(cfg, seed=0)
    got, ws_n = plain_block_attn(inp)
    say(f"plain tt_block_attn decode: workspace {ws_n} B")
    assert ws_n > 0, "the decode plan splits the key range"
    pairs = [(0, 0), (3, 17), (7, 31)]
    ref = oracle_attn(inp, heads=sorted({h for _, h in pairs}), batches=sorted({b for b, _ in pairs}))
    for b, h in pairs:
        check_attn(got[b, h], ref[(b, h)], "bf16", True, f"plain decode b={b} h={h}")


def plain_unmask_step(x, mask, k, tokens0):
    lib = tt.lib()
    Bn, L, V = x.shape
    xd = torch.from_numpy(x).to(DEV)
    m = torch.from_numpy(mask).to(DEV)
    tok = torch.from_numpy(tokens0.astype(np.int32)).to(DEV)
    mo = torch.full((Bn, L), 9, dtype=torch.uint8, device=DEV)
    ws_n = lib.tt_unmask_workspace_bytes(Bn, L, V)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    st = lib.tt_unmask_step(xd.data_ptr(), m.data_ptr(), k, tok.data_ptr(), mo.data_ptr(), Bn, L,
                            V, None, None, ws.data_ptr(), ws_n, None)
    assert st == B.TT_OK, B.status_string(st)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), mo.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny_fp32", "decode_b8_p2048_l32"])
def test_plain_unmask_step_null_diagnostics(name):
    """Every step of the workload (up to 3 sequences) to an empty block,
    teacher-forced, with conf_out and pred_out NULL: ids and commit sets are
    read from tokens and mask."""
    cfg = synth.get_config(name)
    nb = min(cfg.batch, 3)     # the oracle's sorts over 131072 ids are slow on the host
    mask = synth.initial_mask(cfg, batch=nb)
    tokens = np.full(mask.shape, -7, np.int32)
    for step in range(cfg.steps):
        x = synth.logits(cfg, seed=0, step=step, batch=nb)
        ref = oracle.unmask_step(x, mask, cfg.k)
        tok, mo = plain_unmask_step(x, mask, cfg.k, tokens)
        # check_unmask wants the diagnostics: the oracle's at masked positions
        # stand in for them, so only tokens, mask and commit sets are compared.
        got = dict(tokens=tok, mask_out=mo,
                   pred=np.where(mask != 0, ref["pred"], -1),
                   conf=np.where(mask != 0, ref["conf"], -1.0))
        check_unmask(got, ref, mask, cfg.k, tokens, f"plain tt_unmask_step {name} step {step}")
        tokens = tok
        mask = ref["mask_out"]
        del x
    assert mask.sum() == 0


def test_binding_side_stream_not_current():
    """The binding allocates its own workspaces and outputs on the stream the
    call is launched on, so a side stream that is not the current stream is
    safe: results equal those of the same calls on the current stream."""
    cfg = synth.get_config("decode_b8_p2048_l32")
    inp = synth.attn_inputs(cfg, seed=5, batch=2)
    t = {n: to_dev(inp[n], DEV) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}
    x = torch.from_numpy(synth.logits(cfg, seed=5, step=0, batch=2)).to(DEV)
    mask = torch.ones((2, cfg.block_len), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream(DEV)
    torch.cuda.synchronize()
    assert torch.cuda.current_stream(DEV) != side
    outs = []
    for s in (None, side):
        res = []
        for _ in range(3):   # later calls would reuse freed blocks if they were unsafe
            o = tt.block_attn(t["q"], t["k_ctx"], t["v_ctx"], inp["prefix_len"], t["k_blk"],
                              t["v_blk"], inp["scale"], stream=s)
            tok = torch.zeros((2, cfg.block_len), dtype=torch.int32, device=DEV)
            if s is not None:
                tok.record_stream(s)
            _, mo = tt.unmask_step(x, mask, cfg.k, tok, stream=s)
            res.append((o, tok, mo))
            # junk allocations on the current stream in between
            junk = torch.full((1 << 22,), 3.0, device=DEV)
            del junk
        torch.cuda.synchronize()
        outs.append([(o.float().cpu(), tk.cpu(), m.cpu()) for o, tk, m in res])
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
