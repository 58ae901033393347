"""GPU parity of the per-sequence-prefix attention (tt_block_attn_varlen) and
of the training-style pass over all noisy blocks (tt_block_attn_multiblock)
against the oracle, element by element on small shapes with ragged tiles and
on sampled heads at full size.  Cache rows past each entry's own prefix, and
the clean rows of each block and after, hold large garbage: reading one fails
the comparison."""
import numpy as np
import pytest
import torch

import oracle
from denoiser_attention_amd import synth
from helpers import as_f64, check_attn, say, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def base_cfg(**kw):
    return synth.get_config("decode_b8_p2048_l32").with_(**kw)


def gpu_varlen(inp, lens=None, **kw):
    from denoiser_attention_amd import block_attn_varlen
    t = {n: to_dev(inp[n], DEV) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}
    lens = inp["prefix_lens"] if lens is None else lens
    ld = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(DEV)
    out = block_attn_varlen(t["q"], t["k_ctx"], t["v_ctx"], ld, inp["prefix_len"], t["k_blk"],
                            t["v_blk"], inp["scale"], **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def oracle_varlen(inp, lens=None, pairs=None):
    lens = inp["prefix_lens"] if lens is None else lens
    q, kc, vc = as_f64(inp["q"]), as_f64(inp["k_ctx"]), as_f64(inp["v_ctx"])
    kb, vb = as_f64(inp["k_blk"]), as_f64(inp["v_blk"])
    if pairs is None:
        return oracle.block_attn_varlen(q, kc, vc, lens, kb, vb, inp["scale"])[0]
    G = q.shape[1] // kb.shape[1]
    res = {}
    for b, h in pairs:
        g = h // G
        o, _ = oracle.block_attn(q[b:b + 1, h:h + 1], kc[b:b + 1, g:g + 1], vc[b:b + 1, g:g + 1],
                                 int(lens[b]), kb[b:b + 1, g:g + 1], vb[b:b + 1, g:g + 1],
                                 inp["scale"])
        res[(b, h)] = o[0, 0]
    return res


VARLEN_SHAPES = [
    # (B, Hq, Hkv, L, Pmax, Pcap, D)
    (5, 8, 2, 37, 150, 160, 128),
    (4, 6, 3, 20, 96, 96, 64),
    (3, 32, 2, 1, 300, 300, 128),
    (6, 4, 4, 5, 40, 45, 128),      # G*L = 5 (MFMA under auto)
]


@pytest.mark.parametrize("shape", VARLEN_SHAPES, ids=[str(s) for s in VARLEN_SHAPES])
@pytest.mark.parametrize("path", ["auto", "mfma", "shuffle"])
@pytest.mark.parametrize("out_f32", [False, True])
def test_varlen_bf16_shapes(shape, path, out_f32):
    B, Hq, Hkv, L, Pmax, Pcap, D = shape
    cfg = base_cfg(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, block_len=L)
    inp = synth.varlen_inputs(cfg, seed=11, max_prefix_len=Pmax, prefix_cap=Pcap)
    kw = dict(path=path)
    if out_f32:
        kw["out_dtype"] = torch.float32
    got = gpu_varlen(inp, **kw)
    check_attn(got, oracle_varlen(inp), "bf16", not out_f32,
               f"varlen {shape} {path} lens={inp['prefix_lens'].tolist()}")


@pytest.mark.parametrize("groups,splits", [(1, 1), (1, 3), (2, 0), (2, 2), (1, 9)])
def test_varlen_splits_and_groups(groups, splits):
    cfg = base_cfg(batch=6, block_len=24)
    inp = synth.varlen_inputs(cfg, seed=12, max_prefix_len=700, prefix_cap=777)
    got = gpu_varlen(inp, path="mfma", kv_groups=groups, kv_splits=splits,
                     out_dtype=torch.float32)
    check_attn(got, oracle_varlen(inp), "bf16", False, f"varlen groups={groups} splits={splits}")


@pytest.mark.parametrize("splits", [0, 2])
def test_varlen_rows64(splits):
    cfg = base_cfg(batch=5, block_len=40)
    inp = synth.varlen_inputs(cfg, seed=16, max_prefix_len=400, prefix_cap=410)
    got = gpu_varlen(inp, path="mfma", rows_per_wave=64, kv_splits=splits, out_dtype=torch.float32)
    check_attn(got, oracle_varlen(inp), "bf16", False, f"varlen rows64 splits={splits}")


@pytest.mark.parametrize("splits", [0, 2])
def test_varlen_stream8(splits):
    cfg = base_cfg(batch=5, block_len=40)
    inp = synth.varlen_inputs(cfg, seed=17, max_prefix_len=400, prefix_cap=410)
    got = gpu_varlen(inp, path="mfma", stream_waves=8, kv_splits=splits, out_dtype=torch.float32)
    check_attn(got, oracle_varlen(inp), "bf16", False, f"varlen stream8 splits={splits}")


def test_varlen_fp32():
    cfg = synth.get_config("tiny_fp32")
    inp = synth.varlen_inputs(cfg, seed=13, batch=4, max_prefix_len=53, prefix_cap=70)
    got = gpu_varlen(inp)
    check_attn(got, oracle_varlen(inp), "fp32", False, "varlen fp32")


def test_varlen_lengths_are_clamped():
    cfg = base_cfg(batch=4, block_len=16)
    inp = synth.attn_inputs(cfg, seed=14, prefix_len=80, prefix_cap=90)
    lens = np.array([-5, 80, 200, 33], dtype=np.int32)   # 200 > bound: treated as 80
    clamped = np.clip(lens, 0, 80)
    gk = synth.bf16_bits_from_f32(np.float32([synth.GARBAGE]))[0]
    for b, p in enumerate(clamped):                      # rows past each clamped length: garbage
        inp["k_ctx"][b, :, p:] = gk
        inp["v_ctx"][b, :, p:] = gk
    got = gpu_varlen(inp, lens=lens, out_dtype=torch.float32)
    check_attn(got, oracle_varlen(inp, lens=clamped), "bf16", False, "varlen clamped")


def test_varlen_full_size_decode_mix():
    """Decode-shaped workload (B 8, up to 2048 cached rows, block 32), lengths
    mixed across the batch; the oracle checks two heads of every entry."""
    cfg = synth.get_config("decode_b8_p2048_l32")
    inp = synth.varlen_inputs(cfg, seed=15, max_prefix_len=2048)
    say(f"varlen decode lens {inp['prefix_lens'].tolist()}")
    got = gpu_varlen(inp)
    pairs = [(b, h) for b in range(cfg.batch) for h in (3, 30)]
    for (b, h), o in oracle_varlen(inp, pairs=pairs).items():
        check_attn(got[b, h], o, "bf16", True, f"varlen decode b={b} h={h}")


def gpu_multiblock(inp, **kw):
    from denoiser_attention_amd import block_attn_multiblock
    t = {n: to_dev(inp[n], DEV) for n in ("q", "k_ctx", "v_ctx", "k_noisy", "v_noisy")}
    out = block_attn_multiblock(t["q"], t["k_ctx"], t["v_ctx"], t["k_noisy"], t["v_noisy"],
                                inp["block_size"], inp["scale"], **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def oracle_multiblock(inp, pairs=None):
    q, kc, vc = as_f64(inp["q"]), as_f64(inp["k_ctx"]), as_f64(inp["v_ctx"])
    kn, vn = as_f64(inp["k_noisy"]), as_f64(inp["v_noisy"])
    S = inp["block_size"]
    if pairs is None:
        return oracle.block_attn_multiblock(q, kc, vc, kn, vn, S, inp["scale"])[0]
    G = q.shape[1] // kn.shape[1]
    res = {}
    for b, h in pairs:
        g = h // G
        o, _ = oracle.block_attn_multiblock(q[b:b + 1, h:h + 1], kc[b:b + 1, g:g + 1],
                                            vc[b:b + 1, g:g + 1], kn[b:b + 1, g:g + 1],
                                            vn[b:b + 1, g:g + 1], S, inp["scale"])
        res[(b, h)] = o[0, 0]
    return res


MB_SHAPES = [
    # (B, Hq, Hkv, N, S, D)
    (2, 8, 2, 4, 16, 128),
    (2, 6, 3, 3, 37, 64),     # block size not a multiple of the key tile
    (1, 16, 2, 1, 40, 128),   # one block: no context row visible
    (3, 4, 4, 5, 3, 128),     # G*S = 3 (MFMA under auto)
]


@pytest.mark.parametrize("shape", MB_SHAPES, ids=[str(s) for s in MB_SHAPES])
@pytest.mark.parametrize("path", ["auto", "mfma", "shuffle"])
@pytest.mark.parametrize("out_f32", [False, True])
def test_multiblock_bf16_shapes(shape, path, out_f32):
    B, Hq, Hkv, N, S, D = shape
    cfg = base_cfg(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D)
    inp = synth.multiblock_inputs(cfg, N, S, seed=21)
    kw = dict(path=path)
    if out_f32:
        kw["out_dtype"] = torch.float32
    got = gpu_multiblock(inp, **kw)
    check_attn(got, oracle_multiblock(inp), "bf16", not out_f32, f"multiblock {shape} {path}")


@pytest.mark.parametrize("groups,splits", [(1, 3), (2, 2), (2, 0), (1, 0)])
def test_multiblock_splits_and_groups(groups, splits):
    cfg = base_cfg(batch=2, n_q_heads=8, n_kv_heads=2)
    inp = synth.multiblock_inputs(cfg, 6, 48, seed=22)
    got = gpu_multiblock(inp, path="mfma", kv_groups=groups, kv_splits=splits,
                         out_dtype=torch.float32)
    check_attn(got, oracle_multiblock(inp), "bf16", False,
               f"multiblock groups={groups} splits={splits}")


@pytest.mark.parametrize("splits", [0, 3])
def test_multiblock_rows64(splits):
    cfg = base_cfg(batch=2, n_q_heads=16, n_kv_heads=2)
    inp = synth.multiblock_inputs(cfg, 5, 40, seed=25)
    got = gpu_multiblock(inp, path="mfma", rows_per_wave=64, kv_splits=splits)
    check_attn(got, oracle_multiblock(inp), "bf16", True, f"multiblock rows64 splits={splits}")


@pytest.mark.parametrize("splits", [0, 3])
def test_multiblock_stream8(splits):
    cfg = base_cfg(batch=2, n_q_heads=16, n_kv_heads=2)
    inp = synth.multiblock_inputs(cfg, 5, 40, seed=26)
    got = gpu_multiblock(inp, path="mfma", stream_waves=8, kv_splits=splits)
    check_attn(got, oracle_multiblock(inp), "bf16", True, f"multiblock stream8 splits={splits}")


def test_multiblock_fp32():
    cfg = synth.get_config("tiny_fp32")
    inp = synth.multiblock_inputs(cfg, 4, 16, seed=23, batch=2)
    got = gpu_multiblock(inp)
    check_attn(got, oracle_multiblock(inp), "fp32", False, "multiblock fp32")


def test_multiblock_training_size_sampled():
    """An 8-block, 2048-token sequence with 256-token blocks and the
    configurations' head layout (32 query heads, 2 KV heads, head_dim 128)."""
    cfg = synth.get_config("block256_b16_p1024")
    inp = synth.multiblock_inputs(cfg, 8, 256, seed=24, batch=1)
    got = gpu_multiblock(inp)
    for (b, h), o in oracle_multiblock(inp, pairs=[(0, 0), (0, 17)]).items():
        check_attn(got[b, h], o, "bf16", True, f"multiblock 8x256 h={h}")
    assert np.isfinite(got).all()


def test_prepared_calls_match():
    """The prepared (validate once, reissue) varlen and multiblock calls the
    benchmark times produce the unprepared calls' outputs bit for bit, on a
    side stream, call after call."""
    from denoiser_attention_amd import (block_attn_multiblock, block_attn_varlen,
                                        prepare_block_attn_multiblock, prepare_block_attn_varlen)
    st = torch.cuda.Stream(DEV)
    cfg = base_cfg(batch=3, n_q_heads=8, n_kv_heads=2, prefix_len=300, block_len=21)
    inp = synth.varlen_inputs(cfg, seed=41, max_prefix_len=300)
    t = {n: to_dev(inp[n], DEV) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}
    ld = torch.from_numpy(np.asarray(inp["prefix_lens"], dtype=np.int32)).to(DEV)
    ref = block_attn_varlen(t["q"], t["k_ctx"], t["v_ctx"], ld, 300, t["k_blk"], t["v_blk"],
                            inp["scale"], kv_splits=3)
    out = torch.full_like(ref, 7.0)
    with torch.cuda.stream(st):
        call = prepare_block_attn_varlen(t["q"], t["k_ctx"], t["v_ctx"], ld, 300, t["k_blk"],
                                         t["v_blk"], inp["scale"], out, kv_splits=3, stream=st)
        for _ in range(3):
            call()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)

    S, N = 16, 3
    mb = synth.multiblock_inputs(base_cfg(batch=2, n_q_heads=4, n_kv_heads=2), n_blocks=N,
                                 block_size=S, seed=42)
    m = {n: to_dev(mb[n], DEV) for n in ("q", "k_ctx", "v_ctx", "k_noisy", "v_noisy")}
    ref = block_attn_multiblock(m["q"], m["k_ctx"], m["v_ctx"], m["k_noisy"], m["v_noisy"], S,
                                mb["scale"])
    out = torch.full_like(ref, 7.0)
    with torch.cuda.stream(st):
        call = prepare_block_attn_multiblock(m["q"], m["k_ctx"], m["v_ctx"], m["k_noisy"],
                                             m["v_noisy"], S, mb["scale"], out, stream=st)
        for _ in range(3):
            call()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
