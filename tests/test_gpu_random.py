"""Seeded random-shape parity sweeps against the oracle: attention (bf16 and
fp32, every kernel family and launch option, ragged shapes, capacity padding)
and the unmask step under every selection rule (vocabulary sizes that are not
multiples of 4, random masks).  The shapes are drawn once from a fixed seed,
so the cases are the same on every run; each is small enough for the fp64
oracle.  TT_RANDOM_SCALE=n (default 1) draws n times as many cases of each
kind; the first ones are the default cases."""
import os

import numpy as np
import pytest
import torch

import oracle
from denoiser_attention_amd import synth
from helpers import check_attn, gpu_attn, oracle_attn
from test_gpu_select import MASK_ID, MODES, check_select, gpu_step, varied_logits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCALE = max(1, int(os.environ.get("TT_RANDOM_SCALE", "1")))


def attn_cases(n=48, seed=2024):
    rng = np.random.default_rng(seed)
    n *= SCALE
    cases = []
    for i in range(n):
        fp32 = i % 8 == 7
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        L = int(rng.integers(1, 71))
        P = int(rng.integers(0, 301))
        Pcap = P + int(rng.integers(0, 21))
        B = int(rng.integers(1, 4))
        if fp32:
            D = int(rng.choice([64, 128, 256]))
            path = str(rng.choice(["auto", "shuffle"]))
        else:
            path = str(rng.choice(["auto", "mfma", "shuffle"]))
            D = int(rng.choice([64, 128] if path == "mfma" else [64, 128, 256]))
        splits = int(rng.choice([0, 0, 1, 2, 3, 5]))
        groups = int(rng.choice([0, 1, 2])) if path == "mfma" else 0
        out_f32 = bool(rng.integers(0, 2)) or fp32
        cases.append((i, fp32, B, G * Hkv, Hkv, L, P, Pcap, D, path, splits, groups, out_f32))
    return cases


@pytest.mark.parametrize("case", attn_cases(), ids=lambda c: f"attn{c[0]}")
def test_random_attention(case):
    i, fp32, B, Hq, Hkv, L, P, Pcap, D, path, splits, groups, out_f32 = case
    base = synth.get_config("tiny_fp32" if fp32 else "decode_b8_p2048_l32")
    cfg = base.with_(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, prefix_len=P,
                     block_len=L)
    inp = synth.attn_inputs(cfg, seed=100 + i, prefix_cap=Pcap)
    if Pcap == 0:
        inp["k_ctx"] = inp["k_ctx"].reshape(B, Hkv, 0, D)
    kw = dict(path=path, kv_splits=splits, kv_groups=groups)
    if out_f32 and not fp32:
        kw["out_dtype"] = torch.float32
    got = gpu_attn(inp, DEV, **kw)
    check_attn(got, oracle_attn(inp), "fp32" if fp32 else "bf16", not out_f32, f"random {case}")


def wave_layout_cases(n=12, seed=3131):
    """bf16 D = 128 MFMA cases with 64-row waves or 8-wave tile streams."""
    rng = np.random.default_rng(seed)
    n *= SCALE
    cases = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 4, 16]))
        opt = {"rows_per_wave": 64} if i % 2 == 0 else {"stream_waves": 8}
        cases.append((i, int(rng.integers(1, 4)), G * Hkv, Hkv, int(rng.integers(1, 71)),
                      int(rng.integers(0, 301)), int(rng.choice([0, 1, 3])),
                      bool(rng.integers(0, 2)), opt))
    return cases


@pytest.mark.parametrize("case", wave_layout_cases(), ids=lambda c: f"layout{c[0]}")
def test_random_wave_layouts(case):
    i, B, Hq, Hkv, L, P, splits, out_f32, opt = case
    cfg = synth.get_config("decode_b8_p2048_l32").with_(batch=B, n_q_heads=Hq, n_kv_heads=Hkv,
                                                        head_dim=128, prefix_len=P, block_len=L)
    inp = synth.attn_inputs(cfg, seed=600 + i, prefix_cap=P + i % 3)
    if P + i % 3 == 0:
        inp["k_ctx"] = inp["k_ctx"].reshape(B, Hkv, 0, 128)
    kw = dict(path="mfma", kv_splits=splits, **opt)
    if out_f32:
        kw["out_dtype"] = torch.float32
    got = gpu_attn(inp, DEV, **kw)
    check_attn(got, oracle_attn(inp), "bf16", not out_f32, f"random layout {case}")


def unmask_cases(n=32, seed=77):
    rng = np.random.default_rng(seed)
    n *= SCALE
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 7))
        L = int(rng.integers(1, 301))
        V = int(rng.integers(1, 20001))
        density = float(rng.uniform(0.1, 1.0))
        mode = str(rng.choice(list(MODES)))
        if mode in ("top_k", "leftmost"):
            params = dict(k=int(rng.integers(0, L + 3)))
        elif mode == "threshold":
            params = dict(gamma=float(rng.choice([0.0, 0.3, 0.8, 0.99, 1.5])),
                          steps_left=int(rng.integers(1, 9)))
        else:
            T = int(rng.integers(1, 9))
            params = dict(step=int(rng.integers(1, T + 1)), n_steps=T)
        split = bool(rng.integers(0, 2))
        cases.append((i, B, L, V, density, mode, params, split))
    return cases


@pytest.mark.parametrize("case", unmask_cases(), ids=lambda c: f"unmask{c[0]}")
def test_random_unmask(case):
    i, B, L, V, density, mode, params, split = case
    rng = np.random.default_rng(500 + i)
    x = varied_logits(rng, B, L, V)
    mask = (rng.random((B, L)) < density).astype(np.uint8)
    tokens0 = np.full((B, L), MASK_ID, np.int32)
    got = gpu_step(x, mask, tokens0, mode, split=split, **params)
    ref = oracle.unmask_step_select(x.astype(np.float64), mask, MODES[mode], **params)
    check_select(got, ref, mask, tokens0, mode, f"random {case[:6]}", **params)


def varlen_cases(n=16, seed=4048):
    rng = np.random.default_rng(seed)
    n *= SCALE
    cases = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([2, 4, 16]))
        cases.append((i, int(rng.integers(2, 6)), G * Hkv, Hkv, int(rng.integers(1, 41)),
                      int(rng.integers(1, 400)), int(rng.choice([64, 128])),
                      str(rng.choice(["auto", "mfma", "shuffle"])), int(rng.choice([0, 1, 3]))))
    return cases


@pytest.mark.parametrize("case", varlen_cases(), ids=lambda c: f"varlen{c[0]}")
def test_random_varlen(case):
    from test_gpu_varlen import gpu_varlen, oracle_varlen
    i, B, Hq, Hkv, L, Pmax, D, path, splits = case
    cfg = synth.get_config("decode_b8_p2048_l32").with_(batch=B, n_q_heads=Hq, n_kv_heads=Hkv,
                                                        head_dim=D, block_len=L)
    inp = synth.varlen_inputs(cfg, seed=200 + i, max_prefix_len=Pmax, prefix_cap=Pmax + i % 5)
    got = gpu_varlen(inp, path=path, kv_splits=splits, out_dtype=torch.float32)
    check_attn(got, oracle_varlen(inp), "bf16", False, f"random varlen {case}")


def multiblock_cases(n=12, seed=5050):
    rng = np.random.default_rng(seed)
    n *= SCALE
    cases = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([2, 4, 16]))
        cases.append((i, int(rng.integers(1, 3)), G * Hkv, Hkv, int(rng.integers(1, 7)),
                      int(rng.integers(1, 50)), int(rng.choice([64, 128])),
                      str(rng.choice(["auto", "mfma", "shuffle"])), int(rng.choice([0, 2]))))
    return cases


@pytest.mark.parametrize("case", multiblock_cases(), ids=lambda c: f"multiblock{c[0]}")
def test_random_multiblock(case):
    from test_gpu_varlen import gpu_multiblock, oracle_multiblock
    i, B, Hq, Hkv, N, S, D, path, splits = case
    cfg = synth.get_config("decode_b8_p2048_l32").with_(batch=B, n_q_heads=Hq, n_kv_heads=Hkv,
                                                        head_dim=D)
    inp = synth.multiblock_inputs(cfg, N, S, seed=300 + i)
    got = gpu_multiblock(inp, path=path, kv_splits=splits, out_dtype=torch.float32)
    check_attn(got, oracle_multiblock(inp), "bf16", False, f"random multiblock {case}")


def lmhead_cases(n=10, seed=6060):
    rng = np.random.default_rng(seed)
    n *= SCALE
    cases = []
    for i in range(n):
        mode = str(rng.choice(list(MODES)))
        if mode in ("top_k", "leftmost"):
            params = dict(k=int(rng.integers(0, 9)))
        elif mode == "threshold":
            params = dict(gamma=float(rng.choice([0.5, 0.9])), steps_left=int(rng.integers(1, 5)))
        else:
            params = dict(step=1, n_steps=int(rng.integers(1, 5)))
        cases.append((i, int(rng.integers(1, 5)), int(rng.integers(1, 60)),
                      int(rng.integers(1, 3000)), int(32 * rng.integers(1, 9)),
                      float(rng.uniform(0.2, 1.0)), mode, params))
    return cases


@pytest.mark.parametrize("case", lmhead_cases(), ids=lambda c: f"lmhead{c[0]}")
def test_random_lmhead(case):
    from test_gpu_lmhead import check
    i, B, L, V, d, density, mode, params = case
    cfg = synth.get_config("decode_b8_p2048_l32").with_(vocab=V)
    inp = synth.lmhead_inputs(cfg, d_model=d, seed=400 + i, batch=B, block_len=L)
    rng = np.random.default_rng(700 + i)
    mask = (rng.random((B, L)) < density).astype(np.uint8)
    check(inp, mask, mode, f"random lmhead {case[:6]}", **params)
