"""Seeded random-shape parity sweeps against the oracle: attention (bf16 and
fp32, every kernel family and launch option, ragged shapes, capacity padding)
and the unmask step under every selection rule (vocabulary sizes that are not
multiples of 4, random masks).  The shapes are drawn once from a fixed seed,
so the cases are the same on every run; each is small enough for the fp64
oracle."""
import numpy as np
import pytest
import torch

import oracle
from denoiser_attention_amd import synth
from helpers import check_attn, gpu_attn, oracle_attn
from test_gpu_select import MASK_ID, MODES, check_select, gpu_step, varied_logits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def attn_cases(n=48, seed=2024):
    rng = np.random.default_rng(seed)
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


def unmask_cases(n=32, seed=77):
    rng = np.random.default_rng(seed)
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
    check_select(got, ref, mask, tokens0, mode, f"random {case[:6]}")
