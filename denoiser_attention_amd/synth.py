"""Seeded synthetic inputs for the denoising-step workloads.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic (no attention, no softmax, no selection), so both the
CPU oracle and the HIP path can be fed from it without sharing any compute
code.  It imports numpy only: no torch, no HIP library.

Workloads (one per named configuration) follow the five synthetic shapes the
denoising step is measured on, plus two supplementary attention shapes at the
paper's default block size S=16 and at a single-token block.  The pages
publish no tensor shapes, head counts or vocabulary size; every size below is
a synthetic stand-in for the real denoiser inputs and logits (TwoTower paper,
§3 "Results", which evaluates on benchmark problems with trained weights that
are not available here).

Readings taken where the workload descriptions leave a detail open:

* "N(0, s)" draws are ``standard_normal() * s`` (s is a standard deviation).
* bf16 tensors are drawn in fp32 and rounded to bf16 by round-to-nearest-even
  on the host, so both sides see identical bf16 bit patterns.
* Planted peak (decode config): for floor(L/2) seeded positions of every
  sequence a seeded id gets the value ``row max + 8`` (fp32), which makes it
  the unique argmax.
* Injected ties (high-batch config): for round(0.05*B*L) seeded positions, the
  row's maximum value is copied to one other seeded id of the same row.
* Outlier channels (high-batch config): round(0.01*Hkv*D) seeded
  (kv-head, channel) pairs of K and V (cache and block alike) are multiplied
  by 10 before rounding to bf16.
* Every step of a block draws fresh logits and fresh attention inputs (the
  denoiser re-runs on the updated block each step); streams are independent
  through ``SeedSequence([seed, config_id, tensor_id, step])``.
* Rows of the context cache beyond ``prefix_len`` (capacity padding) are
  filled with large finite garbage so that any over-read changes the result.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Config", "CONFIGS", "get_config", "bf16_bits_from_f32", "f32_from_bf16_bits",
    "attn_inputs", "logits", "initial_mask", "GARBAGE",
]

# Magnitude of the garbage written into cache rows that are not visible.
GARBAGE = 3.0e4


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cid: int                 # small integer used in seed derivation
    batch: int
    prefix_len: int
    block_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str               # "fp32" or "bf16" for Q/K/V
    qkv_std: float
    vocab: int
    logit_std: float
    k: int                   # tokens committed per step and sequence
    steps: int               # steps to empty the block (block_len / k)
    plant_peaks: bool = False
    tie_frac: float = 0.0
    outlier_frac: float = 0.0
    outlier_mult: float = 10.0
    scale: float | None = None  # None: 1/sqrt(head_dim)
    description: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS: dict[str, Config] = {c.name: c for c in [
    Config("tiny_fp32", 1, batch=1, prefix_len=64, block_len=16, n_q_heads=4, n_kv_heads=1,
           head_dim=64, dtype="fp32", qkv_std=1.0, vocab=1000, logit_std=2.0, k=4, steps=4,
           scale=1.0 / 8.0,
           description="tiny fp32: B1 P64 L16 4q/1kv D64, V1000, k4 x4 steps"),
    Config("decode_b8_p2048_l32", 2, batch=8, prefix_len=2048, block_len=32, n_q_heads=32,
           n_kv_heads=2, head_dim=128, dtype="bf16", qkv_std=1.0, vocab=131072, logit_std=3.0,
           k=8, steps=4, plant_peaks=True,
           description="bf16 decode-shaped step: B8 P2048 L32 32q/2kv D128, V131072, k8"),
    Config("block256_b16_p1024", 3, batch=16, prefix_len=1024, block_len=256, n_q_heads=32,
           n_kv_heads=2, head_dim=128, dtype="bf16", qkv_std=1.0, vocab=131072, logit_std=3.0,
           k=32, steps=8,
           description="256 tokens as 1 block: B16 P1024 L256 32q/2kv D128, V131072, k32 x8"),
    Config("gen8k_b4_l256", 4, batch=4, prefix_len=8192, block_len=256, n_q_heads=32,
           n_kv_heads=2, head_dim=128, dtype="bf16", qkv_std=1.0, vocab=131072, logit_std=3.0,
           k=32, steps=8,
           description="8K tokens as 32 blocks of 256: B4 L256 32q/2kv D128, prefix swept "
                       "512..8192 then 8192+256*b up to 16128, V131072, k32"),
    Config("highbatch_b64_p4096_l64", 5, batch=64, prefix_len=4096, block_len=64, n_q_heads=32,
           n_kv_heads=2, head_dim=128, dtype="bf16", qkv_std=1.0, vocab=131072, logit_std=3.0,
           k=16, steps=4, tie_frac=0.05, outlier_frac=0.01,
           description="high batch: B64 P4096 L64 32q/2kv D128, K/V outlier channels x10, "
                       "V131072 with 5% injected ties, k16 x4"),
    # Supplementary attention-only shapes (prefix-bound): decode geometry at the
    # paper's default block size S=16, and at a single-token block.
    Config("decode_l16", 6, batch=8, prefix_len=2048, block_len=16, n_q_heads=32, n_kv_heads=2,
           head_dim=128, dtype="bf16", qkv_std=1.0, vocab=131072, logit_std=3.0, k=4, steps=4,
           description="supplementary: decode geometry at L16 (prefix-bound attention)"),
    Config("decode_l1", 7, batch=8, prefix_len=2048, block_len=1, n_q_heads=32, n_kv_heads=2,
           head_dim=128, dtype="bf16", qkv_std=1.0, vocab=131072, logit_std=3.0, k=1, steps=1,
           description="supplementary: decode geometry at L1 (single-token decode attention)"),
    # A prefix-bound shape large enough to be bandwidth-dominated: the high-batch
    # geometry at a single-token block (268 MB of cache K/V per call).
    Config("decode_b64_p4096_l1", 8, batch=64, prefix_len=4096, block_len=1, n_q_heads=32,
           n_kv_heads=2, head_dim=128, dtype="bf16", qkv_std=1.0, vocab=131072, logit_std=3.0,
           k=1, steps=1,
           description="supplementary: high-batch geometry at L1 (prefix-bound, 268 MB of K/V)"),
    # The same 268 MB of cache K/V over twice the sequences at half the prefix:
    # 256 (item, kv head) pairs, one query tile per CU, no key splits.
    Config("decode_b128_p2048_l1", 9, batch=128, prefix_len=2048, block_len=1, n_q_heads=32,
           n_kv_heads=2, head_dim=128, dtype="bf16", qkv_std=1.0, vocab=131072, logit_std=3.0,
           k=1, steps=1,
           description="supplementary: 128 single-token sequences at P2048 (prefix-bound, 268 MB of K/V)"),
]}

# Prefix lengths of the 8K-generation workload: an isolated sweep, and the
# cache lengths seen while 32 blocks of 256 are generated after an 8192 prompt.
GEN8K_SWEEP = tuple(range(512, 8192 + 1, 512))
GEN8K_TRACE = tuple(8192 + 256 * b for b in range(32))


def get_config(name: str, **overrides) -> Config:
    c = CONFIGS[name]
    return c.with_(**overrides) if overrides else c


# --------------------------------------------------------------------------
# bf16 bit patterns (round-to-nearest-even), host side
# --------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs must be finite (the generator never produces NaN/Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, cfg: Config, tensor_id: int, step: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg.cid, tensor_id, step]))


# tensor ids for seed derivation
_T_Q, _T_KCTX, _T_VCTX, _T_KBLK, _T_VBLK, _T_OUTLIER, _T_LOGITS, _T_PLANT, _T_TIE, \
    _T_GARBAGE, _T_LENS, _T_HIDDEN, _T_WEIGHT, _T_HPLANT = range(14)


def attn_inputs(cfg: Config, seed: int = 0, step: int = 0, prefix_len: int | None = None,
                prefix_cap: int | None = None, block_len: int | None = None,
                batch: int | None = None) -> dict:
    """Q, context-cache K/V and in-block K/V for one attention layer call.

    Returns a dict with numpy arrays ``q [B,Hq,L,D]``, ``k_ctx``/``v_ctx``
    ``[B,Hkv,Pcap,D]``, ``k_blk``/``v_blk`` ``[B,Hkv,L,D]`` -- fp32 arrays
    for the fp32 config, uint16 bf16 bit patterns otherwise -- plus the
    scalars ``prefix_len``, ``prefix_cap``, ``scale``, ``dtype``."""
    P = cfg.prefix_len if prefix_len is None else prefix_len
    Pcap = P if prefix_cap is None else prefix_cap
    L = cfg.block_len if block_len is None else block_len
    B = cfg.batch if batch is None else batch
    if Pcap < P:
        raise ValueError("prefix_cap < prefix_len")
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    s = cfg.qkv_std

    def draw(tid, shape):
        return (_rng(seed, cfg, tid, step).standard_normal(shape, dtype=np.float32)
                * np.float32(s))

    q = draw(_T_Q, (B, Hq, L, D))
    k_ctx = draw(_T_KCTX, (B, Hkv, Pcap, D))
    v_ctx = draw(_T_VCTX, (B, Hkv, Pcap, D))
    k_blk = draw(_T_KBLK, (B, Hkv, L, D))
    v_blk = draw(_T_VBLK, (B, Hkv, L, D))
    outliers = []
    if cfg.outlier_frac > 0:
        n_out = int(round(cfg.outlier_frac * Hkv * D))
        r = _rng(seed, cfg, _T_OUTLIER, 0)  # same channels for every step
        flat = r.choice(Hkv * D, size=n_out, replace=False)
        outliers = [(int(f // D), int(f % D)) for f in sorted(flat)]
        m = np.float32(cfg.outlier_mult)
        for (h, c) in outliers:
            for t in (k_ctx, v_ctx, k_blk, v_blk):
                t[:, h, :, c] *= m
    if Pcap > P:
        r = _rng(seed, cfg, _T_GARBAGE, step)
        g = r.choice(np.array([-GARBAGE, GARBAGE], dtype=np.float32), size=(B, Hkv, Pcap - P, D))
        k_ctx[:, :, P:, :] = g
        v_ctx[:, :, P:, :] = -g
    out = dict(q=q, k_ctx=k_ctx, v_ctx=v_ctx, k_blk=k_blk, v_blk=v_blk)
    if cfg.dtype == "bf16":
        out = {n: bf16_bits_from_f32(a) for n, a in out.items()}
    out.update(prefix_len=P, prefix_cap=Pcap, block_len=L, batch=B, scale=cfg.softmax_scale,
               dtype=cfg.dtype, outliers=outliers)
    return out


def logits(cfg: Config, seed: int = 0, step: int = 0, batch: int | None = None,
           block_len: int | None = None, vocab: int | None = None) -> np.ndarray:
    """Fresh fp32 logits ``[B, L, V]`` for one denoising step, with the
    configuration's planted peaks or injected ties."""
    B = cfg.batch if batch is None else batch
    L = cfg.block_len if block_len is None else block_len
    V = cfg.vocab if vocab is None else vocab
    x = _rng(seed, cfg, _T_LOGITS, step).standard_normal((B, L, V), dtype=np.float32)
    x *= np.float32(cfg.logit_std)
    if cfg.plant_peaks:
        r = _rng(seed, cfg, _T_PLANT, step)
        n_plant = L // 2
        for b in range(B):
            pos = r.choice(L, size=n_plant, replace=False)
            ids = r.integers(0, V, size=n_plant)
            for ell, v in zip(pos, ids):
                x[b, ell, v] = x[b, ell].max() + np.float32(8.0)
    if cfg.tie_frac > 0 and V >= 2:
        r = _rng(seed, cfg, _T_TIE, step)
        n_tie = int(round(cfg.tie_frac * B * L))
        flat = r.choice(B * L, size=n_tie, replace=False)
        for f in flat:
            b, ell = divmod(int(f), L)
            row = x[b, ell]
            top = int(np.argmax(row))
            other = int(r.integers(0, V - 1))
            if other >= top:
                other += 1
            row[other] = row[top]
    return x


def initial_mask(cfg: Config, batch: int | None = None, block_len: int | None = None) -> np.ndarray:
    """Mask state at the start of a block: every position is [MASK] (1)."""
    B = cfg.batch if batch is None else batch
    L = cfg.block_len if block_len is None else block_len
    return np.ones((B, L), dtype=np.uint8)


def varlen_inputs(cfg: Config, seed: int = 0, step: int = 0, batch: int | None = None,
                  max_prefix_len: int | None = None, prefix_cap: int | None = None) -> dict:
    """attn_inputs for a batch whose entries have different prefix lengths.

    prefix_lens [B] int32: seeded draws in [0, max_prefix_len] with the two
    extremes (0 and max_prefix_len) always present when B >= 2.  Cache rows
    past each entry's own length hold +-GARBAGE (they must not be read)."""
    B = cfg.batch if batch is None else batch
    Pmax = cfg.prefix_len if max_prefix_len is None else max_prefix_len
    inp = attn_inputs(cfg, seed=seed, step=step, prefix_len=Pmax, prefix_cap=prefix_cap,
                      batch=B)
    r = _rng(seed, cfg, _T_LENS, step)
    lens = r.integers(0, Pmax + 1, size=B).astype(np.int32)
    if B >= 2:
        lens[r.choice(B, size=2, replace=False)] = [0, Pmax]
    g = np.float32(GARBAGE)
    gk, gv = (bf16_bits_from_f32(np.array([g, -g], np.float32)) if cfg.dtype == "bf16"
              else np.array([g, -g], np.float32))
    for b in range(B):
        inp["k_ctx"][b, :, lens[b]:, :] = gk
        inp["v_ctx"][b, :, lens[b]:, :] = gv
    inp["prefix_lens"] = lens
    return inp


def multiblock_inputs(cfg: Config, n_blocks: int, block_size: int, seed: int = 0, step: int = 0,
                      batch: int | None = None) -> dict:
    """Inputs of the training-style pass over all noisy blocks of a sequence:
    q [B,Hq,N*S,D]; k_ctx/v_ctx [B,Hkv,N*S,D] (the context tower over the
    clean sequence; the last block's rows are never visible and hold
    +-GARBAGE); k_noisy/v_noisy [B,Hkv,N*S,D].  Same distributions as
    attn_inputs."""
    B = cfg.batch if batch is None else batch
    T = n_blocks * block_size
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    s = cfg.qkv_std

    def draw(tid, shape):
        return (_rng(seed, cfg, 100 + tid, step).standard_normal(shape, dtype=np.float32)
                * np.float32(s))

    out = dict(q=draw(_T_Q, (B, Hq, T, D)), k_ctx=draw(_T_KCTX, (B, Hkv, T, D)),
               v_ctx=draw(_T_VCTX, (B, Hkv, T, D)), k_noisy=draw(_T_KBLK, (B, Hkv, T, D)),
               v_noisy=draw(_T_VBLK, (B, Hkv, T, D)))
    if n_blocks >= 1:
        out["k_ctx"][:, :, T - block_size:, :] = GARBAGE
        out["v_ctx"][:, :, T - block_size:, :] = -GARBAGE
    if cfg.dtype == "bf16":
        out = {n: bf16_bits_from_f32(a) for n, a in out.items()}
    out.update(n_blocks=n_blocks, block_size=block_size, batch=B, scale=cfg.softmax_scale,
               dtype=cfg.dtype)
    return out


# Hidden width of the synthetic LM head (the pages give none).
LM_D_MODEL = 2688


def lmhead_inputs(cfg: Config, d_model: int = LM_D_MODEL, seed: int = 0, step: int = 0,
                  batch: int | None = None, block_len: int | None = None,
                  vocab: int | None = None, plant_frac: float = 0.25) -> dict:
    """Final hidden states and an LM-head weight for the fused projection +
    unmask step, as bf16 bit patterns.

    hidden [B, L, d] ~ N(0, 1); weight [V, d] ~ N(0, logit_std / sqrt(d)), so
    the logits are about N(0, logit_std).  A seeded fraction of the positions
    (plant_frac) get a hidden state that is a scaled copy of one seeded
    weight row, which makes that id a confident prediction (the same weights
    serve every step).  Returns dict(hidden, weight, d_model, planted)."""
    B = cfg.batch if batch is None else batch
    L = cfg.block_len if block_len is None else block_len
    V = cfg.vocab if vocab is None else vocab
    r_w = _rng(seed, cfg, _T_WEIGHT, 0)
    w = r_w.standard_normal((V, d_model), dtype=np.float32) * np.float32(cfg.logit_std / np.sqrt(d_model))
    h = _rng(seed, cfg, _T_HIDDEN, step).standard_normal((B, L, d_model), dtype=np.float32)
    r = _rng(seed, cfg, _T_HPLANT, step)
    n_plant = int(round(plant_frac * B * L))
    planted = []
    if n_plant > 0:
        flat = r.choice(B * L, size=n_plant, replace=False)
        ids = r.integers(0, V, size=n_plant)
        for f, v in zip(flat, ids):
            b, l = divmod(int(f), L)
            h[b, l] = w[v] * np.float32(1.5 * np.sqrt(d_model) / cfg.logit_std)
            planted.append((b, l, int(v)))
    return dict(hidden=bf16_bits_from_f32(h), weight=bf16_bits_from_f32(w), d_model=d_model,
                planted=planted)
