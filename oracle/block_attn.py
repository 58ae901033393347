"""Oracle for the denoiser's block attention (test infrastructure only).

Definition followed: TwoTower paper §2.1 "Bidirectional Attention", Eq. (1).
At denoiser layer i the queries of the noisy block b attend over ONE key/value
sequence that is the concatenation, along the sequence axis, of the context
tower's layer-i K/V for the clean prefix (blocks 0..b-1) and the denoiser's own
layer-i K/V for block b.  Inside the block the causal mask is relaxed: every
block query sees every block key; towards the past it sees every prefix key.
So with the visible set {prefix rows 0..P-1} U {block rows 0..L-1}, the
output is the plain softmax attention over that set, one softmax per query row.

Readings where the pages are silent (each listed in the design notes):
* "[A; B]" is concatenation along the sequence axis.
* Grouped-query attention: query head h reads KV head floor(h / G) with
  G = Hq / Hkv (contiguous groups).  The pages give no head counts.
* The kernel is position-free: any rotary embedding is already applied to Q/K.
* No sliding window, sinks, soft-capping, dropout or bias.
* The context cache may have capacity Pcap >= P rows; rows P..Pcap-1 are
  not visible (explicit mask below).

Method: upcast to float64, build the full key axis [cache rows 0..Pcap-1 ;
block rows 0..L-1], an explicit 0/1 visibility mask, the full score matrix,
a row softmax (subtract row max, exponentiate, sum, divide) and the
weighted sum of value rows.  A loop over (batch, query head) bounds memory.
"""
from __future__ import annotations

import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values, exactly (a bf16 value is
    the upper 16 bits of an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def block_attn(q, k_ctx, v_ctx, prefix_len, k_blk, v_blk, scale, *,
               return_weights: bool = False):
    """Eq. (1) attention of the block queries over [prefix cache ; block].

    Arguments (float arrays; bf16 inputs must be decoded with
    ``decode_bf16`` first):
      q      [B, Hq, L, D]   block queries
      k_ctx  [B, Hkv, Pcap, D], v_ctx same: context-tower layer-i cache,
             rows 0..prefix_len-1 valid
      k_blk  [B, Hkv, L, D], v_blk same: denoiser's own layer-i block K/V
      scale  softmax temperature multiplier on q.k

    Returns (out [B,Hq,L,D], lse [B,Hq,L]) in float64, and additionally the
    weights [B,Hq,L,Pcap+L] (zero at invisible keys) if ``return_weights``.
    """
    q = np.asarray(q, dtype=np.float64)
    k_ctx = np.asarray(k_ctx, dtype=np.float64)
    v_ctx = np.asarray(v_ctx, dtype=np.float64)
    k_blk = np.asarray(k_blk, dtype=np.float64)
    v_blk = np.asarray(v_blk, dtype=np.float64)
    B, Hq, L, D = q.shape
    Hkv, Pcap = k_ctx.shape[1], k_ctx.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if not (0 <= prefix_len <= Pcap):
        raise ValueError("prefix_len out of range")
    if k_blk.shape != (B, Hkv, L, D) or v_blk.shape != (B, Hkv, L, D):
        raise ValueError("block K/V shape mismatch")
    if k_ctx.shape != (B, Hkv, Pcap, D) or v_ctx.shape != (B, Hkv, Pcap, D):
        raise ValueError("cache K/V shape mismatch")
    G = Hq // Hkv
    n_keys = Pcap + L
    # Explicit visibility: prefix rows 0..P-1 and every block row.
    visible = np.zeros(n_keys, dtype=bool)
    visible[:prefix_len] = True
    visible[Pcap:] = True
    if not (np.isfinite(q).all() and np.isfinite(k_blk).all() and np.isfinite(v_blk).all()
            and np.isfinite(k_ctx[:, :, :prefix_len]).all()
            and np.isfinite(v_ctx[:, :, :prefix_len]).all()):
        raise ValueError("non-finite attention input")

    out = np.empty((B, Hq, L, D), dtype=np.float64)
    lse = np.empty((B, Hq, L), dtype=np.float64)
    weights = np.zeros((B, Hq, L, n_keys), dtype=np.float64) if return_weights else None
    for b in range(B):
        for h in range(Hq):
            g = h // G
            K = np.concatenate([k_ctx[b, g], k_blk[b, g]], axis=0)   # [n_keys, D]
            V = np.concatenate([v_ctx[b, g], v_blk[b, g]], axis=0)
            S = scale * (q[b, h] @ K.T)                                 # [L, n_keys]
            S = np.where(visible[None, :], S, -np.inf)
            row_max = S.max(axis=1, keepdims=True)
            E = np.exp(S - row_max)                                     # 0 where invisible
            den = E.sum(axis=1, keepdims=True)
            W = E / den
            # Invisible rows carry zero weight; they are excluded from the
            # product so that garbage there cannot leak in.
            out[b, h] = W[:, visible] @ V[visible]
            lse[b, h] = row_max[:, 0] + np.log(den[:, 0])
            if return_weights:
                weights[b, h] = W
    if return_weights:
        return out, lse, weights
    return out, lse


def block_attn_varlen(q, k_ctx, v_ctx, prefix_lens, k_blk, v_blk, scale):
    """Eq. (1) where every batch entry b has its own prefix length P_b (a batch
    of sequences generated to different lengths).  Entry b sees cache rows
    0..P_b-1 and all of its block rows; everything else is as in block_attn,
    which is applied to each entry on its own.

    prefix_lens: [B] integers, 0 <= P_b <= Pcap.  Returns (out, lse)."""
    q = np.asarray(q, dtype=np.float64)
    B = q.shape[0]
    lens = [int(p) for p in np.asarray(prefix_lens).reshape(-1)]
    if len(lens) != B:
        raise ValueError("one prefix length per batch entry")
    outs, lses = [], []
    for b in range(B):
        o, s = block_attn(q[b:b + 1], k_ctx[b:b + 1], v_ctx[b:b + 1], lens[b], k_blk[b:b + 1],
                          v_blk[b:b + 1], scale)
        outs.append(o)
        lses.append(s)
    return np.concatenate(outs, axis=0), np.concatenate(lses, axis=0)


def block_attn_multiblock(q, k_ctx, v_ctx, k_noisy, v_noisy, block_size, scale):
    """The denoiser's training-style pass over all noisy blocks of a sequence
    at once (TwoTower paper §2.3 "Training", Implementation paragraph; the
    visibility of §2.1 Eq. (1) applied to every block): with blocks of S =
    block_size rows, query row t of block j = t // S sees the clean context
    tower's rows 0..j*S-1 (the clean blocks before j) and the noisy rows
    j*S..(j+1)*S-1 of its own block (bidirectionally); nothing else.

      q        [B, Hq, N*S, D]   noisy queries, N blocks
      k_ctx    [B, Hkv, Tc, D]   context tower K of the clean sequence, Tc >= (N-1)*S
      v_ctx    same
      k_noisy  [B, Hkv, N*S, D]  denoiser K of the noisy blocks
      v_noisy  same

    Method: one key axis [context rows 0..Tc-1 ; noisy rows 0..N*S-1], an
    explicit per-row visibility mask, the full score matrix, a row softmax
    and the weighted sum of values, per (batch, query head).  Returns
    (out [B,Hq,N*S,D], lse [B,Hq,N*S])."""
    q = np.asarray(q, dtype=np.float64)
    k_ctx = np.asarray(k_ctx, dtype=np.float64)
    v_ctx = np.asarray(v_ctx, dtype=np.float64)
    k_noisy = np.asarray(k_noisy, dtype=np.float64)
    v_noisy = np.asarray(v_noisy, dtype=np.float64)
    B, Hq, T, D = q.shape
    Hkv, Tc = k_ctx.shape[1], k_ctx.shape[2]
    S = int(block_size)
    if S < 1 or T % S != 0:
        raise ValueError("the query length must be a whole number of blocks")
    N = T // S
    if Hq % Hkv != 0 or Tc < (N - 1) * S:
        raise ValueError("head counts or context length do not fit")
    if k_noisy.shape != (B, Hkv, T, D) or v_noisy.shape != (B, Hkv, T, D):
        raise ValueError("noisy K/V shape mismatch")
    G = Hq // Hkv
    blk = np.arange(T) // S                                      # block of each query / noisy row
    visible = np.zeros((T, Tc + T), dtype=bool)
    visible[:, :Tc] = np.arange(Tc)[None, :] < (blk * S)[:, None]   # clean rows before the block
    visible[:, Tc:] = blk[None, :] == blk[:, None]                  # own noisy block
    out = np.empty((B, Hq, T, D), dtype=np.float64)
    lse = np.empty((B, Hq, T), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            K = np.concatenate([k_ctx[b, g], k_noisy[b, g]], axis=0)
            V = np.concatenate([v_ctx[b, g], v_noisy[b, g]], axis=0)
            Sc = np.where(visible, scale * (q[b, h] @ K.T), -np.inf)
            row_max = Sc.max(axis=1, keepdims=True)
            E = np.exp(Sc - row_max)
            den = E.sum(axis=1, keepdims=True)
            W = E / den
            out[b, h] = np.where(visible, W, 0.0) @ np.where(visible.any(axis=0)[:, None], V, 0.0)
            lse[b, h] = row_max[:, 0] + np.log(den[:, 0])
    return out, lse
