"""Pins of the per-sequence-prefix and multi-block attention oracles: the
library SDPA (float64, CPU) with masks built here from the visibility rule,
reduction to the pinned single-block oracle, and the invariance of each
output to every key row it must not see."""
import numpy as np
import pytest
import torch

import oracle


def _sdpa(q, k, v, scale, mask):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(np.ascontiguousarray(mask)),
        is_causal=False, scale=scale, enable_gqa=True).numpy()


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_varlen_matches_library_per_entry():
    rng = np.random.default_rng(40)
    B, Hq, Hkv, L, Pcap, D = 4, 6, 2, 5, 19, 8
    lens = [0, 7, 19, 1]
    q, kb, vb = _rand(rng, B, Hq, L, D), _rand(rng, B, Hkv, L, D), _rand(rng, B, Hkv, L, D)
    kc, vc = _rand(rng, B, Hkv, Pcap, D), _rand(rng, B, Hkv, Pcap, D)
    for b, p in enumerate(lens):          # garbage past each entry's length
        kc[b, :, p:] = 40.0
        vc[b, :, p:] = -40.0
    out, lse = oracle.block_attn_varlen(q, kc, vc, lens, kb, vb, 0.3)
    for b, p in enumerate(lens):
        k = np.concatenate([kc[b:b + 1, :, :p], kb[b:b + 1]], axis=2)
        v = np.concatenate([vc[b:b + 1, :, :p], vb[b:b + 1]], axis=2)
        ref = _sdpa(q[b:b + 1], k, v, 0.3, np.ones((L, p + L), dtype=bool))
        assert np.max(np.abs(out[b:b + 1] - ref)) <= 1e-12
    assert lse.shape == (B, Hq, L) and np.isfinite(lse).all()


def test_varlen_equal_lengths_is_block_attn():
    rng = np.random.default_rng(41)
    B, Hq, Hkv, L, P, D = 3, 4, 4, 6, 9, 16
    q, kb, vb = _rand(rng, B, Hq, L, D), _rand(rng, B, Hkv, L, D), _rand(rng, B, Hkv, L, D)
    kc, vc = _rand(rng, B, Hkv, P + 3, D), _rand(rng, B, Hkv, P + 3, D)
    a, la = oracle.block_attn_varlen(q, kc, vc, [P] * B, kb, vb, 0.25)
    b, lb = oracle.block_attn(q, kc, vc, P, kb, vb, 0.25)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    with pytest.raises(ValueError):
        oracle.block_attn_varlen(q, kc, vc, [P] * (B - 1), kb, vb, 0.25)


def _mb_inputs(rng, B, Hq, Hkv, N, S, D, extra_ctx=0):
    T = N * S
    return (_rand(rng, B, Hq, T, D), _rand(rng, B, Hkv, T + extra_ctx, D),
            _rand(rng, B, Hkv, T + extra_ctx, D), _rand(rng, B, Hkv, T, D), _rand(rng, B, Hkv, T, D))


@pytest.mark.parametrize("N,S", [(1, 5), (3, 4), (4, 16)])
def test_multiblock_matches_library_with_mask(N, S):
    rng = np.random.default_rng(42 + N)
    B, Hq, Hkv, D = 2, 4, 2, 8
    q, kc, vc, kn, vn = _mb_inputs(rng, B, Hq, Hkv, N, S, D, extra_ctx=3)
    out, _ = oracle.block_attn_multiblock(q, kc, vc, kn, vn, S, 0.35)
    T, Tc = N * S, kc.shape[2]
    mask = np.zeros((T, Tc + T), dtype=bool)
    for t in range(T):                      # the visibility rule, one entry at a time
        j = t // S
        for c in range(Tc):
            mask[t, c] = c < j * S
        for r in range(T):
            mask[t, Tc + r] = j * S <= r < (j + 1) * S
    ref = _sdpa(q, np.concatenate([kc, kn], 2), np.concatenate([vc, vn], 2), 0.35, mask)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_multiblock_block_j_is_single_block_with_prefix():
    rng = np.random.default_rng(43)
    B, Hq, Hkv, N, S, D = 2, 6, 3, 4, 8, 16
    q, kc, vc, kn, vn = _mb_inputs(rng, B, Hq, Hkv, N, S, D)
    out, lse = oracle.block_attn_multiblock(q, kc, vc, kn, vn, S, 0.2)
    for j in range(N):
        sl = slice(j * S, (j + 1) * S)
        o, s = oracle.block_attn(q[:, :, sl], kc, vc, j * S, kn[:, :, sl], vn[:, :, sl], 0.2)
        assert np.max(np.abs(out[:, :, sl] - o)) <= 1e-12
        assert np.max(np.abs(lse[:, :, sl] - s)) <= 1e-12


def test_multiblock_ignores_invisible_rows():
    rng = np.random.default_rng(44)
    B, Hq, Hkv, N, S, D = 1, 2, 1, 4, 6, 8
    q, kc, vc, kn, vn = _mb_inputs(rng, B, Hq, Hkv, N, S, D, extra_ctx=2)
    base, _ = oracle.block_attn_multiblock(q, kc, vc, kn, vn, S, 0.5)
    j = 2
    sl = slice(j * S, (j + 1) * S)
    kc2, vc2, kn2, vn2 = kc.copy(), vc.copy(), kn.copy(), vn.copy()
    kc2[:, :, j * S:] += 30.0              # clean rows from block j on
    vc2[:, :, j * S:] -= 30.0
    kn2[:, :, :j * S] += 30.0              # other noisy blocks
    kn2[:, :, (j + 1) * S:] += 30.0
    vn2[:, :, :j * S] -= 30.0
    vn2[:, :, (j + 1) * S:] -= 30.0
    out2, _ = oracle.block_attn_multiblock(q, kc2, vc2, kn2, vn2, S, 0.5)
    assert np.array_equal(out2[:, :, sl], base[:, :, sl])
    # a visible row does matter: the clean row just before block j, and block j's own row
    for arr, row in ((kc, j * S - 1), (kn, j * S)):
        pert = arr.copy()
        pert[:, :, row] += 3.0
        args = [q, kc, vc, kn, vn]
        args[1 if arr is kc else 3] = pert
        o, _ = oracle.block_attn_multiblock(*args, S, 0.5)
        assert np.max(np.abs(o[:, :, sl] - base[:, :, sl])) > 1e-6


def test_multiblock_rejects_ragged_and_short_context():
    rng = np.random.default_rng(45)
    q, kc, vc, kn, vn = _mb_inputs(rng, 1, 2, 1, 3, 4, 8)
    with pytest.raises(ValueError):
        oracle.block_attn_multiblock(q[:, :, :11], kc, vc, kn[:, :, :11], vn[:, :, :11], 4, 0.5)
    with pytest.raises(ValueError):
        oracle.block_attn_multiblock(q, kc[:, :, :7], vc[:, :, :7], kn, vn, 4, 0.5)
