"""The seeded input generator: determinism, bf16 rounding, and the planted
structure (peaks, ties, outlier channels, cache padding) the workloads ask for."""
import numpy as np
import torch

from denoiser_attention_amd import synth


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3e-39,
                                  -1.0009765625], dtype=np.float32)])
    ours = synth.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.f32_from_bf16_bits(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy())


def test_attn_inputs_deterministic_and_shaped():
    cfg = synth.get_config("decode_b8_p2048_l32")
    a = synth.attn_inputs(cfg, seed=0, step=1, batch=2, prefix_len=100)
    b = synth.attn_inputs(cfg, seed=0, step=1, batch=2, prefix_len=100)
    c = synth.attn_inputs(cfg, seed=0, step=2, batch=2, prefix_len=100)
    for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk"):
        assert a[n].dtype == np.uint16
        assert np.array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])
    assert a["q"].shape == (2, 32, 32, 128)
    assert a["k_ctx"].shape == (2, 2, 100, 128)


def test_cache_padding_is_garbage():
    cfg = synth.get_config("tiny_fp32")
    a = synth.attn_inputs(cfg, prefix_len=10, prefix_cap=16)
    assert np.all(np.abs(a["k_ctx"][:, :, 10:]) == synth.GARBAGE)
    assert np.all(np.abs(a["k_ctx"][:, :, :10]) < 10)


def test_outlier_channels():
    cfg = synth.get_config("highbatch_b64_p4096_l64")
    a = synth.attn_inputs(cfg, batch=2, prefix_len=256)
    assert len(a["outliers"]) == round(0.01 * 2 * 128) == 3
    k = synth.f32_from_bf16_bits(a["k_ctx"])
    for (h, c) in a["outliers"]:
        assert np.std(k[:, h, :, c]) > 5.0
    mask = np.ones((2, 128), bool)
    for (h, c) in a["outliers"]:
        mask[h, c] = False
    assert np.std(k.transpose(1, 3, 0, 2)[mask]) < 1.5


def test_planted_peaks_unique_argmax():
    cfg = synth.get_config("decode_b8_p2048_l32")
    x = synth.logits(cfg, batch=2, vocab=4096)
    top2 = np.sort(x, axis=-1)[..., -2:]
    planted = (top2[..., 1] - top2[..., 0]) >= 7.99  # fp32 rounding of max + 8
    assert np.all(planted.sum(axis=1) >= cfg.block_len // 2)


def test_injected_ties():
    cfg = synth.get_config("highbatch_b64_p4096_l64")
    x = synth.logits(cfg, batch=4, vocab=2048)
    mx = x.max(-1, keepdims=True)
    n_max = (x == mx).sum(-1)
    assert (n_max >= 2).sum() == round(0.05 * 4 * 64)


def test_varlen_inputs_lengths_and_garbage():
    cfg = synth.get_config("decode_b8_p2048_l32")
    a = synth.varlen_inputs(cfg, seed=3, batch=6, max_prefix_len=90, prefix_cap=96)
    b = synth.varlen_inputs(cfg, seed=3, batch=6, max_prefix_len=90, prefix_cap=96)
    lens = a["prefix_lens"]
    assert np.array_equal(lens, b["prefix_lens"]) and lens.dtype == np.int32
    assert lens.min() == 0 and lens.max() == 90 and np.all((lens >= 0) & (lens <= 90))
    for bi, p in enumerate(lens):
        kc = synth.f32_from_bf16_bits(a["k_ctx"][bi])
        assert np.all(np.abs(kc[:, p:]) > 0.99 * synth.GARBAGE)   # bf16-rounded
        assert np.all(np.abs(kc[:, :p]) < 100)


def test_multiblock_inputs_shapes_and_hidden_rows():
    cfg = synth.get_config("decode_b8_p2048_l32")
    m = synth.multiblock_inputs(cfg, n_blocks=3, block_size=16, seed=1, batch=2)
    assert m["q"].shape == (2, 32, 48, 128) and m["k_noisy"].shape == (2, 2, 48, 128)
    kc = synth.f32_from_bf16_bits(m["k_ctx"])
    assert np.all(np.abs(kc[:, :, 32:]) > 0.99 * synth.GARBAGE) and np.all(np.abs(kc[:, :, :32]) < 100)
    m2 = synth.multiblock_inputs(cfg, n_blocks=3, block_size=16, seed=1, batch=2)
    assert all(np.array_equal(m[k], m2[k]) for k in ("q", "k_ctx", "v_noisy"))
