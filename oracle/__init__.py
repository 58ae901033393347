"""CPU oracle for the TwoTower denoising step -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct definition of what the
HIP library computes, in float64 numpy.  Only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import it.  The product path
(``denoiser_attention_amd``) never imports, calls or links anything here, and
nothing here imports the product path: the two share no code.  The seeded
input generator (``denoiser_attention_amd.synth``) is the only thing both
sides consume, and it holds no arithmetic of the method.

Source of the definitions.  "TwoTower paper" below means *Nemotron-Labs-
TwoTower: Diffusion Language Modeling with Pretrained Autoregressive Context*
(Kamalu et al.), as quoted on the bittide.aicompass.dev article page; its
equations and algorithms are garbled by text extraction, and the readings
taken are stated next to each function.

* ``block_attn``   -- TwoTower paper §2.1 "Bidirectional Attention", Eq. (1).
* ``block_attn_varlen`` -- Eq. (1) with a prefix length per batch entry.
* ``block_attn_multiblock`` -- the training-style pass over all noisy blocks
  of a sequence (§2.3 "Training", Implementation paragraph).
* ``vocab_stats``  -- TwoTower paper §2.2 "Sampling" (confidence of the
  prediction at each masked position) and Algorithm 2 (the denoiser's
  distribution p_theta).
* ``unmask_step``  -- TwoTower paper §2.2 "Sampling" and Algorithm 2
  (ConfidenceSample), in its fixed-k reading (threshold switched off).
* ``lmhead_unmask_step`` -- the unmask step fed by the LM-head projection of
  the masked positions' hidden states (logits = hidden . W^T), §2.2
  "Sampling" / Algorithm 2 (p_theta of DenoiserTower).
* ``unmask_step_select`` -- the same step under the other selection rules of
  §2.2 "Sampling": Algorithm 2's threshold gamma with its T-r+1 deadline, the
  predict-and-noise sampler with the linear schedule alpha_t = 1 - t, and the
  one-token-per-step mock-autoregressive mode of the article's "Three
  Generation Modes" list.

Pins: every function here is checked by the ``-m "not gpu"`` tests against
brute force in 50-digit arithmetic, closed forms, invariants and library
routines (tests/test_oracle_*.py).  No function is "parity unpinned".
"""
from .block_attn import block_attn, block_attn_multiblock, block_attn_varlen, decode_bf16
from .lmhead import lmhead_logits, lmhead_unmask_step
from .unmask import (LEFTMOST, SCHEDULE, THRESHOLD, TOP_K, commit_count, select_step, topk_select,
                     unmask_step, unmask_step_select, vocab_stats)

__all__ = ["block_attn", "block_attn_varlen", "block_attn_multiblock", "decode_bf16", "vocab_stats", "unmask_step", "topk_select",
           "unmask_step_select", "select_step", "commit_count", "TOP_K", "THRESHOLD", "SCHEDULE",
           "LEFTMOST", "lmhead_logits", "lmhead_unmask_step"]
