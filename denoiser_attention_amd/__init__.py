"""TwoTower denoising-step kernels for AMD MI355X (gfx950).

The compute lives in libtt.so (hand-written HIP kernels behind the C ABI of
include/tt.h); this package is its thin Python binding plus the seeded
synthetic-input generator (``synth``).

    block_attn(q, k_ctx, v_ctx, prefix_len, k_blk, v_blk, scale)  -> out
    block_attn_varlen(..., prefix_lens, max_prefix_len, ...)       -> out (per-sequence prefix)
    block_attn_multiblock(q, k_ctx, v_ctx, k_noisy, v_noisy, S, scale) -> out (all noisy blocks)
    unmask_step(logits, mask_state, k, tokens)                     -> (tokens, mask_out)
    unmask_step_noalloc(logits, mask_state, k, tokens)             -> (tokens, mask_out) (no workspace)
    unmask_step_ex(logits, mask_state, select_rule(...), tokens)   -> (tokens, mask_out)
    lmhead_unmask_step(hidden, weight, mask_state, select, tokens) -> (tokens, mask_out)
"""
from ._binding import (  # noqa: F401
    LIB_PATH, SELECT_MODES, Prepared, Select, TTError, attn_multiblock_workspace_bytes,
    attn_workspace_bytes, block_attn, block_attn_multiblock, block_attn_varlen, lib,
    lmhead_unmask_step, lmhead_unmask_workspace_bytes, prepare_block_attn,
    prepare_block_attn_multiblock, prepare_block_attn_varlen, prepare_lmhead_unmask_step,
    prepare_unmask_commit, prepare_unmask_commit_ex, prepare_unmask_reduce, select_rule,
    status_string, unmask_commit, unmask_commit_ex, unmask_reduce, unmask_step, unmask_step_ex,
    unmask_step_noalloc, unmask_workspace_bytes, version,
)

__all__ = [
    "LIB_PATH", "SELECT_MODES", "Prepared", "Select", "TTError", "attn_multiblock_workspace_bytes",
    "attn_workspace_bytes", "block_attn", "block_attn_multiblock", "block_attn_varlen", "lib",
    "lmhead_unmask_step", "lmhead_unmask_workspace_bytes", "prepare_block_attn",
    "prepare_block_attn_multiblock", "prepare_block_attn_varlen", "prepare_lmhead_unmask_step",
    "prepare_unmask_commit", "prepare_unmask_commit_ex", "prepare_unmask_reduce", "select_rule",
    "status_string", "unmask_commit", "unmask_commit_ex", "unmask_reduce", "unmask_step",
    "unmask_step_ex", "unmask_step_noalloc", "unmask_workspace_bytes", "version",
]
