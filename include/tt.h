/*
 * tt.h -- C ABI of libtt, the TwoTower denoising-step kernels for AMD MI355X (gfx950).
 *
 * One denoising step of the denoiser tower over a block of masked tokens has two
 * GPU operations, both defined by the TwoTower paper ("Nemotron-Labs-TwoTower:
 * Diffusion Language Modeling with Pretrained Autoregressive Context", quoted on
 * the bittide.aicompass.dev article page):
 *
 *   tt_block_attn   -- Eq. (1) of §2.1 "Bidirectional Attention": the block's
 *                      queries attend, under one softmax, to the context tower's
 *                      layer-aligned KV cache of the clean prefix and, with no
 *                      causal mask, to every position of their own block.
 *   tt_unmask_step  -- §2.2 "Sampling" / Algorithm 2 (ConfidenceSample): predict
 *                      every still-masked position, commit the most confident ones.
 *                      Implemented in its fixed-k form (k positions per sequence
 *                      and step, the sampler's deadline floor with the confidence
 *                      threshold switched off).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays on the
 *     current HIP device.  The caller owns every buffer; the library never
 *     allocates or frees memory and keeps no state between calls.
 *   - Calls only ENQUEUE work on `stream` (0 = the null stream) and return at
 *     once.  Results are valid after the caller synchronises the stream.
 *   - Arguments are validated on the host before anything is enqueued; a bad
 *     argument returns TT_EINVAL and enqueues nothing.  A combination the
 *     compiled kernels do not cover returns TT_EUNSUPPORTED.  No visible HIP
 *     device returns TT_ENODEV.  A failed launch returns TT_EHIP.  Faults inside
 *     a kernel surface at the caller's stream synchronisation.
 *   - The attention and LM-head entry points move tiles with 16-byte loads and
 *     stores from each tensor's base: q, k_ctx, v_ctx, k_blk, v_blk, out,
 *     hidden, weight and any workspace must be 16-byte aligned (prefix_lens
 *     4-byte aligned), else TT_EINVAL.  A contiguous torch tensor that starts
 *     its own allocation is always aligned; a view at an odd element offset
 *     may not be.  The unmask entry points accept logits at any 4-byte
 *     alignment.
 *   - Workspaces are caller-provided device memory of at least the size the
 *     matching *_workspace_bytes query returns (NULL is allowed when it returns
 *     0).  Two calls that run concurrently must not share a workspace.
 *   - No C++ exception crosses this interface.
 */
#ifndef TT_H_
#define TT_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TT_OK = 0,
  TT_EINVAL = 1,        /* invalid argument (null pointer, bad size, short workspace) */
  TT_EUNSUPPORTED = 2,  /* valid, but not covered by the compiled kernels */
  TT_ENODEV = 3,        /* no HIP device visible */
  TT_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} tt_status;

typedef enum { TT_FP32 = 0, TT_BF16 = 1 } tt_dtype;

/* Attention kernel family.  AUTO picks MFMA for bf16 inputs with a head_dim of
 * 64 or 128, at every number of packed query rows per KV head (measured faster
 * than the wavefront-shuffle kernel from 1 to 32 such rows), and the
 * wavefront-shuffle kernel for fp32 inputs and head_dim 256.  Either family
 * can be forced through tt_attn_opts. */
typedef enum { TT_ATTN_AUTO = 0, TT_ATTN_MFMA = 1, TT_ATTN_SHUFFLE = 2 } tt_attn_path;

/* Optional tuning knobs of tt_block_attn_ex.  kv_splits = 0 lets the library
 * choose how many workgroups share one query tile's key range; a positive value
 * forces that many (clamped so that no split is empty; partial results are then
 * merged in a second pass).  kv_groups (MFMA kernel only) = 0 lets the library
 * choose, 1 or 2 forces how many wave groups inside one workgroup divide that
 * workgroup's key range between them (merged on chip).  rows_per_wave (MFMA
 * kernel only) = 0 lets the library choose, 32 or 64 forces how many query rows
 * one wavefront owns; 64 needs head_dim 128 and one wave group (otherwise
 * TT_EUNSUPPORTED).  stream_waves (MFMA kernel only) = 0 lets the library
 * choose, 4 or 8 forces how many wavefronts of a workgroup share one stream of
 * K/V tiles through LDS (8: 256 query rows per workgroup, half the tile loads
 * per unit of work; needs head_dim 128, one wave group and 32-row waves,
 * otherwise TT_EUNSUPPORTED).  Values outside these sets give TT_EINVAL. */
typedef struct {
  int path;           /* tt_attn_path */
  int kv_splits;      /* 0 = auto */
  int kv_groups;      /* 0 = auto, 1 or 2 */
  int rows_per_wave;  /* 0 = auto, 32 or 64 */
  int stream_waves;   /* 0 = auto, 4 or 8 */
} tt_attn_opts;

/* Human-readable name of a status code (static storage, never NULL). */
const char* tt_status_string(tt_status status);

/* Library version, e.g. "0.1.0" (static storage). */
const char* tt_version(void);

/* ------------------------------------------------------------------------ */
/* Block attention: TwoTower paper §2.1, Eq. (1).                            */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace tt_block_attn / tt_block_attn_ex need for this shape and
 * these options (opts may be NULL = defaults).  Returns 0 when no workspace is
 * needed, and SIZE_MAX when the arguments are invalid.
 * Additions to the query the path's definition names (batch and the shape):
 * dtype, because the kernel family and its split plan depend on it, and opts,
 * the tuning knobs of tt_block_attn_ex (NULL for tt_block_attn). */
size_t tt_block_attn_workspace_bytes(int batch, int prefix_len, int block_len, int n_q_heads,
                                     int n_kv_heads, int head_dim, tt_dtype dtype,
                                     const tt_attn_opts* opts);

/* out = softmax(scale * Q Kᵀ) V over the key sequence [cache rows 0..P-1 ; block
 * rows 0..L-1], for every batch entry b and query head h, where query head h
 * reads KV head h / (n_q_heads / n_kv_heads).  Every block query sees every
 * prefix row and every block row (bidirectional inside the block); cache rows
 * P..prefix_cap-1 are never read.
 *
 *   q      [batch, n_q_heads, block_len, head_dim]          dtype
 *   k_ctx  [batch, n_kv_heads, prefix_cap, head_dim]        dtype  context-tower layer-i K
 *   v_ctx  [batch, n_kv_heads, prefix_cap, head_dim]        dtype  context-tower layer-i V
 *          (both may be NULL when prefix_cap == 0)
 *   prefix_len  P >= 0 valid cache rows (0 = plain bidirectional block attention)
 *   k_blk  [batch, n_kv_heads, block_len, head_dim]         dtype  denoiser's own layer-i K
 *   v_blk  [batch, n_kv_heads, block_len, head_dim]         dtype  denoiser's own layer-i V
 *   block_len   L >= 0 (L == 0 or batch == 0: nothing to do, TT_OK)
 *   n_q_heads, n_kv_heads  >= 1, n_q_heads a multiple of n_kv_heads
 *   head_dim    D: 64, 128 or 256 (the MFMA kernel covers 64 and 128)
 *   scale       finite multiplier of q.k (typically 1/sqrt(D)); |scale| * log2(e)
 *               must be finite too (|scale| < 2.3e38), else TT_EINVAL
 *   out    [batch, n_q_heads, block_len, head_dim]          out_dtype; must not
 *          alias any input
 *   batch       B >= 0
 *   prefix_cap  allocated cache rows per (b, kv head), >= prefix_len
 *   dtype       TT_FP32 or TT_BF16 for q/k/v (fp32 accumulation either way)
 *   out_dtype   dtype, or TT_FP32 for bf16 inputs
 *   workspace, workspace_bytes  see tt_block_attn_workspace_bytes (opts NULL)
 *   stream      HIP stream the kernels are enqueued on (0 = null stream)
 * Inputs are read only.  The call is deterministic: the same inputs give the
 * same output bits.
 * Arguments beyond the path's named signature (q, k_ctx, v_ctx, prefix_len,
 * k_blk, v_blk, block_len, n_q_heads, n_kv_heads, head_dim, scale, out), all
 * after it so that its order is kept: batch (the named form is per sequence);
 * prefix_cap (the cache's capacity stride: a growing cache is allocated once);
 * dtype and out_dtype (bf16 or fp32 inputs; fp32 output for bf16 inputs);
 * workspace and workspace_bytes (key-split partials: the library never
 * allocates); stream. */
tt_status tt_block_attn(const void* q, const void* k_ctx, const void* v_ctx, int prefix_len,
                        const void* k_blk, const void* v_blk, int block_len, int n_q_heads,
                        int n_kv_heads, int head_dim, float scale, void* out, int batch,
                        int prefix_cap, tt_dtype dtype, tt_dtype out_dtype, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* tt_block_attn with explicit kernel-family / split options (opts may be NULL). */
tt_status tt_block_attn_ex(const void* q, const void* k_ctx, const void* v_ctx, int prefix_len,
                           const void* k_blk, const void* v_blk, int block_len, int n_q_heads,
                           int n_kv_heads, int head_dim, float scale, void* out, int batch,
                           int prefix_cap, tt_dtype dtype, tt_dtype out_dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream, const tt_attn_opts* opts);

/* tt_block_attn_ex where every batch entry b has its own prefix length
 * prefix_lens[b] (a batch of sequences generated to different lengths): entry
 * b's queries see cache rows 0..prefix_lens[b]-1 and all of its block rows.
 *   prefix_lens     DEVICE int32 [batch]; each value in [0, max_prefix_len]
 *                   (values outside are clamped into that range)
 *   max_prefix_len  bound on prefix_lens (work is planned for it), <= prefix_cap
 * Workspace: tt_block_attn_workspace_bytes with prefix_len = max_prefix_len.
 * All other arguments are those of tt_block_attn_ex. */
tt_status tt_block_attn_varlen(const void* q, const void* k_ctx, const void* v_ctx,
                               const int32_t* prefix_lens, int max_prefix_len, const void* k_blk,
                               const void* v_blk, int block_len, int n_q_heads, int n_kv_heads,
                               int head_dim, float scale, void* out, int batch, int prefix_cap,
                               tt_dtype dtype, tt_dtype out_dtype, void* workspace,
                               size_t workspace_bytes, hipStream_t stream,
                               const tt_attn_opts* opts);

/* The denoiser's training-style pass over all noisy blocks of a sequence at
 * once (TwoTower paper §2.3 "Training", Implementation paragraph, with the
 * visibility of Eq. (1) for every block): the sequence is n_blocks blocks of
 * S = block_size rows; query row t of block j = t / S attends, under one
 * softmax, to the context tower's rows 0..j*S-1 (the clean blocks before j)
 * and to the noisy rows j*S..(j+1)*S-1 of its own block, bidirectionally.
 *   q        [batch, n_q_heads, n_blocks*S, head_dim]   dtype
 *   k_ctx    [batch, n_kv_heads, ctx_cap, head_dim]     context tower K of the
 *            clean sequence; ctx_cap >= (n_blocks-1)*S
 *   v_ctx    same                                        (both may be NULL if ctx_cap == 0)
 *   k_noisy  [batch, n_kv_heads, n_blocks*S, head_dim]  denoiser K of the noisy blocks
 *   v_noisy  same
 *   out      [batch, n_q_heads, n_blocks*S, head_dim]   out_dtype
 * Workspace: tt_block_attn_multiblock_workspace_bytes.  Kernel family,
 * options, dtypes and errors as for tt_block_attn_ex; block_size plays the
 * role of block_len. */
size_t tt_block_attn_multiblock_workspace_bytes(int batch, int block_size, int n_blocks,
                                                int n_q_heads, int n_kv_heads, int head_dim,
                                                tt_dtype dtype, const tt_attn_opts* opts);
tt_status tt_block_attn_multiblock(const void* q, const void* k_ctx, const void* v_ctx,
                                   const void* k_noisy, const void* v_noisy, int block_size,
                                   int n_blocks, int n_q_heads, int n_kv_heads, int head_dim,
                                   float scale, void* out, int batch, int ctx_cap, tt_dtype dtype,
                                   tt_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream, const tt_attn_opts* opts);

/* ------------------------------------------------------------------------ */
/* Confidence unmask: TwoTower paper §2.2 "Sampling", Algorithm 2.           */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace tt_unmask_step needs (SIZE_MAX for invalid sizes). */
size_t tt_unmask_workspace_bytes(int batch, int block_len, int vocab);

/* One fixed-k confidence-unmasking step over `batch` blocks of `block_len`
 * positions.  For every position with mask_state != 0 (still [MASK]):
 *   pred = argmax_v logits[b,l,v]           (lowest id among equal maxima)
 *   conf = 1 / sum_v exp(logits[b,l,v] - max_v logits[b,l,v])
 *        = the largest probability of softmax(logits[b,l,:]).
 * Then per sequence b, the min(k, n_masked(b)) masked positions first in the
 * order (conf descending, position ascending) are committed:
 *   tokens_out[b,l] = pred,  mask_out[b,l] = 0.
 * Every other position keeps its token (tokens_out is not written there) and
 * gets mask_out[b,l] = (mask_state[b,l] != 0).  Logit rows of positions that
 * are not masked are never read.
 *
 *   logits      [batch, block_len, vocab]  fp32, finite (NaN/Inf: undefined result)
 *   mask_state  [batch, block_len]  uint8, nonzero = still [MASK]
 *   k           >= 0 positions to commit per sequence (0 = no-op)
 *   tokens_out  [batch, block_len]  int32, in/out
 *   mask_out    [batch, block_len]  uint8, may alias mask_state
 *   batch, block_len >= 0 (0: nothing to do), block_len <= 1024; vocab >= 1
 *   conf_out    optional [batch, block_len] fp32: conf at masked positions,
 *               -1 elsewhere (NULL = not written)
 *   pred_out    optional [batch, block_len] int32: pred at masked positions,
 *               -1 elsewhere (NULL = not written)
 *   workspace, workspace_bytes  at least tt_unmask_workspace_bytes(batch,
 *               block_len, vocab) bytes: the per-chunk vocabulary partials
 *   stream      HIP stream the kernels are enqueued on (0 = null stream)
 * The call is deterministic.
 * Arguments beyond the path's named signature (logits, mask_state, k,
 * tokens_out, mask_out), all after it: batch, block_len and vocab (the sizes
 * of logits[B,L,V]); conf_out and pred_out (diagnostics, NULL = not
 * written); workspace and workspace_bytes; stream. */
tt_status tt_unmask_step(const float* logits, const uint8_t* mask_state, int k,
                         int32_t* tokens_out, uint8_t* mask_out, int batch, int block_len,
                         int vocab, float* conf_out, int32_t* pred_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* The two halves of tt_unmask_step, for callers that schedule them apart (for
 * instance to time the vocabulary pass alone).  tt_unmask_reduce writes the
 * per-chunk (max, argmax, sum of exponentials) partials of every masked row into
 * the workspace; tt_unmask_commit merges them, selects and commits.  Calling
 * reduce then commit on one stream with the same workspace, mask_state, batch,
 * block_len and vocab is exactly tt_unmask_step. */
tt_status tt_unmask_reduce(const float* logits, const uint8_t* mask_state, int batch,
                           int block_len, int vocab, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);
tt_status tt_unmask_commit(const uint8_t* mask_state, int k, int32_t* tokens_out,
                           uint8_t* mask_out, int batch, int block_len, int vocab,
                           float* conf_out, int32_t* pred_out, const void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Selection rule of one unmasking step: TwoTower paper §2.2 "Sampling" and
 * Algorithm 2, plus the one-token-per-step mode named in the "Versatile
 * Operation: Three Generation Modes" list of the article "NVIDIA's
 * Nemotron-Labs-TwoTower: Boosting AI Text Generation Speed".  Every rule
 * ranks the still-masked positions of a sequence and commits a prefix of that
 * ranking; n is the number of masked positions of the sequence.
 *   TT_SELECT_TOP_K      ranking (conf descending, position ascending);
 *                        commits min(k, n).  Same as tt_unmask_step.
 *   TT_SELECT_THRESHOLD  Algorithm 2's ConfidenceSample with threshold gamma and
 *                        steps_left = T - r + 1 remaining steps: every position
 *                        with conf > gamma (strict, in fp32), and at least
 *                        ceil(n / steps_left) of them, i.e. the first
 *                        min(n, max(#{conf > gamma}, ceil(n / steps_left))) of
 *                        the same ranking.  n masked positions are therefore
 *                        gone after steps_left steps; steps_left == 1 commits all.
 *   TT_SELECT_SCHEDULE   predict-and-noise with the linear schedule
 *                        alpha_t = 1 - t: step `step` (1-based) of `n_steps`
 *                        leaves floor(block_len * (n_steps - step) / n_steps)
 *                        positions masked and re-masks the least confident
 *                        predictions, i.e. commits the first
 *                        max(0, n - floor(block_len * (n_steps - step) / n_steps))
 *                        of the same ranking.
 *   TT_SELECT_LEFTMOST   mock-autoregressive: commits the min(k, n) masked
 *                        positions of lowest index, whatever their confidence
 *                        (k = 1: one token per step, left to right).
 * Fields a rule does not use are ignored. */
typedef enum {
  TT_SELECT_TOP_K = 0,
  TT_SELECT_THRESHOLD = 1,
  TT_SELECT_SCHEDULE = 2,
  TT_SELECT_LEFTMOST = 3
} tt_select_mode;

typedef struct {
  int mode;        /* tt_select_mode */
  int k;           /* TOP_K, LEFTMOST: >= 0 */
  float gamma;     /* THRESHOLD: finite */
  int steps_left;  /* THRESHOLD: >= 1 */
  int step;        /* SCHEDULE: 1 <= step <= n_steps */
  int n_steps;     /* SCHEDULE: >= 1 */
} tt_select;

/* tt_unmask_step / tt_unmask_commit under any selection rule.  `select` must
 * not be NULL; an unknown mode or a field outside its range returns TT_EINVAL.
 * All other arguments, outputs and guarantees are those of tt_unmask_step
 * (conf_out and pred_out report every masked position, committed or not). */
tt_status tt_unmask_step_ex(const float* logits, const uint8_t* mask_state,
                            const tt_select* select, int32_t* tokens_out, uint8_t* mask_out,
                            int batch, int block_len, int vocab, float* conf_out,
                            int32_t* pred_out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);
tt_status tt_unmask_commit_ex(const uint8_t* mask_state, const tt_select* select,
                              int32_t* tokens_out, uint8_t* mask_out, int batch, int block_len,
                              int vocab, float* conf_out, int32_t* pred_out,
                              const void* workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * tt_unmask_step, with the same arguments, outputs and guarantees, except that
 * its vocabulary partials live in a static device array of
 * TT_NOALLOC_SCRATCH_BYTES owned by the library (one per GPU, held until the
 * process ends) instead of a caller workspace.  The call allocates and frees
 * nothing.  Sizes whose workspace (tt_unmask_workspace_bytes) would exceed
 * TT_NOALLOC_SCRATCH_BYTES return TT_EUNSUPPORTED (8 MiB: e.g. 16384
 * positions of a 131072-word vocabulary).  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (other streams, other
 * threads) race and give undefined results; calls ordered on one stream are
 * safe.  The array needs no clearing between calls. */
#define TT_NOALLOC_SCRATCH_BYTES (8u << 20)
tt_status tt_unmask_step_noalloc(const float* logits, const uint8_t* mask_state, int k,
                                 int32_t* tokens_out, uint8_t* mask_out, int batch, int block_len,
                                 int vocab, float* conf_out, int32_t* pred_out,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Fused LM head + unmask: TwoTower paper §2.2 "Sampling", Algorithm 2.       */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace tt_lmhead_unmask_step needs (SIZE_MAX for invalid or
 * unsupported sizes). */
size_t tt_lmhead_unmask_workspace_bytes(int batch, int block_len, int vocab, int d_model);

/* One unmasking step whose logits come from the denoiser's LM head, without
 * writing them to memory: for every still-masked position,
 *   logits[v] = sum_i hidden[b,l,i] * weight[v,i]      (bf16 inputs, fp32 sums)
 * and then pred, conf and the selection exactly as tt_unmask_step_ex does on
 * those logits.  The hidden rows of positions that are not masked are never
 * read.
 *   hidden      [batch, block_len, d_model]  bf16
 *   weight      [vocab, d_model]             bf16 (the projection, one row per id)
 *   d_model     a positive multiple of 32 (otherwise TT_EUNSUPPORTED); also
 *               batch*block_len*d_model*2 < 2^32
 *   select, tokens_out, mask_out, conf_out, pred_out, batch, block_len
 *   (<= 1024), vocab, workspace, stream: as for tt_unmask_step_ex.
 * The logits are fp32 sums of d_model exact bf16 products, so pred, conf and
 * the commit set can differ from an exact computation only where the top two
 * logits, or two confidences at the selection boundary, are that close.
 * The call is deterministic. */
tt_status tt_lmhead_unmask_step(const void* hidden, const void* weight,
                                const uint8_t* mask_state, const tt_select* select,
                                int32_t* tokens_out, uint8_t* mask_out, int batch, int block_len,
                                int vocab, int d_model, float* conf_out, int32_t* pred_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* TT_H_ */
