// Internal declarations shared by the host entry points and the kernel files
// of libtt.  Not part of the public interface (include/tt.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tt {

// One block-attention call, resolved to kernel parameters.
struct AttnParams {
  const void* q;       // [B, Hq, L, D]
  const void* k_ctx;   // [B, Hkv, Pcap, D]
  const void* v_ctx;
  const void* k_blk;   // [B, Hkv, L, D]
  const void* v_blk;
  void* out;           // [B, Hq, L, D]
  float* part_o;       // [splits, B*Hq*L, D]   (splits > 1 only)
  float* part_lse;     // [splits, B*Hq*L]      base-2 log-sum-exp of each split
  int B, Hq, Hkv, G, L, P, Pcap, D;
  int M;               // G*L packed query rows per (batch, kv head)
  int n_keys;          // P + L
  int splits;          // key-range splits per query tile (>= 1), one workgroup each
  int tiles_per_split; // key tiles handled by one split
  int kgroups;         // MFMA kernel: 1 or 2 key groups inside a workgroup
  int out_bf16;        // 1: write bf16 output, 0: fp32
  float scale_log2;    // softmax scale * log2(e)
};

// Keys per tile of the MFMA kernel and packed query rows per workgroup.
constexpr int kAttnMfmaBN = 32;
constexpr int kAttnMfmaBM = 128;
// Keys per tile (one tile per split iteration) and rows per workgroup of the
// wavefront-shuffle kernel.
constexpr int kAttnShufRows = 8;
constexpr int kAttnShufBN = 16;

hipError_t launch_attn_mfma(const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_shuffle(const AttnParams& p, int in_bf16, hipStream_t stream);
hipError_t launch_attn_merge(const AttnParams& p, hipStream_t stream);

// Per-chunk partial of the vocabulary pass for one masked row.
struct VocabPartial {
  float m;        // max logit in the chunk
  int32_t arg;    // lowest id attaining it
  float s;        // sum over the chunk of exp(x - m)
  int32_t pad;
};

constexpr int kVocabChunk = 8192;    // logits per chunk (32 KB)
constexpr int kUnmaskMaxL = 1024;    // block_len limit of the commit kernel

struct UnmaskParams {
  const float* logits;      // [B, L, V]
  const uint8_t* mask_state;
  uint8_t* mask_out;
  int32_t* tokens_out;
  float* conf_out;          // optional
  int32_t* pred_out;        // optional
  VocabPartial* partials;   // [B*L, n_chunks]
  int B, L, V, k, n_chunks;
  // Selection rule (values of tt_select_mode) and its parameters.
  int mode;
  float gamma;
  int steps_left, step, n_steps;
};
enum { kSelTopK = 0, kSelThreshold = 1, kSelSchedule = 2, kSelLeftmost = 3 };

hipError_t launch_vocab_reduce(const UnmaskParams& p, hipStream_t stream);
hipError_t launch_topk_commit(const UnmaskParams& p, hipStream_t stream);

}  // namespace tt
