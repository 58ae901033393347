// Internal declarations shared by the host entry points and the kernel files
// of libtt.  Not part of the public interface (include/tt.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tt {

// One block-attention call, resolved to kernel parameters.
//
// Work items.  A call covers n_items = B * NB items; item w is block
// j = w % NB of batch entry b = w / NB (NB = 1 except for the multi-block
// pass).  Item w's queries are rows j*L .. j*L+L-1 of every query head of
// entry b in q (whose heads hold T = NB*L rows each), its block keys/values
// are rows j*L .. j*L+L-1 of each KV head in k_blk/v_blk (also T rows per
// head), and its prefix is rows 0 .. P_w-1 of the cache, with
//   P_w = P                       (prefix_mode 0, one length for all)
//   P_w = min(max(prefix_lens[b], 0), P)   (prefix_mode 1, P = the bound)
//   P_w = j*L                     (prefix_mode 2, the clean blocks before j)
// Packed query rows: the G*L rows of an (item, kv head) pair form M = G*L
// packed rows r -> (head g = r / L, position l = r % L); partial results of
// split-KV use the packed row index ((w*Hkv + kvh)*M + r).
struct AttnParams {
  const void* q;       // [B, Hq, T, D]
  const void* k_ctx;   // [B, Hkv, Pcap, D]
  const void* v_ctx;
  const void* k_blk;   // [B, Hkv, T, D]
  const void* v_blk;
  void* out;           // [B, Hq, T, D]
  float* part_o;       // [splits, rows, D]   (splits > 1 only)
  float* part_lse;     // [splits, rows]      base-2 log-sum-exp of each split
  const int32_t* prefix_lens;   // [B] device, prefix_mode 1 only
  int B, Hq, Hkv, G, L, P, Pcap, D;
  int NB;              // blocks per batch entry (items = B * NB)
  int T;               // rows per head of q / out / k_blk / v_blk (NB * L)
  int prefix_mode;     // 0, 1 or 2 (above)
  uint32_t L_magic;    // floor(2^32 / L) (2^32 - 1 for L = 1), for r / L
  int M;               // G*L packed query rows per (item, kv head)
  int n_keys;          // P + L: the longest item's key count (split planning)
  int tile_keys;       // keys per tile of the launched kernel (split planning)
  int splits;          // key-range splits per query tile (>= 1), one workgroup each
  int tiles_per_split; // key tiles handled by one split
  int kgroups;         // MFMA kernel: 1 or 2 key groups inside a workgroup
  int rows_per_wave;   // MFMA kernel: 32, or 64 (head_dim 128, one key group)
  int stream_waves;    // MFMA kernel: waves sharing one K/V stream, 4 or 8 (head_dim 128,
                       // one key group, 32-row waves)
  int nt_loads;        // MFMA kernel: 1 = K/V tile loads carry the non-temporal hint
                       // (each tile is read by few query-tile workgroups)
  int out_bf16;        // 1: write bf16 output, 0: fp32
  float scale_log2;    // softmax scale * log2(e)
};

// Item geometry, shared by every attention kernel.
struct AttnItem {
  int b, j;            // batch entry, block
  int P;               // prefix rows of this item
  int n_keys;          // P + L
  size_t q_head0;      // row of q/out where head (kvh*G) of this item starts (before j*L)
  size_t blk_row0;     // row of k_blk/v_blk of block row 0 of this item
  size_t ctx_row0;     // row of k_ctx/v_ctx of cache row 0 of this item
};

__device__ __forceinline__ AttnItem attn_item(const AttnParams& p, int w, int kvh) {
  AttnItem it;
  it.b = w / p.NB;
  it.j = w - it.b * p.NB;
  if (p.prefix_mode == 1)
    it.P = min(max(p.prefix_lens[it.b], 0), p.P);
  else if (p.prefix_mode == 2)
    it.P = it.j * p.L;
  else
    it.P = p.P;
  it.n_keys = it.P + p.L;
  it.q_head0 = ((size_t)it.b * p.Hq + (size_t)kvh * p.G) * p.T + (size_t)it.j * p.L;
  it.blk_row0 = ((size_t)it.b * p.Hkv + kvh) * p.T + (size_t)it.j * p.L;
  it.ctx_row0 = ((size_t)it.b * p.Hkv + kvh) * p.Pcap;
  return it;
}

// Offset of packed row r (head g = r / L, position l = r % L) from the item's
// q_head0: g*T + l, which is just r when T == L.
__device__ __forceinline__ size_t attn_row_off(const AttnParams& p, int r) {
  if (p.T == p.L) return (size_t)r;
  uint32_t g = __umulhi((uint32_t)r, p.L_magic);
  uint32_t l = (uint32_t)r - g * (uint32_t)p.L;
  if (l >= (uint32_t)p.L) {
    ++g;
    l -= (uint32_t)p.L;
  }
  return (size_t)g * p.T + l;
}

// Number of splits that hold keys of an item with n_keys keys.
__device__ __forceinline__ int attn_item_splits(const AttnParams& p, int n_keys) {
  const int tiles = (n_keys + p.tile_keys - 1) / p.tile_keys;
  return (tiles + p.tiles_per_split - 1) / p.tiles_per_split;
}

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

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Map dispatch index i of n to a logical index such that XCD x receives
// a contiguous range of logical ids.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int xcd = i & 7, local = i >> 3;
  const int per = (n + 7) >> 3;
  const int tall = ((n & 7) == 0) ? 8 : (n & 7);
  return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

// Per-chunk partial of the vocabulary pass for one masked row.
struct VocabPartial {
  float m;        // max logit in the chunk
  int32_t arg;    // lowest id attaining it
  float s;        // sum over the chunk of exp(x - m)
  int32_t pad;
};

constexpr int kVocabChunk = 8192;    // logits per chunk (32 KB)
constexpr int kVocabChunkManyRows = 4096;   // logits per chunk from kVocabChunkRows rows on
constexpr int kVocabChunkRows = 1024;
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
  int chunk;                // logits per chunk of the vocabulary pass
  // Selection rule (values of tt_select_mode) and its parameters.
  int mode;
  float gamma;
  int steps_left, step, n_steps;
};
enum { kSelTopK = 0, kSelThreshold = 1, kSelSchedule = 2, kSelLeftmost = 3 };

hipError_t launch_vocab_reduce(const UnmaskParams& p, hipStream_t stream);
hipError_t launch_topk_commit(const UnmaskParams& p, hipStream_t stream);

// Fused LM-head projection + vocabulary statistics.
constexpr int kLmRows = 256;     // hidden rows per workgroup
constexpr int kLmVocab = 256;    // vocabulary entries per workgroup (one slice)
constexpr int kLmK = 32;         // d_model granularity (stages take 64 columns, the last may take 32)
constexpr int kLmWorkgroups = 256;   // persistent stats workgroups: one per CU of an MI355X
struct LmParams {
  const void* hidden;        // [B*L, d] bf16
  const void* weight;        // [V, d] bf16
  const uint8_t* mask_state; // [B*L]
  int32_t* row_ids;          // [B*L] masked rows in order (workspace)
  int32_t* n_rows;           // [1] their count (workspace)
  VocabPartial* slices;      // [B*L, n_slices] per-slice partials (workspace)
  VocabPartial* merged;      // [B*L] one partial per masked row (workspace)
  int n_pos;                 // B*L
  int V, d, n_slices;
};
hipError_t launch_lmhead(const LmParams& p, hipStream_t stream);

}  // namespace tt
