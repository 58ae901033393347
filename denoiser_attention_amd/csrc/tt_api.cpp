// Host side of libtt: argument validation, kernel-family and split planning,
// workspace layout, and launches on the caller's stream.  The public contract
// is include/tt.h.  Nothing here allocates device memory.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "tt.h"
#include "tt_internal.h"

#define TT_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using tt::AttnParams;
using tt::UnmaskParams;

constexpr size_t kAlign = 256;
constexpr float kLog2e = 1.4426950408889634f;
// Workgroups the split heuristic aims for: two resident 256-thread
// workgroups on each of the 256 CUs for the MFMA kernel; more, smaller
// one-wave workgroups for the shuffle kernel.
constexpr long long kMfmaTargetWG = 512;
constexpr long long kShufTargetWG = 2048;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

tt_status device_present() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return TT_ENODEV;
  }
  return TT_OK;
}

struct AttnPlan {
  int path = TT_ATTN_SHUFFLE;  // resolved family
  int kgroups = 1;             // MFMA: wave groups splitting a workgroup's keys
  int rows_per_wave = 32;      // MFMA: query rows per wavefront
  int stream_waves = 4;        // MFMA: waves sharing one K/V tile stream
  bool nt_loads = false;       // MFMA: non-temporal hint on the K/V tile loads
  int splits = 1;
  int tiles_per_split = 1;
  bool empty = false;          // nothing to compute
  size_t ws_bytes = 0;
  size_t lse_offset = 0;
};

bool mfma_head_dim(int d) { return d == 64 || d == 128; }
bool shuffle_head_dim(int d) { return d == 64 || d == 128 || d == 256; }

// B counts work items (batch entries times blocks per entry); P is the
// longest item's prefix.
tt_status plan_attn(long long B, int P, int L, int Hq, int Hkv, int D, tt_dtype dtype,
                    const tt_attn_opts* opts, AttnPlan* plan) {
  if (B < 0 || P < 0 || L < 0 || Hq < 1 || Hkv < 1 || D < 1) return TT_EINVAL;
  if (B > INT_MAX) return TT_EUNSUPPORTED;
  if (Hq % Hkv != 0) return TT_EINVAL;
  if (dtype != TT_FP32 && dtype != TT_BF16) return TT_EINVAL;
  const int req = opts ? opts->path : TT_ATTN_AUTO;
  if (req != TT_ATTN_AUTO && req != TT_ATTN_MFMA && req != TT_ATTN_SHUFFLE) return TT_EINVAL;
  if (opts && opts->kv_splits < 0) return TT_EINVAL;
  if (opts && (opts->kv_groups < 0 || opts->kv_groups > 2)) return TT_EINVAL;
  if (opts && opts->rows_per_wave != 0 && opts->rows_per_wave != 32 && opts->rows_per_wave != 64)
    return TT_EINVAL;
  if (opts && opts->stream_waves != 0 && opts->stream_waves != 4 && opts->stream_waves != 8)
    return TT_EINVAL;
  if ((long long)P + L > INT_MAX / 2) return TT_EUNSUPPORTED;
  const int G = Hq / Hkv;
  const long long M = (long long)G * L;
  if (M > INT_MAX / 2) return TT_EUNSUPPORTED;

  if (req == TT_ATTN_MFMA) {
    if (dtype != TT_BF16 || !mfma_head_dim(D)) return TT_EUNSUPPORTED;
    plan->path = TT_ATTN_MFMA;
  } else if (req == TT_ATTN_SHUFFLE) {
    if (!shuffle_head_dim(D)) return TT_EUNSUPPORTED;
    plan->path = TT_ATTN_SHUFFLE;
  } else {
    // bf16 runs on the matrix cores at every packed-row count.  Forcing each
    // kernel at B64 P4096 (2 KV heads, D 128, G*L packed rows per KV head from
    // 1 to 32) measured the MFMA kernel 2.2x (G*L = 1) to 8x (G*L = 24)
    // faster than the wavefront-shuffle kernel: the call streams the cache K/V
    // either way, and the MFMA kernel's direct-to-LDS tile stream moves it at
    // 5.1-5.6 TB/s, its mostly empty row tiles costing nothing there, where the
    // shuffle kernel's per-key register loads reach 0.6-2.5 TB/s.  The shuffle
    // kernel serves fp32 inputs and head_dim 256.
    if (dtype == TT_BF16 && mfma_head_dim(D)) {
      plan->path = TT_ATTN_MFMA;
    } else if (shuffle_head_dim(D)) {
      plan->path = TT_ATTN_SHUFFLE;
    } else {
      return TT_EUNSUPPORTED;
    }
  }
  plan->empty = (B == 0 || L == 0);
  if (plan->empty) {
    plan->splits = 1;
    plan->tiles_per_split = 1;
    plan->ws_bytes = 0;
    return TT_OK;
  }

  const long long n_keys = (long long)P + L;
  long long n_tiles, splits;
  if (plan->path == TT_ATTN_MFMA) {
    // Units of 4 waves x 128 query rows; 512 of them fill 256 CUs at 2 waves
    // per SIMD.  With fewer query tiles than that, two wave groups per
    // workgroup split each workgroup's key range on chip, and workgroups split
    // it further (with a merge pass) only as far as still needed.
    n_tiles = cdiv(n_keys, tt::kAttnMfmaBN);
    const int req_groups = opts ? opts->kv_groups : 0;
    const int req_rows = opts ? opts->rows_per_wave : 0;
    // 64-row waves only on request: with one wave per SIMD they have measured
    // slower than 32-row waves at two waves per SIMD on every workload here.
    const long long base64 = cdiv(M, 2 * tt::kAttnMfmaBM) * B * Hkv;
    const bool rows64 = req_rows == 64;
    if (rows64 && (D != 128 || req_groups == 2)) return TT_EUNSUPPORTED;
    plan->rows_per_wave = rows64 ? 64 : 32;
    // Eight waves (256 rows) sharing one K/V stream halve the tile loads per
    // unit of matrix work; they need enough query tiles to fill the chip with
    // one such workgroup per CU.
    const int req_sw = opts ? opts->stream_waves : 0;
    if (req_sw == 8 && (D != 128 || rows64 || req_groups == 2)) return TT_EUNSUPPORTED;
    const long long base128 = cdiv(M, tt::kAttnMfmaBM) * B * Hkv;
    const bool sw8 = req_sw == 8;
    plan->stream_waves = sw8 ? 8 : 4;
    const long long base = (rows64 || sw8) ? base64 : base128;
    // When at most 4 query-tile workgroups read each K/V tile, the tiles are a
    // stream and the non-temporal hint moves them faster (B64 P4096 L1: 53.6 ->
    // 50.5 us; B8 P2048 L32: -1.6%); with 8 or more readers the hint costs L2
    // reuse (B64 P4096 L64: +2%), and from 32 it is neutral.
    plan->nt_loads = (rows64 || sw8 ? cdiv(M, 2 * tt::kAttnMfmaBM) : cdiv(M, tt::kAttnMfmaBM)) <= 4;
    // With few query tiles, two wave groups per workgroup split each key range
    // on chip -- unless that leaves each group 8 tiles or fewer, where the
    // pipeline start and the on-chip merge dominate: one group per workgroup
    // and about one workgroup per CU of key splits measured faster there.
    long long target = kMfmaTargetWG;
    if (rows64 || sw8) {
      plan->kgroups = 1;
      target = kMfmaTargetWG / 2;
    } else if (req_groups) {
      plan->kgroups = req_groups;
    } else if (base >= kMfmaTargetWG) {
      plan->kgroups = 1;
    } else if (M < tt::kAttnMfmaBM) {
      // Fewer packed rows than one query tile (single-token and very short
      // blocks): the matrix work is light and the call is a stream of K/V.
      // When the query tiles fill 3/4 to all of the CUs once, two key groups
      // per workgroup stream each tile's keys without splits (P2048 L1: 192
      // tiles 37.1 vs 42.7 us, 224: 42.5 vs 45.5, 256: 47.4 vs 49.6); with
      // more, 8-wave workgroups would need a second round (320 tiles: 81.6 vs
      // 61.7), and with fewer, one 4-wave workgroup per CU streaming a split
      // of the key range moved the bytes as fast or faster (B32 P8192 L1:
      // 50.5 vs 52.3).
      const long long cus = kMfmaTargetWG / 2;
      if (base * 4 >= 3 * cus && base <= cus) {
        plan->kgroups = 2;
        target = 2 * base;   // one split
      } else {
        plan->kgroups = 1;
        target = cus;
      }
    } else {
      const long long s2 = std::min(cdiv(kMfmaTargetWG / 2, base), std::max(n_tiles / 4, 1LL));
      const bool short_groups = n_tiles / (2 * s2) <= 8;
      plan->kgroups = short_groups ? 1 : 2;
      if (short_groups) target = kMfmaTargetWG / 2;
    }
    if (opts && opts->kv_splits > 0) {
      splits = opts->kv_splits < n_tiles ? opts->kv_splits : n_tiles;
    } else {
      splits = cdiv(target / plan->kgroups, base);
      const long long min_tiles = 2 * plan->kgroups;   // per workgroup
      const long long max_splits = n_tiles / min_tiles > 1 ? n_tiles / min_tiles : 1;
      if (splits > max_splits) splits = max_splits;
      if (splits < 1) splits = 1;
    }
    if (base * splits > INT_MAX) return TT_EUNSUPPORTED;
  } else {
    n_tiles = cdiv(n_keys, tt::kAttnShufBN);
    const long long base = cdiv(M, tt::kAttnShufRows) * B * Hkv;
    if (opts && opts->kv_splits > 0) {
      splits = opts->kv_splits < n_tiles ? opts->kv_splits : n_tiles;
    } else {
      splits = cdiv(kShufTargetWG, base);
      const long long max_splits = n_tiles / 2 > 1 ? n_tiles / 2 : 1;
      if (splits > max_splits) splits = max_splits;
      if (splits < 1) splits = 1;
    }
    if (base * splits > INT_MAX) return TT_EUNSUPPORTED;
  }
  const long long tps = cdiv(n_tiles, splits);
  splits = cdiv(n_tiles, tps);   // no empty split
  plan->splits = (int)splits;
  plan->tiles_per_split = (int)tps;
  if (splits > 1) {
    const size_t rows = (size_t)B * Hq * L;
    // The merge pass indexes (row, 4 columns) with 32-bit arithmetic.
    if (rows * (size_t)(D / 4) > 0xffffff00ULL) return TT_EUNSUPPORTED;
    const size_t o_bytes = align_up((size_t)splits * rows * D * sizeof(float));
    plan->lse_offset = o_bytes;
    plan->ws_bytes = o_bytes + align_up((size_t)splits * rows * sizeof(float));
  } else {
    plan->ws_bytes = 0;
  }
  return TT_OK;
}

tt_status to_status(hipError_t e) { return e == hipSuccess ? TT_OK : TT_EHIP; }

// The attention and LM-head kernels move tiles with 16-byte loads and stores
// (and direct-to-LDS loads) from each tensor's base address.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct UnmaskPlan {
  int n_chunks = 0;
  int chunk = 0;
  size_t ws_bytes = 0;
  bool empty = false;
};

tt_status plan_unmask(int B, int L, int V, UnmaskPlan* plan) {
  if (B < 0 || L < 0 || V < 1) return TT_EINVAL;
  if (L > tt::kUnmaskMaxL) return TT_EUNSUPPORTED;
  // With many positions per call the grid is large either way, and 16 KB
  // chunks stream faster (4096 rows: step 2.5% faster); with few, the commit's
  // second round of chunk loads would cost more than the pass gains.
  plan->chunk = (long long)B * L >= tt::kVocabChunkRows ? tt::kVocabChunkManyRows : tt::kVocabChunk;
  plan->n_chunks = (int)cdiv(V, plan->chunk);
  plan->empty = (B == 0 || L == 0);
  const long long wgs = (long long)B * L * plan->n_chunks;
  if (wgs > INT_MAX) return TT_EUNSUPPORTED;
  plan->ws_bytes = plan->empty ? 0 : align_up((size_t)wgs * sizeof(tt::VocabPartial));
  return TT_OK;
}

}  // namespace

TT_EXPORT const char* tt_status_string(tt_status s) {
  switch (s) {
    case TT_OK: return "TT_OK";
    case TT_EINVAL: return "TT_EINVAL: invalid argument";
    case TT_EUNSUPPORTED: return "TT_EUNSUPPORTED: not covered by the compiled kernels";
    case TT_ENODEV: return "TT_ENODEV: no HIP device visible";
    case TT_EHIP: return "TT_EHIP: HIP runtime or launch failure";
  }
  return "unknown tt_status";
}

TT_EXPORT const char* tt_version(void) { return "0.1.0"; }

TT_EXPORT size_t tt_block_attn_workspace_bytes(int batch, int prefix_len, int block_len,
                                               int n_q_heads, int n_kv_heads, int head_dim,
                                               tt_dtype dtype, const tt_attn_opts* opts) {
  AttnPlan plan;
  if (plan_attn(batch, prefix_len, block_len, n_q_heads, n_kv_heads, head_dim, dtype, opts,
                &plan) != TT_OK)
    return SIZE_MAX;
  return plan.ws_bytes;
}

namespace {

// One attention call in any of its three forms.
struct AttnCall {
  const void *q, *k_ctx, *v_ctx, *k_blk, *v_blk;
  void* out;
  const int32_t* prefix_lens;   // mode 1
  int prefix_mode;              // 0 uniform, 1 per batch entry, 2 multi-block
  int P;                        // mode 0: the prefix; mode 1: the bound; mode 2: unused
  int L, NB, Hq, Hkv, D, batch, Pcap;
  float scale;
  tt_dtype dtype, out_dtype;
  void* workspace;
  size_t workspace_bytes;
  hipStream_t stream;
  const tt_attn_opts* opts;
};

// Longest prefix of any item of the call.
int call_max_prefix(const AttnCall& c) {
  return c.prefix_mode == 2 ? (c.NB > 0 ? (c.NB - 1) * c.L : 0) : c.P;
}

tt_status attn_run(const AttnCall& c) {
  if (c.NB < 0 || c.L < 0) return TT_EINVAL;
  if (c.prefix_mode == 2 && (long long)c.NB * c.L > INT_MAX / 2) return TT_EUNSUPPORTED;
  const int Pmax = call_max_prefix(c);
  AttnPlan plan;
  tt_status st = plan_attn((long long)c.batch * c.NB, Pmax, c.L, c.Hq, c.Hkv, c.D, c.dtype,
                           c.opts, &plan);
  if (st != TT_OK) return st;
  if (c.Pcap < Pmax) return TT_EINVAL;
  // The kernels work in base-2 units: scale * log2(e) must stay finite.
  if (!std::isfinite(c.scale) || !std::isfinite(c.scale * kLog2e)) return TT_EINVAL;
  if (c.out_dtype != TT_FP32 && c.out_dtype != TT_BF16) return TT_EINVAL;
  if (c.dtype == TT_FP32 && c.out_dtype != TT_FP32) return TT_EINVAL;
  if (plan.empty) return TT_OK;
  if (!c.q || !c.k_blk || !c.v_blk || !c.out) return TT_EINVAL;
  if (c.Pcap > 0 && (!c.k_ctx || !c.v_ctx)) return TT_EINVAL;
  if (c.prefix_mode == 1 && !c.prefix_lens) return TT_EINVAL;
  if (plan.ws_bytes > 0 && (!c.workspace || c.workspace_bytes < plan.ws_bytes)) return TT_EINVAL;
  if (!aligned16(c.q) || !aligned16(c.k_ctx) || !aligned16(c.v_ctx) || !aligned16(c.k_blk) ||
      !aligned16(c.v_blk) || !aligned16(c.out))
    return TT_EINVAL;
  if (plan.ws_bytes > 0 && !aligned16(c.workspace)) return TT_EINVAL;
  if (c.prefix_mode == 1 && (reinterpret_cast<uintptr_t>(c.prefix_lens) & 3u) != 0)
    return TT_EINVAL;
  st = device_present();
  if (st != TT_OK) return st;

  AttnParams p{};
  p.q = c.q;
  p.k_ctx = c.k_ctx;
  p.v_ctx = c.v_ctx;
  p.k_blk = c.k_blk;
  p.v_blk = c.v_blk;
  p.out = c.out;
  p.prefix_lens = c.prefix_lens;
  p.B = c.batch;
  p.Hq = c.Hq;
  p.Hkv = c.Hkv;
  p.G = c.Hq / c.Hkv;
  p.L = c.L;
  p.P = Pmax;
  p.Pcap = c.Pcap;
  p.D = c.D;
  p.NB = c.NB;
  p.T = c.NB * c.L;
  p.prefix_mode = c.prefix_mode;
  p.L_magic = c.L == 1 ? 0xffffffffu : (uint32_t)((1ull << 32) / (unsigned)c.L);
  p.M = p.G * c.L;
  p.n_keys = Pmax + c.L;
  p.tile_keys = plan.path == TT_ATTN_MFMA ? tt::kAttnMfmaBN : tt::kAttnShufBN;
  p.splits = plan.splits;
  p.tiles_per_split = plan.tiles_per_split;
  p.kgroups = plan.kgroups;
  p.rows_per_wave = plan.rows_per_wave;
  p.stream_waves = plan.stream_waves;
  p.nt_loads = plan.nt_loads ? 1 : 0;
  p.out_bf16 = c.out_dtype == TT_BF16 ? 1 : 0;
  p.scale_log2 = c.scale * kLog2e;
  if (plan.splits > 1) {
    p.part_o = static_cast<float*>(c.workspace);
    p.part_lse = reinterpret_cast<float*>(static_cast<char*>(c.workspace) + plan.lse_offset);
  }

  (void)hipGetLastError();  // clear any stale error so it is not reported as ours
  hipError_t e = plan.path == TT_ATTN_MFMA
                     ? tt::launch_attn_mfma(p, c.stream)
                     : tt::launch_attn_shuffle(p, c.dtype == TT_BF16, c.stream);
  if (e != hipSuccess) return TT_EHIP;
  if (plan.splits > 1) {
    e = tt::launch_attn_merge(p, c.stream);
    if (e != hipSuccess) return TT_EHIP;
  }
  return TT_OK;
}

}  // namespace

TT_EXPORT tt_status tt_block_attn_ex(const void* q, const void* k_ctx, const void* v_ctx,
                                     int prefix_len, const void* k_blk, const void* v_blk,
                                     int block_len, int n_q_heads, int n_kv_heads, int head_dim,
                                     float scale, void* out, int batch, int prefix_cap,
                                     tt_dtype dtype, tt_dtype out_dtype, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream,
                                     const tt_attn_opts* opts) {
  if (prefix_len < 0) return TT_EINVAL;
  AttnCall c{q, k_ctx, v_ctx, k_blk, v_blk, out, nullptr, 0, prefix_len, block_len, 1,
             n_q_heads, n_kv_heads, head_dim, batch, prefix_cap, scale, dtype, out_dtype,
             workspace, workspace_bytes, stream, opts};
  return attn_run(c);
}

TT_EXPORT tt_status tt_block_attn(const void* q, const void* k_ctx, const void* v_ctx,
                                  int prefix_len, const void* k_blk, const void* v_blk,
                                  int block_len, int n_q_heads, int n_kv_heads, int head_dim,
                                  float scale, void* out, int batch, int prefix_cap,
                                  tt_dtype dtype, tt_dtype out_dtype, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return tt_block_attn_ex(q, k_ctx, v_ctx, prefix_len, k_blk, v_blk, block_len, n_q_heads,
                          n_kv_heads, head_dim, scale, out, batch, prefix_cap, dtype, out_dtype,
                          workspace, workspace_bytes, stream, nullptr);
}

TT_EXPORT tt_status tt_block_attn_varlen(const void* q, const void* k_ctx, const void* v_ctx,
                                         const int32_t* prefix_lens, int max_prefix_len,
                                         const void* k_blk, const void* v_blk, int block_len,
                                         int n_q_heads, int n_kv_heads, int head_dim, float scale,
                                         void* out, int batch, int prefix_cap, tt_dtype dtype,
                                         tt_dtype out_dtype, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream,
                                         const tt_attn_opts* opts) {
  if (max_prefix_len < 0) return TT_EINVAL;
  AttnCall c{q, k_ctx, v_ctx, k_blk, v_blk, out, prefix_lens, 1, max_prefix_len, block_len, 1,
             n_q_heads, n_kv_heads, head_dim, batch, prefix_cap, scale, dtype, out_dtype,
             workspace, workspace_bytes, stream, opts};
  return attn_run(c);
}

TT_EXPORT size_t tt_block_attn_multiblock_workspace_bytes(int batch, int block_size,
                                                          int n_blocks, int n_q_heads,
                                                          int n_kv_heads, int head_dim,
                                                          tt_dtype dtype,
                                                          const tt_attn_opts* opts) {
  if (batch < 0 || block_size < 0 || n_blocks < 0) return SIZE_MAX;
  if ((long long)n_blocks * block_size > INT_MAX / 2) return SIZE_MAX;
  AttnPlan plan;
  const int Pmax = n_blocks > 0 ? (n_blocks - 1) * block_size : 0;
  if (plan_attn((long long)batch * n_blocks, Pmax, block_size, n_q_heads, n_kv_heads, head_dim,
                dtype, opts, &plan) != TT_OK)
    return SIZE_MAX;
  return plan.ws_bytes;
}

TT_EXPORT tt_status tt_block_attn_multiblock(const void* q, const void* k_ctx, const void* v_ctx,
                                             const void* k_noisy, const void* v_noisy,
                                             int block_size, int n_blocks, int n_q_heads,
                                             int n_kv_heads, int head_dim, float scale, void* out,
                                             int batch, int ctx_cap, tt_dtype dtype,
                                             tt_dtype out_dtype, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream,
                                             const tt_attn_opts* opts) {
  AttnCall c{q, k_ctx, v_ctx, k_noisy, v_noisy, out, nullptr, 2, 0, block_size, n_blocks,
             n_q_heads, n_kv_heads, head_dim, batch, ctx_cap, scale, dtype, out_dtype,
             workspace, workspace_bytes, stream, opts};
  return attn_run(c);
}

TT_EXPORT size_t tt_unmask_workspace_bytes(int batch, int block_len, int vocab) {
  UnmaskPlan plan;
  if (plan_unmask(batch, block_len, vocab, &plan) != TT_OK) return SIZE_MAX;
  return plan.ws_bytes;
}

namespace {

tt_status unmask_prepare(const float* logits, const uint8_t* mask_state, int batch,
                         int block_len, int vocab, const void* workspace,
                         size_t workspace_bytes, UnmaskPlan* plan, UnmaskParams* p) {
  tt_status st = plan_unmask(batch, block_len, vocab, plan);
  if (st != TT_OK) return st;
  if (plan->empty) return TT_OK;
  if (!mask_state) return TT_EINVAL;
  if (!workspace || workspace_bytes < plan->ws_bytes) return TT_EINVAL;
  p->logits = logits;
  p->mask_state = mask_state;
  p->partials = static_cast<tt::VocabPartial*>(const_cast<void*>(workspace));
  p->B = batch;
  p->L = block_len;
  p->V = vocab;
  p->n_chunks = plan->n_chunks;
  p->chunk = plan->chunk;
  return TT_OK;
}

}  // namespace

TT_EXPORT tt_status tt_unmask_reduce(const float* logits, const uint8_t* mask_state, int batch,
                                     int block_len, int vocab, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  UnmaskPlan plan;
  UnmaskParams p{};
  tt_status st = unmask_prepare(logits, mask_state, batch, block_len, vocab, workspace,
                                workspace_bytes, &plan, &p);
  if (st != TT_OK || plan.empty) return st;
  if (!logits) return TT_EINVAL;
  st = device_present();
  if (st != TT_OK) return st;
  (void)hipGetLastError();
  return to_status(tt::launch_vocab_reduce(p, stream));
}

namespace {

// Validates a selection rule and stores it in p.
tt_status set_select(const tt_select* sel, UnmaskParams* p) {
  if (!sel) return TT_EINVAL;
  p->mode = sel->mode;
  p->k = 0;
  p->gamma = 0.0f;
  p->steps_left = p->step = p->n_steps = 1;
  switch (sel->mode) {
    case TT_SELECT_TOP_K:
    case TT_SELECT_LEFTMOST:
      if (sel->k < 0) return TT_EINVAL;
      p->k = sel->k;
      return TT_OK;
    case TT_SELECT_THRESHOLD:
      if (!std::isfinite(sel->gamma) || sel->steps_left < 1) return TT_EINVAL;
      p->gamma = sel->gamma;
      p->steps_left = sel->steps_left;
      return TT_OK;
    case TT_SELECT_SCHEDULE:
      if (sel->n_steps < 1 || sel->step < 1 || sel->step > sel->n_steps) return TT_EINVAL;
      p->step = sel->step;
      p->n_steps = sel->n_steps;
      return TT_OK;
    default:
      return TT_EINVAL;
  }
}

tt_status unmask_run(const float* logits, const uint8_t* mask_state, const tt_select* sel,
                     int32_t* tokens_out, uint8_t* mask_out, int batch, int block_len, int vocab,
                     float* conf_out, int32_t* pred_out, const void* workspace,
                     size_t workspace_bytes, hipStream_t stream, bool reduce) {
  UnmaskParams p{};
  tt_status st = set_select(sel, &p);
  if (st != TT_OK) return st;
  UnmaskPlan plan;
  st = unmask_prepare(logits, mask_state, batch, block_len, vocab, workspace, workspace_bytes,
                      &plan, &p);
  if (st != TT_OK || plan.empty) return st;
  if ((reduce && !logits) || !tokens_out || !mask_out) return TT_EINVAL;
  st = device_present();
  if (st != TT_OK) return st;
  p.tokens_out = tokens_out;
  p.mask_out = mask_out;
  p.conf_out = conf_out;
  p.pred_out = pred_out;
  (void)hipGetLastError();
  if (reduce) {
    const hipError_t e = tt::launch_vocab_reduce(p, stream);
    if (e != hipSuccess) return TT_EHIP;
  }
  return to_status(tt::launch_topk_commit(p, stream));
}

}  // namespace

TT_EXPORT tt_status tt_unmask_commit(const uint8_t* mask_state, int k, int32_t* tokens_out,
                                     uint8_t* mask_out, int batch, int block_len, int vocab,
                                     float* conf_out, int32_t* pred_out, const void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  tt_select sel{TT_SELECT_TOP_K, k, 0.0f, 1, 1, 1};
  return unmask_run(nullptr, mask_state, &sel, tokens_out, mask_out, batch, block_len, vocab,
                    conf_out, pred_out, workspace, workspace_bytes, stream, false);
}

TT_EXPORT tt_status tt_unmask_commit_ex(const uint8_t* mask_state, const tt_select* select,
                                        int32_t* tokens_out, uint8_t* mask_out, int batch,
                                        int block_len, int vocab, float* conf_out,
                                        int32_t* pred_out, const void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  return unmask_run(nullptr, mask_state, select, tokens_out, mask_out, batch, block_len, vocab,
                    conf_out, pred_out, workspace, workspace_bytes, stream, false);
}

TT_EXPORT tt_status tt_unmask_step(const float* logits, const uint8_t* mask_state, int k,
                                   int32_t* tokens_out, uint8_t* mask_out, int batch,
                                   int block_len, int vocab, float* conf_out, int32_t* pred_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  tt_select sel{TT_SELECT_TOP_K, k, 0.0f, 1, 1, 1};
  return unmask_run(logits, mask_state, &sel, tokens_out, mask_out, batch, block_len, vocab,
                    conf_out, pred_out, workspace, workspace_bytes, stream, true);
}

TT_EXPORT tt_status tt_unmask_step_ex(const float* logits, const uint8_t* mask_state,
                                      const tt_select* select, int32_t* tokens_out,
                                      uint8_t* mask_out, int batch, int block_len, int vocab,
                                      float* conf_out, int32_t* pred_out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return unmask_run(logits, mask_state, select, tokens_out, mask_out, batch, block_len, vocab,
                    conf_out, pred_out, workspace, workspace_bytes, stream, true);
}

namespace {

struct LmPlan {
  int n_slices = 0;
  size_t slices_off = 0, merged_off = 0, rows_off = 0, count_off = 0, ws_bytes = 0;
  bool empty = false;
};

tt_status plan_lmhead(int B, int L, int V, int d, LmPlan* plan) {
  if (B < 0 || L < 0 || V < 1 || d < 1) return TT_EINVAL;
  if (L > tt::kUnmaskMaxL) return TT_EUNSUPPORTED;
  if (d % tt::kLmK != 0) return TT_EUNSUPPORTED;
  const long long n_pos = (long long)B * L;
  if (n_pos > INT_MAX / 2) return TT_EUNSUPPORTED;
  // 32-bit byte offsets inside the hidden matrix and a weight slice.
  if (n_pos * d * 2 >= (1ll << 32) || (long long)tt::kLmVocab * d * 2 >= (1ll << 32))
    return TT_EUNSUPPORTED;
  plan->empty = n_pos == 0;
  plan->n_slices = (int)cdiv(V, tt::kLmVocab);
  if (plan->empty) return TT_OK;
  size_t off = 0;
  plan->slices_off = off;
  off += align_up((size_t)n_pos * plan->n_slices * sizeof(tt::VocabPartial));
  plan->merged_off = off;
  off += align_up((size_t)n_pos * sizeof(tt::VocabPartial));
  plan->rows_off = off;
  off += align_up((size_t)n_pos * sizeof(int32_t));
  plan->count_off = off;
  off += align_up(sizeof(int32_t));
  plan->ws_bytes = off;
  return TT_OK;
}

}  // namespace

TT_EXPORT size_t tt_lmhead_unmask_workspace_bytes(int batch, int block_len, int vocab,
                                                  int d_model) {
  LmPlan plan;
  if (plan_lmhead(batch, block_len, vocab, d_model, &plan) != TT_OK) return SIZE_MAX;
  return plan.ws_bytes;
}

TT_EXPORT tt_status tt_lmhead_unmask_step(const void* hidden, const void* weight,
                                          const uint8_t* mask_state, const tt_select* select,
                                          int32_t* tokens_out, uint8_t* mask_out, int batch,
                                          int block_len, int vocab, int d_model,
                                          float* conf_out, int32_t* pred_out, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  UnmaskParams up{};
  tt_status st = set_select(select, &up);
  if (st != TT_OK) return st;
  LmPlan plan;
  st = plan_lmhead(batch, block_len, vocab, d_model, &plan);
  if (st != TT_OK || plan.empty) return st;
  if (!hidden || !weight || !mask_state || !tokens_out || !mask_out) return TT_EINVAL;
  if (!workspace || workspace_bytes < plan.ws_bytes) return TT_EINVAL;
  if (!aligned16(hidden) || !aligned16(weight) || !aligned16(workspace)) return TT_EINVAL;
  st = device_present();
  if (st != TT_OK) return st;
  char* ws = static_cast<char*>(workspace);
  tt::LmParams lp{};
  lp.hidden = hidden;
  lp.weight = weight;
  lp.mask_state = mask_state;
  lp.slices = reinterpret_cast<tt::VocabPartial*>(ws + plan.slices_off);
  lp.merged = reinterpret_cast<tt::VocabPartial*>(ws + plan.merged_off);
  lp.row_ids = reinterpret_cast<int32_t*>(ws + plan.rows_off);
  lp.n_rows = reinterpret_cast<int32_t*>(ws + plan.count_off);
  lp.n_pos = batch * block_len;
  lp.V = vocab;
  lp.d = d_model;
  lp.n_slices = plan.n_slices;
  up.mask_state = mask_state;
  up.partials = lp.merged;
  up.B = batch;
  up.L = block_len;
  up.V = vocab;
  up.n_chunks = 1;
  up.tokens_out = tokens_out;
  up.mask_out = mask_out;
  up.conf_out = conf_out;
  up.pred_out = pred_out;
  (void)hipGetLastError();
  const hipError_t e = tt::launch_lmhead(lp, stream);
  if (e != hipSuccess) return TT_EHIP;
  return to_status(tt::launch_topk_commit(up, stream));
}

// ---------------------------------------------------------------------------
// tt_unmask_step_noalloc: tt_unmask_step with its vocabulary partials in a
// static device array instead of a caller workspace.
// ---------------------------------------------------------------------------

// Every GPU the library runs on holds its own copy of this array until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: only the address hipGetSymbolAddress returns for the current device
// is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[TT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up once per device (with
// that device current) and kept.
tt_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return TT_ENODEV;
  }
  if (dev >= kMaxDevices) return TT_EUNSUPPORTED;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
        (void)hipGetLastError();
        return TT_EHIP;
      }
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return TT_OK;
}

}  // namespace

TT_EXPORT tt_status tt_unmask_step_noalloc(const float* logits, const uint8_t* mask_state, int k,
                                           int32_t* tokens_out, uint8_t* mask_out, int batch,
                                           int block_len, int vocab, float* conf_out,
                                           int32_t* pred_out, hipStream_t stream) {
  tt_select sel{TT_SELECT_TOP_K, k, 0.0f, 1, 1, 1};
  UnmaskParams p{};
  tt_status st = set_select(&sel, &p);
  if (st != TT_OK) return st;
  UnmaskPlan plan;
  st = plan_unmask(batch, block_len, vocab, &plan);
  if (st != TT_OK || plan.empty) return st;
  if (plan.ws_bytes > (size_t)TT_NOALLOC_SCRATCH_BYTES) return TT_EUNSUPPORTED;
  if (!logits || !mask_state || !tokens_out || !mask_out) return TT_EINVAL;
  st = device_present();
  if (st != TT_OK) return st;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != TT_OK) return st;
  // Nothing in the array needs clearing: the vocabulary pass writes the
  // partial of every (masked position, chunk) before the commit reads it, and
  // the slots of unmasked positions are read and ignored.
  return unmask_run(logits, mask_state, &sel, tokens_out, mask_out, batch, block_len, vocab,
                    conf_out, pred_out, ws, (size_t)TT_NOALLOC_SCRATCH_BYTES, stream, true);
}
