// Confidence unmasking: fused vocabulary reduction and per-sequence top-k.
//
// Operation: TwoTower paper §2.2 "Sampling" and Algorithm 2 (ConfidenceSample),
// fixed-k form.  For every still-masked position the denoiser's prediction is
// the argmax of its logit row and its confidence is the largest softmax
// probability, 1 / sum_v exp(x_v - max); the k most confident masked positions
// of each sequence are committed (ties: lower position first), the rest stay
// masked.  Logit rows of positions that are not masked are never read.
//
// vocab_reduce_kernel -- the HBM-bound pass.  A workgroup reduces one chunk
//   of one masked row: 8192 logits (32 KB), or 4096 when a call covers at least
//   1024 positions (the plan's choice).  Every thread issues all of its 128-bit
//   loads up front (8 or 4 x 16 B), takes the max / lowest-id argmax over its
//   values on the raw fp32 logits, then its sum of exp2((x - max) * log2 e);
//   across the wave the maximum is found first (xor shuffles), then the lowest
//   id attaining it and the sum rescaled once to it; the 4 waves' (max,
//   argmax, sum) triples merge through LDS, ties going to the lower id at
//   every stage.  Chunks of unmasked rows exit at once.
// topk_commit_kernel -- one workgroup per sequence: merges the chunk triples of
//   each masked position (one thread per position, in chunk order), forms the
//   confidence, ranks every masked position by counting the positions ahead
//   of it in the order (confidence descending, position ascending) with one
//   64-bit key comparison each (or by counting the masked positions before it,
//   for the mock-autoregressive rule), and commits rank < k, where k comes
//   from the selection rule: fixed, or derived from the sequence's masked
//   count and its count of confidences above gamma.
#include <climits>

#include "tt_internal.h"

namespace tt {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
static_assert(kVocabChunk % (kThreads * 4) == 0 && kVocabChunkManyRows % (kThreads * 4) == 0,
              "chunks must be multiples of 1024 logits");

struct Triple {
  float m;
  int arg;
  float s;
};

// Merge two (max, lowest argmax, sum of exp(x - max)) triples.  An empty
// triple is (-inf, INT_MAX, 0).
__device__ __forceinline__ Triple combine(Triple a, Triple b) {
  Triple r;
  r.m = fmaxf(a.m, b.m);
  const float sa = a.m == -INFINITY ? 0.0f : a.s * __builtin_amdgcn_exp2f((a.m - r.m) * kLog2e);
  const float sb = b.m == -INFINITY ? 0.0f : b.s * __builtin_amdgcn_exp2f((b.m - r.m) * kLog2e);
  r.s = sa + sb;
  r.arg = a.m > b.m ? a.arg : (b.m > a.m ? b.arg : min(a.arg, b.arg));
  return r;
}

template <bool VEC, int CHUNK>
__global__ __launch_bounds__(kThreads) void vocab_reduce_kernel(UnmaskParams p) {
  constexpr int kVecPerThread = CHUNK / (kThreads * 4);   // float4 loads per thread
  constexpr int kScalarPerThread = CHUNK / kThreads;      // scalar loads per thread
  const size_t gid = blockIdx.x;
  const size_t row = gid / (size_t)p.n_chunks;
  const int chunk = (int)(gid % (size_t)p.n_chunks);
  {
    // The row's flag, read through the aligned 32-bit word that holds it when
    // that word lies inside the mask (a uniform address: one scalar load,
    // 1.7% faster than the byte load); otherwise through the byte itself.
    const size_t n_pos = (size_t)p.B * p.L;
    uint32_t flag;
    if ((reinterpret_cast<uintptr_t>(p.mask_state) & 3) == 0 && (row | 3) < n_pos) {
      const uint32_t w = reinterpret_cast<const uint32_t*>(p.mask_state)[row >> 2];
      flag = (w >> (8 * (row & 3))) & 0xffu;
    } else {
      flag = p.mask_state[row];
    }
    if (flag == 0) return;
  }

  const int tid = threadIdx.x;
  const int V = p.V;
  const int c0 = chunk * CHUNK;
  const int c1 = min(V, c0 + CHUNK);
  const float* x = p.logits + row * (size_t)V;

  Triple t{-INFINITY, INT_MAX, 0.0f};
  if (VEC) {
    // V % 4 == 0 and 16-byte aligned rows: ids c0 + i*1024 + 4*tid + {0..3}.
    f32x4 v[kVecPerThread];
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
      const int idx = c0 + i * (kThreads * 4) + 4 * tid;
      v[i] = idx < c1 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + idx))
                      : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    // Values are visited in increasing id order; strict '>' keeps the lowest id.
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
      const int idx = c0 + i * (kThreads * 4) + 4 * tid;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (v[i][e] > t.m) { t.m = v[i][e]; t.arg = idx + e; }
      }
    }
    if (t.m != -INFINITY) {
      const float mb = t.m * kLog2e;
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < kVecPerThread; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) s += __builtin_amdgcn_exp2f(fmaf(v[i][e], kLog2e, -mb));
      t.s = s;
    }
  } else {
    float v[kScalarPerThread];
#pragma unroll
    for (int i = 0; i < kScalarPerThread; ++i) {
      const int idx = c0 + i * kThreads + tid;
      v[i] = idx < c1 ? x[idx] : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < kScalarPerThread; ++i) {
      if (v[i] > t.m) { t.m = v[i]; t.arg = c0 + i * kThreads + tid; }
    }
    if (t.m != -INFINITY) {
      const float mb = t.m * kLog2e;
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < kScalarPerThread; ++i) s += __builtin_amdgcn_exp2f(fmaf(v[i], kLog2e, -mb));
      t.s = s;
    }
  }

  // Across the wave: the maximum first, then the lowest id attaining it and
  // the sum rescaled once to that maximum (one exponential per lane).
  {
    float m = t.m;
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) m = fmaxf(m, __shfl_xor(m, mask));
    int arg = t.m == m ? t.arg : INT_MAX;
    float s = t.m == -INFINITY ? 0.0f : t.s * __builtin_amdgcn_exp2f((t.m - m) * kLog2e);
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) {
      arg = min(arg, __shfl_xor(arg, mask));
      s += __shfl_xor(s, mask);
    }
    t = Triple{m, arg, s};
  }

  __shared__ Triple s_t[kThreads / 64];
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) s_t[wave] = t;
  __syncthreads();
  if (tid == 0) {
    Triple r = s_t[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = combine(r, s_t[w]);
    VocabPartial out;
    out.m = r.m;
    out.arg = r.arg;
    out.s = r.s;
    out.pad = 0;
    p.partials[row * (size_t)p.n_chunks + chunk] = out;
  }
}

__global__ __launch_bounds__(kThreads) void topk_commit_kernel(UnmaskParams p) {
  // Ranking key of each position: (bits of conf) << 32 | (2^32 - 1 - position)
  // for a masked position, 0 otherwise.  conf is positive, so its bits order
  // like its value, and one unsigned 64-bit comparison orders the positions
  // by (conf descending, position ascending); unmasked positions (and the
  // padding to a multiple of 16) never rank ahead of a masked one.
  __shared__ __attribute__((aligned(16))) uint64_t s_key[kUnmaskMaxL];
  __shared__ int s_pred[kUnmaskMaxL];
  __shared__ uint64_t s_bits[kUnmaskMaxL / 64];   // masked flags, 64 positions per word
  __shared__ int s_count[2];   // masked positions, masked positions with conf > gamma

  const int b = blockIdx.x;
  const int L = p.L;
  const int L16 = (L + 15) >> 4;
  const int tid = threadIdx.x;
  const size_t row0 = (size_t)b * L;
  if (tid < 2) s_count[tid] = 0;
  for (int l = L + tid; l < 16 * L16; l += kThreads) s_key[l] = 0;

  // Merge: one thread per position combines the position's chunk triples,
  // 16 at a time: the batch maximum first, then the lowest id attaining it
  // and the sum rescaled once to it (independent exponentials, a fixed
  // order).  The first batch is loaded together with the mask flag (the
  // workspace holds a slot for every position; an unmasked position's slot is
  // loaded and ignored).  Every mask flag of the sequence is read before any
  // is written, so mask_out may alias mask_state.
  constexpr int kMergeBatch = 16;
  int my_masked = 0, my_above = 0;
  for (int l = tid; l < L; l += kThreads) {
    uint64_t key = 0;
    int pred = -1;
    const VocabPartial* pp = p.partials + (row0 + l) * (size_t)p.n_chunks;
    VocabPartial q[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
      if (i < p.n_chunks) q[i] = pp[i];
    if (p.mask_state[row0 + l] != 0) {
      Triple t{-INFINITY, INT_MAX, 0.0f};
      for (int c0 = 0; c0 < p.n_chunks; c0 += kMergeBatch) {
        if (c0 > 0) {
#pragma unroll
          for (int i = 0; i < kMergeBatch; ++i)
            if (c0 + i < p.n_chunks) q[i] = pp[c0 + i];
        }
        const int nb = min(kMergeBatch, p.n_chunks - c0);
        float bm = -INFINITY;
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i)
          if (i < nb) bm = fmaxf(bm, q[i].m);
        int barg = INT_MAX;
        float bs = 0.0f;
        if (bm != -INFINITY) {
#pragma unroll
          for (int i = 0; i < kMergeBatch; ++i) {
            if (i < nb && q[i].m != -INFINITY) {
              bs += q[i].s * __builtin_amdgcn_exp2f((q[i].m - bm) * kLog2e);
              if (q[i].m == bm) barg = min(barg, q[i].arg);
            }
          }
        }
        t = combine(t, Triple{bm, barg, bs});
      }
      const float conf = 1.0f / t.s;
      key = ((uint64_t)__float_as_uint(conf) << 32) | (uint64_t)(0xffffffffu - (uint32_t)l);
      pred = t.arg;
      ++my_masked;
      my_above += conf > p.gamma ? 1 : 0;
    }
    s_key[l] = key;
    s_pred[l] = pred;
  }
  __syncthreads();
  if (p.mode == kSelThreshold || p.mode == kSelSchedule) {
    if (my_masked) atomicAdd(&s_count[0], my_masked);
    if (my_above) atomicAdd(&s_count[1], my_above);
  }
  const bool leftmost = p.mode == kSelLeftmost;
  if (leftmost) {
    // Masked flags as bit words (each wave covers 64 positions at a time).
    const int lane = tid & 63, wave = tid >> 6;
    for (int w = wave; w < (L + 63) / 64; w += kThreads / 64) {
      const int l = 64 * w + lane;
      const unsigned long long bal = __ballot(l < L && s_key[l] != 0);
      if (lane == 0) s_bits[w] = bal;
    }
  }
  __syncthreads();

  // Number of positions this sequence commits.
  int k = p.k;
  if (p.mode == kSelThreshold) {
    const int n = s_count[0];
    k = min(n, max(s_count[1], (n + p.steps_left - 1) / p.steps_left));
  } else if (p.mode == kSelSchedule) {
    const long long keep = (long long)L * (p.n_steps - p.step) / p.n_steps;
    k = (int)max(0LL, (long long)s_count[0] - keep);
  }

  // rank(l) = #{j : key_j > key_l} (or, mock-autoregressive, the masked
  // positions before l); commit when rank < k.  Every lane reads the same LDS
  // words (broadcast), 16 keys per iteration.
  typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
  const u64x2* k2 = reinterpret_cast<const u64x2*>(s_key);
  for (int l = tid; l < L; l += kThreads) {
    const size_t row = row0 + l;
    const uint64_t kl = s_key[l];
    const bool masked = kl != 0;
    int ahead = 0;
    if (masked && k > 0 && leftmost) {
      const int w = l >> 6;
      for (int i = 0; i < w; ++i) ahead += __popcll(s_bits[i]);
      ahead += __popcll(s_bits[w] & ((1ull << (l & 63)) - 1ull));
    } else if (masked && k > 0) {
      for (int j16 = 0; j16 < L16; ++j16) {
        u64x2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = k2[8 * j16 + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) ahead += (v[u].x > kl ? 1 : 0) + (v[u].y > kl ? 1 : 0);
      }
    }
    const bool commit = masked && ahead < k;
    const float c = __uint_as_float((uint32_t)(kl >> 32));
    if (commit) p.tokens_out[row] = s_pred[l];
    p.mask_out[row] = (masked && !commit) ? 1 : 0;
    if (p.conf_out) p.conf_out[row] = masked ? c : -1.0f;
    if (p.pred_out) p.pred_out[row] = s_pred[l];
  }
}

}  // namespace

hipError_t launch_vocab_reduce(const UnmaskParams& p, hipStream_t stream) {
  const long long n = (long long)p.B * p.L * p.n_chunks;
  if (n <= 0 || n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const bool vec = (p.V % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.logits) & 15) == 0);
  if (p.chunk == kVocabChunk) {
    if (vec)
      hipLaunchKernelGGL((vocab_reduce_kernel<true, kVocabChunk>), dim3((unsigned)n), dim3(kThreads),
                         0, stream, p);
    else
      hipLaunchKernelGGL((vocab_reduce_kernel<false, kVocabChunk>), dim3((unsigned)n),
                         dim3(kThreads), 0, stream, p);
  } else if (p.chunk == kVocabChunkManyRows) {
    if (vec)
      hipLaunchKernelGGL((vocab_reduce_kernel<true, kVocabChunkManyRows>), dim3((unsigned)n),
                         dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((vocab_reduce_kernel<false, kVocabChunkManyRows>), dim3((unsigned)n),
                         dim3(kThreads), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_topk_commit(const UnmaskParams& p, hipStream_t stream) {
  if (p.B <= 0 || p.L > kUnmaskMaxL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(topk_commit_kernel, dim3((unsigned)p.B), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tt
