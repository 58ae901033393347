// Block attention on the vector ALU with wavefront shuffles, and the merge of
// split-KV partial results.
//
// Operation: TwoTower paper §2.1 "Bidirectional Attention", Eq. (1) -- one
// softmax over [cache rows 0..P-1 ; block rows 0..L-1] for every query row.
//
// This kernel serves the shapes the matrix-core kernel does not: fp32 inputs
// (full fp32 arithmetic, no bf16 rounding anywhere), and bf16 inputs with
// fewer than 16 packed query rows per KV head, where an MFMA tile would be
// mostly empty.  It is written for the long-prefix decode regime, where the
// K/V stream from HBM is the bound.
//
//   * One wave per workgroup; its 64 lanes form 4 key groups of 16 lanes.
//     Each group takes every 4th key of the workgroup's key range; lane i of a
//     group holds head_dim/16 consecutive columns of the key, the value and the
//     8 query rows the workgroup owns.
//   * Per key: 8 partial dot products per lane, each reduced over the 16 lanes
//     of the group with xor shuffles (all 16 lanes end with the full score),
//     then an online-softmax update of the row state, all in fp32 base 2.
//   * The four groups' (max, sum, output) states are merged through LDS.
//   * Key-range splits use the same partial format as the MFMA kernel.
#include "tt_internal.h"

namespace tt {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int R = kAttnShufRows;   // query rows per workgroup
constexpr int BNS = kAttnShufBN;   // split granularity in keys

// Load E consecutive elements (fp32 or bf16) as fp32.
template <typename T, int E>
__device__ __forceinline__ void load_slice(const T* src, float (&dst)[E]);

template <>
__device__ __forceinline__ void load_slice<float, 4>(const float* src, float (&dst)[4]) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(src);
  dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
}
template <>
__device__ __forceinline__ void load_slice<float, 8>(const float* src, float (&dst)[8]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(src)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(src)[1];
  dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
  dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
}
template <>
__device__ __forceinline__ void load_slice<float, 16>(const float* src, float (&dst)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 a = reinterpret_cast<const f32x4*>(src)[i];
    dst[4 * i] = a.x; dst[4 * i + 1] = a.y; dst[4 * i + 2] = a.z; dst[4 * i + 3] = a.w;
  }
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
template <>
__device__ __forceinline__ void load_slice<uint16_t, 4>(const uint16_t* src, float (&dst)[4]) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(src);
  dst[0] = bf16_lo(v.x); dst[1] = bf16_hi(v.x); dst[2] = bf16_lo(v.y); dst[3] = bf16_hi(v.y);
}
template <>
__device__ __forceinline__ void load_slice<uint16_t, 8>(const uint16_t* src, float (&dst)[8]) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) { dst[2 * i] = bf16_lo(v[i]); dst[2 * i + 1] = bf16_hi(v[i]); }
}
template <>
__device__ __forceinline__ void load_slice<uint16_t, 16>(const uint16_t* src, float (&dst)[16]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4 v = reinterpret_cast<const u32x4*>(src)[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[8 * h + 2 * i] = bf16_lo(v[i]);
      dst[8 * h + 2 * i + 1] = bf16_hi(v[i]);
    }
  }
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, size_t idx, float v);
template <>
__device__ __forceinline__ void store_out<float>(void* out, size_t idx, float v) {
  static_cast<float*>(out)[idx] = v;
}
template <>
__device__ __forceinline__ void store_out<uint16_t>(void* out, size_t idx, float v) {
  static_cast<uint16_t*>(out)[idx] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

template <int D, typename T, typename TO>
__global__ __launch_bounds__(64) void attn_shuffle_kernel(AttnParams p, int row_tiles) {
  constexpr int E = D / 16;
  __shared__ float s_m[4][R], s_l[4][R];
  __shared__ float s_o[4][R][D];

  const int lane = threadIdx.x;
  const int grp = lane >> 4, li = lane & 15;

  int logical = blockIdx.x;
  const int rt = logical % row_tiles;
  logical /= row_tiles;
  const int split = logical % p.splits;
  const int pair = logical / p.splits;       // item * Hkv + kv head
  const int w = pair / p.Hkv, kvh = pair % p.Hkv;
  const AttnItem it = attn_item(p, w, kvh);

  const int n_keys = it.n_keys, P = it.P;
  const int k_begin = split * p.tiles_per_split * BNS;
  if (k_begin >= n_keys) return;   // this item has fewer splits (whole workgroup)
  const int k_end = min(n_keys, k_begin + p.tiles_per_split * BNS);

  const T* kc = static_cast<const T*>(p.k_ctx) + it.ctx_row0 * D;
  const T* vc = static_cast<const T*>(p.v_ctx) + it.ctx_row0 * D;
  const T* kb = static_cast<const T*>(p.k_blk) + it.blk_row0 * D;
  const T* vb = static_cast<const T*>(p.v_blk) + it.blk_row0 * D;
  const size_t prow_base = ((size_t)w * p.Hkv + kvh) * p.M;   // packed row of row 0
  const int r0 = rt * R;

  // Query slices, pre-multiplied by scale*log2(e) (fp32 arithmetic).
  float q[R][E];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r0 + r < p.M) {
      load_slice<T, E>(static_cast<const T*>(p.q) + (it.q_head0 + attn_row_off(p, r0 + r)) * D +
                           li * E, q[r]);
#pragma unroll
      for (int e = 0; e < E; ++e) q[r][e] *= p.scale_log2;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) q[r][e] = 0.0f;
    }
  }

  float m[R], l[R], o[R][E];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[r][e] = 0.0f;
  }

  for (int j = k_begin + grp; j < k_end; j += 4) {
    float kk[E], vv[E];
    const T* krow = j < P ? kc + (size_t)j * D : kb + (size_t)(j - P) * D;
    const T* vrow = j < P ? vc + (size_t)j * D : vb + (size_t)(j - P) * D;
    load_slice<T, E>(krow + li * E, kk);
    load_slice<T, E>(vrow + li * E, vv);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) s = fmaf(q[r][e], kk[e], s);
      s += __shfl_xor(s, 1, 16);
      s += __shfl_xor(s, 2, 16);
      s += __shfl_xor(s, 4, 16);
      s += __shfl_xor(s, 8, 16);
      const float m_new = fmaxf(m[r], s);
      const float alpha = __builtin_amdgcn_exp2f(m[r] - m_new);
      const float pe = __builtin_amdgcn_exp2f(s - m_new);
      l[r] = fmaf(l[r], alpha, pe);
#pragma unroll
      for (int e = 0; e < E; ++e) o[r][e] = fmaf(o[r][e], alpha, pe * vv[e]);
      m[r] = m_new;
    }
  }

  // Merge the four key groups.
  if (li == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) { s_m[grp][r] = m[r]; s_l[grp][r] = l[r]; }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < E; ++e) s_o[grp][r][li * E + e] = o[r][e];
  __syncthreads();

  const size_t rows_total = (size_t)p.B * p.NB * p.Hq * p.L;
  for (int idx = lane; idx < R * D; idx += 64) {
    const int r = idx / D, d = idx % D;
    if (r0 + r >= p.M) continue;
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g) mx = fmaxf(mx, s_m[g][r]);
    float lt = 0.0f, ot = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (s_m[g][r] == -INFINITY) continue;   // group saw no key
      const float w = __builtin_amdgcn_exp2f(s_m[g][r] - mx);
      lt = fmaf(s_l[g][r], w, lt);
      ot = fmaf(s_o[g][r][d], w, ot);
    }
    const size_t grow = prow_base + r0 + r;
    if (p.splits == 1) {
      store_out<TO>(p.out, (it.q_head0 + attn_row_off(p, r0 + r)) * D + d, ot / lt);
    } else {
      p.part_o[((size_t)split * rows_total + grow) * D + d] = ot / lt;
      if (d == 0) p.part_lse[(size_t)split * rows_total + grow] = mx + __log2f(lt);
    }
  }
}

// Merge split-KV partials: out = sum_s 2^(lse_s - lse) * O_s with
// lse = log2 sum_s 2^lse_s.  One thread per (row, 4 columns).  Loads are
// issued in batches of kMergeBatch independent splits so that their latencies
// overlap; the merge is an online (running max) combination in split order.
constexpr int kMergeBatch = 8;

// Four consecutive output columns of one row, in the output type.
template <typename T>
__device__ __forceinline__ void store_out4(void* out, size_t idx, f32x4 v);
template <>
__device__ __forceinline__ void store_out4<float>(void* out, size_t idx, f32x4 v) {
  *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = v;
}
template <>
__device__ __forceinline__ void store_out4<uint16_t>(void* out, size_t idx, f32x4 v) {
  const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.x) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.y) << 16);
  const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.z) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.w) << 16);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = make_uint2(lo, hi);
}

// One thread per (packed row, 4 columns); rows * D / 4 < 2^32 (checked at
// launch), so the index arithmetic is 32-bit, and D / 4 is a power of two.
template <typename TO>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  const uint32_t rows = (uint32_t)p.B * p.NB * p.Hq * p.L;
  const int gshift = __builtin_ctz((unsigned)(p.D / 4));
  // Workgroups follow the attention kernel's XCD order (contiguous runs of
  // (item, KV head) pairs per XCD), so each XCD merges partials its own L2
  // received.
  const uint32_t gid = (uint32_t)xcd_remap(blockIdx.x, gridDim.x) * 256u + threadIdx.x;
  if (gid >= rows << gshift) return;
  const uint32_t row = gid >> gshift;          // packed row ((item * Hkv + kvh) * M + r)
  const int g = (int)(gid & ((1u << gshift) - 1));
  const int pair = (int)(row / (uint32_t)p.M), r = (int)(row - (uint32_t)pair * p.M);
  const int w = pair / p.Hkv, kvh = pair - w * p.Hkv;
  const AttnItem it = attn_item(p, w, kvh);
  const int n_splits = attn_item_splits(p, it.n_keys);   // splits that hold keys of this item
  float m = -INFINITY, wsum = 0.0f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_splits; s0 += kMergeBatch) {
    float lse[kMergeBatch];
    f32x4 o[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (s0 + i < n_splits) {
        const size_t r2 = (size_t)(s0 + i) * rows + row;
        lse[i] = p.part_lse[r2];
        o[i] = *reinterpret_cast<const f32x4*>(p.part_o + r2 * p.D + 4 * g);
      }
    }
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (s0 + i < n_splits) {
        const float m_new = fmaxf(m, lse[i]);
        const float a = __builtin_amdgcn_exp2f(m - m_new);       // 0 on the first split
        const float wt = __builtin_amdgcn_exp2f(lse[i] - m_new);
        wsum = wsum * a + wt;
        acc = acc * a + wt * o[i];
        m = m_new;
      }
    }
  }
  const float inv = 1.0f / wsum;
  store_out4<TO>(p.out, (it.q_head0 + attn_row_off(p, r)) * p.D + 4 * g, acc * inv);
}

template <int D, typename T, typename TO>
hipError_t launch_shuf(const AttnParams& p, hipStream_t stream) {
  const int row_tiles = (p.M + R - 1) / R;
  const long long n = (long long)row_tiles * p.splits * p.B * p.NB * p.Hkv;
  if (n <= 0 || n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_shuffle_kernel<D, T, TO>), dim3((unsigned)n), dim3(64), 0, stream, p,
                     row_tiles);
  return hipGetLastError();
}

template <typename T, typename TO>
hipError_t launch_shuf_d(const AttnParams& p, hipStream_t stream) {
  switch (p.D) {
    case 64: return launch_shuf<64, T, TO>(p, stream);
    case 128: return launch_shuf<128, T, TO>(p, stream);
    case 256: return launch_shuf<256, T, TO>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_shuffle(const AttnParams& p, int in_bf16, hipStream_t stream) {
  // With splits > 1 the kernel writes fp32 partials and the output type of
  // the kernel itself is irrelevant.
  const bool ob = p.out_bf16 && p.splits == 1;
  if (in_bf16) {
    return ob ? launch_shuf_d<uint16_t, uint16_t>(p, stream)
              : launch_shuf_d<uint16_t, float>(p, stream);
  }
  return launch_shuf_d<float, float>(p, stream);
}

hipError_t launch_attn_merge(const AttnParams& p, hipStream_t stream) {
  const size_t n = (size_t)p.B * p.NB * p.Hq * p.L * (p.D / 4);
  if (n == 0 || n > 0xffffff00ULL) return hipErrorInvalidConfiguration;   // 32-bit indices
  const size_t blocks = (n + 255) / 256;
  if (p.out_bf16) {
    hipLaunchKernelGGL(attn_merge_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       p);
  } else {
    hipLaunchKernelGGL(attn_merge_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace tt
