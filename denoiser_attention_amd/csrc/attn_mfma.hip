// Block attention on bf16 matrix cores (gfx950 MFMA).
//
// Operation: TwoTower paper §2.1 "Bidirectional Attention", Eq. (1).  The
// queries of the noisy block attend, under ONE softmax, over the key sequence
// [context-tower cache rows 0..P-1 ; denoiser block rows 0..L-1]; there is no
// mask inside the block and none inside the prefix, so every query row sees
// all P+L keys.
//
// Work decomposition
//   * Grouped-query packing: the G = Hq/Hkv query heads that read one KV head
//     are contiguous in q[B,Hq,L,D], so the G*L query rows of a (batch, kv
//     head) pair form one contiguous matrix of M = G*L rows.  A workgroup takes
//     128 of those rows (4 waves x 32) and streams the pair's keys once for all
//     of them, so each K/V byte fetched from HBM feeds G*L rows.
//   * Key tiles of 64 rows are fetched with 128-bit global loads into
//     registers, then written to a double-buffered LDS tile: K row-major, V
//     transposed (V^T, with keys permuted inside each 16-key group to match the
//     MFMA operand order below).  One barrier per tile.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held in registers), so
//     that in the accumulator layout each lane owns ONE query row and 16 keys
//     of each 32-key block; the other 16 keys of that row sit in lane ^ 32.
//     Softmax statistics are therefore per lane, with one cross-half exchange
//     for the tile maximum.
//   * Online softmax in base 2 with the scale folded into the exponent.  The
//     running maximum is refreshed lazily: the accumulators are rescaled only
//     when a tile's maximum exceeds the reference by more than 2^8, so
//     unnormalised weights stay below 256 (exact in the final normalisation).
//   * O^T += V^T P^T with the same MFMA: A = V^T from LDS, B = P (bf16) taken
//     straight from the score accumulators, so P never leaves registers.
//   * Optional key-range splitting (split-KV) when there are too few query
//     tiles to fill 256 CUs; each split writes an fp32 partial output and its
//     base-2 log-sum-exp, merged by attn_merge_kernel.
//   * Workgroup ids are remapped so that each XCD (own L2) receives a
//     contiguous range of query tiles of the same (pair, split).
#include "tt_internal.h"

namespace tt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = kAttnMfmaBM;   // 128 packed query rows per workgroup
constexpr int BN = kAttnMfmaBN;   // 64 keys per tile
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the max is refreshed
static_assert(BM == 32 * kWaves, "one 32-row MFMA tile per wave");

template <int D>
struct Lay {
  static constexpr int KS = D + 8;       // K tile row stride, bf16 elements (pad: bank spread)
  static constexpr int VS = BN + 8;      // V^T tile row stride
  static constexpr int K_EL = BN * KS;
  static constexpr int V_EL = D * VS;
  static constexpr int BUF_EL = K_EL + V_EL;
  static constexpr int CH = D / 8;       // 16-byte chunks per K/V row
  static constexpr int DS = D / 16;      // MFMA k-steps over head_dim (16 per step)
  static constexpr int DB = D / 32;      // 32-wide blocks of output columns
  static constexpr int K_PER_THREAD = BN * CH / kThreads;
  static constexpr int V_ITEMS = CH * (BN / 4);   // (d-chunk, 4-key quad) items
  static_assert(BN * CH % kThreads == 0, "K tile chunks must divide evenly");
  static_assert(V_ITEMS <= kThreads, "one V item per thread at most");
};

__device__ __forceinline__ int xcd_remap(int i, int n) {
  // Workgroups are dispatched round-robin over the 8 XCDs.  Map them so that
  // XCD x receives a contiguous range of logical ids.
  const int xcd = i & 7, local = i >> 3;
  const int per = (n + 7) >> 3;
  const int tall = ((n & 7) == 0) ? 8 : (n & 7);
  return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

__device__ __forceinline__ uint32_t half_of(uint32_t w, int hi) {
  return hi ? (w >> 16) : (w & 0xFFFFu);
}

template <int D>
__device__ __forceinline__ const u32x4* key_row(const uint16_t* ctx, const uint16_t* blk,
                                                int j, int P) {
  return reinterpret_cast<const u32x4*>(j < P ? ctx + (size_t)j * D
                                              : blk + (size_t)(j - P) * D);
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void attn_mfma_kernel(AttnParams p, int m_tiles,
                                                             int n_blocks) {
  using L = Lay<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::BUF_EL];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, hh = lane >> 5;

  int logical = xcd_remap(blockIdx.x, n_blocks);
  const int mt = logical % m_tiles;
  logical /= m_tiles;
  const int split = logical % p.splits;
  const int pair = logical / p.splits;       // b * Hkv + kv head
  const int b = pair / p.Hkv, kvh = pair - (pair / p.Hkv) * p.Hkv;

  const int n_keys = p.n_keys, P = p.P;
  const int n_tiles = (n_keys + BN - 1) / BN;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(n_tiles, t_begin + p.tiles_per_split);

  const uint16_t* kc = static_cast<const uint16_t*>(p.k_ctx) + (size_t)pair * p.Pcap * D;
  const uint16_t* vc = static_cast<const uint16_t*>(p.v_ctx) + (size_t)pair * p.Pcap * D;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k_blk) + (size_t)pair * p.L * D;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v_blk) + (size_t)pair * p.L * D;

  // First row of this pair in the flattened [B*Hq*L] row space.
  const size_t row_base = ((size_t)b * p.Hq + (size_t)kvh * p.G) * p.L;
  const int wave_row0 = mt * BM + wave * 32;
  const int r_local = wave_row0 + lr;
  const bool row_ok = r_local < p.M;
  const bool wave_active = wave_row0 < p.M;

  // Q fragments: lane holds row r_local, columns 16s + 8hh .. +7 for every s.
  bf16x8 qf[L::DS];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) +
                                                      (row_base + (row_ok ? r_local : 0)) * D);
#pragma unroll
    for (int s = 0; s < L::DS; ++s) {
      u32x4 v = row_ok ? src[2 * s + hh] : u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Register staging of one K/V tile.
  u32x4 kreg[L::K_PER_THREAD];
  u32x4 vreg[4];

  auto load_tile = [&](int t) {
    const int key0 = t * BN;
#pragma unroll
    for (int i = 0; i < L::K_PER_THREAD; ++i) {
      const int id = tid + i * kThreads;
      const int row = id / L::CH, c = id % L::CH;
      const int j = key0 + row;
      kreg[i] = j < n_keys ? key_row<D>(kc, kb, j, P)[c] : u32x4{0, 0, 0, 0};
    }
    if (tid < L::V_ITEMS) {
      const int c = tid % L::CH, quad = tid / L::CH;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = key0 + 4 * quad + i;
        vreg[i] = j < n_keys ? key_row<D>(vc, vb, j, P)[c] : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* Ks = smem + buf * L::BUF_EL;
    uint16_t* Vt = Ks + L::K_EL;
#pragma unroll
    for (int i = 0; i < L::K_PER_THREAD; ++i) {
      const int id = tid + i * kThreads;
      const int row = id / L::CH, c = id % L::CH;
      *reinterpret_cast<u32x4*>(Ks + row * L::KS + 8 * c) = kreg[i];
    }
    if (tid < L::V_ITEMS) {
      const int c = tid % L::CH, quad = tid / L::CH;
      const int qq = quad & 3;
      // Position of keys 4qq..4qq+3 inside their 16-key group: the MFMA B
      // operand of P holds, for lane half h and element e, the key
      // (e < 4 ? 4h + e : 8 + 4h + e - 4); store V^T in that order.
      const int pos = (quad >> 2) * 16 + (qq & 1) * 8 + (qq >> 1) * 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1, hi = e & 1;
        u32x2 pk;
        pk.x = half_of(vreg[0][w], hi) | (half_of(vreg[1][w], hi) << 16);
        pk.y = half_of(vreg[2][w], hi) | (half_of(vreg[3][w], hi) << 16);
        *reinterpret_cast<u32x2*>(Vt + (8 * c + e) * L::VS + pos) = pk;
      }
    }
  };

  f32x16 oacc[L::DB];
#pragma unroll
  for (int db = 0; db < L::DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;   // reference max (base-2 scaled units)
  float l_run = 0.0f;        // this lane's partial row sum (its 32 keys per tile)
  const float c = p.scale_log2;

  load_tile(t_begin);
  store_tile(0);
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool has_next = t + 1 < t_end;
    if (has_next) load_tile(t + 1);

    if (wave_active) {
      const uint16_t* Ks = smem + buf * L::BUF_EL;
      const uint16_t* Vt = Ks + L::K_EL;

      // S^T = K Q^T for two 32-key blocks.
      f32x16 sacc[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        sacc[kb2] = f32x16{};
        const uint16_t* krow = Ks + (kb2 * 32 + lr) * L::KS + 8 * hh;
#pragma unroll
        for (int s = 0; s < L::DS; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * s);
          sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb2], 0, 0, 0);
        }
      }

      // Scale to base-2 units; mask keys past the end of the sequence.
      const int key0 = t * BN;
      const bool tail = key0 + BN > n_keys;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = sacc[kb2][r] * c;
          if (tail) {
            const int key = key0 + kb2 * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= n_keys) v = -INFINITY;
          }
          sacc[kb2][r] = v;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));

      // Lazy refresh of the reference max (uniform branch over the wave).
      const bool need = mx > m_run + kLazyRescale;
      if (__any(need)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < L::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_run = m_new;
      }

      // P = exp2(S - m) in bf16, straight into MFMA B fragments.
      bf16x8 pf[4];
      float psum = 0.0f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(sacc[kb2][r] - m_run);
          psum += pv;
          pf[kb2 * 2 + (r >> 3)][r & 7] = (__bf16)pv;
        }
      l_run += psum;

      // O^T += V^T P^T.
#pragma unroll
      for (int db = 0; db < L::DB; ++db) {
        const uint16_t* vrow = Vt + (db * 32 + lr) * L::VS + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + 16 * ks);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], oacc[db], 0, 0, 0);
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const size_t grow = row_base + r_local;
  if (p.splits == 1) {
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < L::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = db * 32 + 8 * g + 4 * hh;
        const float o0 = oacc[db][4 * g + 0] * inv, o1 = oacc[db][4 * g + 1] * inv;
        const float o2 = oacc[db][4 * g + 2] * inv, o3 = oacc[db][4 * g + 3] * inv;
        if (OUT_BF16) {
          u32x2 pk;
          pk.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o0) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o1) << 16);
          pk.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o2) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o3) << 16);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + grow * D + col) = pk;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + grow * D + col) =
              f32x4{o0, o1, o2, o3};
        }
      }
  } else {
    const size_t rows_total = (size_t)p.B * p.Hq * p.L;
    const float inv = 1.0f / l_tot;
    float* po = p.part_o + ((size_t)split * rows_total + grow) * D;
#pragma unroll
    for (int db = 0; db < L::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = db * 32 + 8 * g + 4 * hh;
        *reinterpret_cast<f32x4*>(po + col) =
            f32x4{oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                  oacc[db][4 * g + 3] * inv};
      }
    if (hh == 0) p.part_lse[(size_t)split * rows_total + grow] = m_run + __log2f(l_tot);
  }
}

template <int D, bool OUT_BF16>
hipError_t launch_typed(const AttnParams& p, hipStream_t stream) {
  const int m_tiles = (p.M + BM - 1) / BM;
  const long long n = (long long)m_tiles * p.splits * p.B * p.Hkv;
  if (n <= 0 || n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_mfma_kernel<D, OUT_BF16>), dim3((unsigned)n), dim3(kThreads), 0,
                     stream, p, m_tiles, (int)n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams& p, hipStream_t stream) {
  const bool ob = p.out_bf16 && p.splits == 1;
  switch (p.D) {
    case 64: return ob ? launch_typed<64, true>(p, stream) : launch_typed<64, false>(p, stream);
    case 128: return ob ? launch_typed<128, true>(p, stream) : launch_typed<128, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tt
