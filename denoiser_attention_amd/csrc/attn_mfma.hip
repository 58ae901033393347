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
//     128 of them (4 waves x 32) and streams the pair's keys once for all of
//     them: every K/V byte fetched from HBM feeds G*L query rows.
//   * K/V stream: 32-key tiles go straight from global memory into a ring of
//     NS LDS stages with 16-byte direct-to-LDS loads (no register staging, no
//     LDS store instructions); while one tile's V and the next tile's K are
//     read, NS-2 further tiles stream in.
//     Waits are explicit vmcnt counts and raw barriers, so that loads of later
//     stages stay in flight across the barrier.
//   * LDS layout: K and V tiles are row-major with the 16-byte chunks of each
//     row XOR-swizzled by a function of the row, chosen so that both operand
//     read patterns below hit distinct banks.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q in registers): in the
//     accumulator layout each lane owns ONE query row and 16 of the tile's 32
//     keys (the other 16 sit in lane ^ 32), so the softmax statistics are
//     per lane plus one cross-half exchange.
//   * Online softmax in base 2 with the scale folded into the exponent.  The
//     reference maximum is the first tile's row maximum, refreshed lazily:
//     only when some lane's share of a tile's weights sums past 2^8 (so some
//     weight may exceed 256, or overflowed) are the accumulators rescaled to
//     the tile's maximum and that tile's weights formed again.  Unnormalised
//     weights stay at most 256 and the final normalisation makes this exact;
//     the steady state needs no per-tile row maximum.
//   * O^T += V^T P^T with the same MFMA: P (bf16) comes straight from the score
//     accumulators; the V^T operand is read from the row-major V tile with the
//     transposing LDS read ds_read_b64_tr_b16 (each 16-lane group turns a
//     4-key x 16-column block into 16 lanes x 4 keys).
//   * Optional key-range splitting (split-KV) when the query tiles alone
//     cannot fill 256 CUs; each split writes an fp32 partial output and its
//     base-2 log-sum-exp, merged by attn_merge_kernel.
//   * Workgroup ids are remapped so that each XCD (own L2) receives a
//     contiguous range of query tiles of the same (pair, split).
#include <type_traits>

#include "tt_internal.h"

namespace tt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = kAttnMfmaBM;   // 128 packed query rows per workgroup
constexpr int BN = kAttnMfmaBN;   // 32 keys per pipeline stage
constexpr float kLazyLimit = 256.0f;  // a lane's tile weight sum that triggers a rescale
static_assert(BM == 32 * kWaves, "one 32-row MFMA tile per wave");
static_assert(BN == 32, "the score tile is one 32x32 MFMA block");

template <int D>
struct Lay {
  static constexpr int CH = D / 8;           // 16-byte chunks per K/V row
  static constexpr int ROWB = D * 2;         // bytes per K/V row
  static constexpr int TILE_B = BN * ROWB;   // one K (or V) tile
  static constexpr int STAGE_B = 2 * TILE_B; // K tile then V tile
  static constexpr int DS = D / 16;          // MFMA k-steps over head_dim
  static constexpr int DB = D / 32;          // 32-wide blocks of output columns
  // Swizzle: chunk c of row r lives in slot c ^ f(r).
  // K is read as 16 rows x one chunk per 16 lanes: f_k spreads 16 rows over all banks.
  __device__ static int fk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  // V is read by the transposing load as 4 rows x 32 bytes per 16 lanes.
  __device__ static int fv(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier without the memory fence of __syncthreads (which would
// also drain the loads that must stay in flight).  The memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// One 16-byte direct-to-LDS load per lane: lane i's 16 bytes land at LDS byte
// address lds + 16*i (lds is the same for the whole wave and goes in M0).  It
// is issued from asm so that the compiler, which cannot tell these writes
// apart from later LDS reads, does not drain them before every LDS read; the
// explicit vmcnt waits and barriers below order them instead.  The asm has no
// register outputs.
__device__ __forceinline__ void dma16(const char* g, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// The same load with a wave-uniform 64-bit base in SGPRs and a per-lane
// 32-bit byte offset.
__device__ __forceinline__ void dma16_s(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// Both forms with the non-temporal hint, for K/V tiles that few workgroups
// read (a stream rather than a shared working set).
__device__ __forceinline__ void dma16_nt(const char* g, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma16_s_nt(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// Maximum of x over lanes l and l ^ 32, for every lane l.  v_permlane32_swap
// exchanges the two 32-lane halves between its two results, so together they
// hold both halves' values for each lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Marks a register value as used (forces its load to complete here).
__device__ __forceinline__ void consume(bf16x8 v) { asm volatile("" ::"v"(v)); }

template <int PER_TILE, int NS>
__device__ __forceinline__ void wait_tiles(int n_after) {
  constexpr int per = PER_TILE;
  static_assert(NS >= 3 && NS - 3 <= 3, "ring depth outside the waits below");
  switch (n_after) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<per>(); break;
    case 2: wait_vmcnt<2 * per>(); break;
    default: wait_vmcnt<3 * per>(); break;
  }
}

// KG = 1: a workgroup is one group of 4 waves (128 query rows) streaming the
// workgroup's key range.  KG = 2: two such groups share the same 128 rows and
// split the key range between them (group 0 the leading floor(n/2) tiles,
// group 1 the trailing ceil(n/2)), each with its own LDS ring; their partial
// softmax states are merged through LDS at the end.  KG = 2 supplies key-range
// parallelism without writing split partials to memory.
//
// RB = 1: each wave owns 32 query rows (128 per group), two waves per SIMD.
// RB = 2 (KG = 1 only): each wave owns 64 rows as two 32-row blocks that
// share every K and V fragment read from LDS (two MFMAs per fragment, two
// independent score chains), halving the LDS traffic, the tile loads and the
// barriers per unit of matrix work; one wave per SIMD, with the output
// accumulators in the accumulation registers.
// RG = 2 (KG = 1, RB = 1 only): eight waves (256 query rows) share one ring, so
// each K/V tile fetched into LDS feeds twice the matrix work: half the
// global-to-LDS traffic, load instructions and LDS writes per unit of work.
// One such workgroup per CU (two waves per SIMD).
// NT_LOADS: the K/V tile loads carry the non-temporal hint.  The launch plan
// sets it when at most 4 query-tile workgroups read each tile, where the tiles
// are a stream rather than a working set shared through L2.
template <int D, int NS, int KG, int RB, int RG, bool OUT_BF16, bool POS_SCALE, bool NT_LOADS>
__global__ __launch_bounds__(kThreads * KG * RG, RB == 2 ? 1 : 2 / (KG * RG))
void attn_mfma_kernel(AttnParams p, int m_tiles, int n_blocks) {
  using L = Lay<D>;
  static_assert(RB == 1 || (RB == 2 && KG == 1), "64-row waves use one key group");
  static_assert(RG == 1 || (RG == 2 && KG == 1 && RB == 1), "shared streams use one key group");
  constexpr int NW = kWaves * RG;         // waves sharing one ring
  constexpr int NT = 64 * NW;             // threads filling one ring
  constexpr int LOADS = L::CH * BN / NT;  // 16-byte loads per thread per tile (K or V)
  static_assert(L::CH * BN % NT == 0 && LOADS >= 1, "tile chunks must divide evenly");
  constexpr int WBM = 32 * RB * NW;       // packed query rows per group
  constexpr int RING_B = KG * NS * L::STAGE_B;
  constexpr int STAGE_OUT_B = NW * 32 * D * 4;   // fp32 output staging (RG = 2)
  __shared__ __attribute__((aligned(1024))) char smem_all[RG == 2 && STAGE_OUT_B > RING_B ? STAGE_OUT_B : RING_B];

  const int gtid = threadIdx.x;
  const int kgrp = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane(gtid >> 8);  // key group
  const int tid = KG == 1 ? gtid : gtid & (kThreads - 1);   // thread index within the group
  char* const smem = smem_all + kgrp * NS * L::STAGE_B;     // this group's ring
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave within the group
  const int lr = lane & 31, hh = lane >> 5;     // MFMA row/column lane, lane half
  const int grp = lane >> 4, gi = lane & 15;    // 16-lane group, index in group

  // Items of the multi-block pass differ in length: they are taken longest
  // first and spread over all XCDs instead of grouped per XCD.
  int logical = p.prefix_mode == 2 ? (int)blockIdx.x : xcd_remap(blockIdx.x, n_blocks);
  const int mt = logical % m_tiles;
  logical /= m_tiles;
  const int split = logical % p.splits;
  const int pair = logical / p.splits;       // item * Hkv + kv head
  int w = pair / p.Hkv;
  const int kvh = pair - w * p.Hkv;
  if (p.prefix_mode == 2) {
    const int bb = w / p.NB;
    w = bb * p.NB + (p.NB - 1 - (w - bb * p.NB));
  }
  const AttnItem it = attn_item(p, w, kvh);

  const int n_keys = it.n_keys, P = it.P;
  const int n_tiles = (n_keys + BN - 1) / BN;
  const int wg_begin = split * p.tiles_per_split;
  if (wg_begin >= n_tiles) return;   // this item has fewer splits (whole workgroup)
  const int wg_end = min(n_tiles, wg_begin + p.tiles_per_split);
  const int wg_n = wg_end - wg_begin;
  const int n_lead = KG == 1 ? 0 : wg_n / 2;        // tiles of group 0 when KG == 2
  const int t_begin = kgrp == 0 ? wg_begin : wg_begin + n_lead;
  const int t_end = KG == 1 ? wg_end : (kgrp == 0 ? wg_begin + n_lead : wg_end);
  const int cnt = t_end - t_begin;                  // this group's tiles (may be 0)
  const int nit = wg_n - n_lead;                    // iterations, equal for every group

  const char* kc = static_cast<const char*>(p.k_ctx) + it.ctx_row0 * L::ROWB;
  const char* vc = static_cast<const char*>(p.v_ctx) + it.ctx_row0 * L::ROWB;
  const char* kb = static_cast<const char*>(p.k_blk) + it.blk_row0 * L::ROWB;
  const char* vb = static_cast<const char*>(p.v_blk) + it.blk_row0 * L::ROWB;

  // Packed row index of this (item, kv head)'s row 0 (split partials).
  const size_t prow_base = ((size_t)w * p.Hkv + kvh) * p.M;
  const int wave_row0 = mt * WBM + wave * 32 * RB;
  const bool wave_active = wave_row0 < p.M;

  // Q fragments: for row block rb the lane holds row wave_row0 + 32*rb + lr,
  // columns 16s + 8hh .. +7 for every s.
  bf16x8 qf[RB][L::DS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r_local = wave_row0 + 32 * rb + lr;
    const bool row_ok = r_local < p.M;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(p.q) + (it.q_head0 + attn_row_off(p, row_ok ? r_local : 0)) * D);
#pragma unroll
    for (int s = 0; s < L::DS; ++s) {
      const u32x4 v = row_ok ? src[2 * s + hh] : u32x4{0, 0, 0, 0};
      qf[rb][s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // LDS byte address of the ring.
  const uint32_t smem_u32 = (uint32_t)(uintptr_t)(lds_char*)smem;

  // Direct-to-LDS loads of tile t into ring slot `slot`.  Thread tid fills
  // 16-byte slot i*256 + tid of each K and V tile: row r_i, slot column q_i,
  // holding global chunk q_i ^ f(r_i).  A tile lying wholly in the cache or
  // wholly in the block uses a uniform base and per-thread constant offsets;
  // the tile that straddles the two (or runs past the end) computes each row's
  // address, with rows past the end loading the last valid row (their scores
  // are masked).
  uint32_t koff[LOADS], voff[LOADS];
  int rrow[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int s = i * NT + tid;
    const int r = s / L::CH, q = s % L::CH;
    rrow[i] = r;
    koff[i] = r * L::ROWB + ((q ^ L::fk(r)) << 4);
    voff[i] = r * L::ROWB + ((q ^ L::fv(r)) << 4);
  }
  auto issue = [&](int t, auto slot) {
    const uint32_t kst = smem_u32 + slot * L::STAGE_B;
    const uint32_t vst = kst + L::TILE_B;
    const int key0 = t * BN;
    const bool in_prefix = key0 + BN <= P;
    const bool in_block = key0 >= P && key0 + BN <= n_keys;
    if (__builtin_expect(in_prefix || in_block, 1)) {
      // A tile wholly in the cache or wholly in the block (every tile but
      // the one straddling the two and a ragged last one): one uniform base,
      // chosen without a branch.
      const char* kbase = in_prefix ? kc + (size_t)key0 * L::ROWB : kb + (size_t)(key0 - P) * L::ROWB;
      const char* vbase = in_prefix ? vc + (size_t)key0 * L::ROWB : vb + (size_t)(key0 - P) * L::ROWB;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const uint32_t wofs = (i * NT + wave * 64) * 16;   // wave-uniform destination
        if constexpr (NT_LOADS) {
          dma16_s_nt(kbase, koff[i], kst + wofs);
          dma16_s_nt(vbase, voff[i], vst + wofs);
        } else {
          dma16_s(kbase, koff[i], kst + wofs);
          dma16_s(vbase, voff[i], vst + wofs);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const uint32_t wofs = (i * NT + wave * 64) * 16;
        const int j = min(key0 + rrow[i], n_keys - 1);
        const size_t rel = (size_t)rrow[i] * L::ROWB;
        const char* krow = j < P ? kc + (size_t)j * L::ROWB : kb + (size_t)(j - P) * L::ROWB;
        const char* vrow = j < P ? vc + (size_t)j * L::ROWB : vb + (size_t)(j - P) * L::ROWB;
        dma16(krow + (koff[i] - rel), kst + wofs);
        dma16(vrow + (voff[i] - rel), vst + wofs);
      }
    }
  };

  // Per-lane LDS offsets.  K operand: row lr, chunk 2s + hh.
  const int k_row_off = lr * L::ROWB;
  const int fkl = L::fk(lr);
  // V^T operand through the transposing read: as a source lane of its 16-lane
  // group this lane points at V[k0 + gi/4][d0 + 4*(gi%4) .. +3], with
  // k0 = 4*(grp/2) (+16 per k-step, +8 for the second half) and
  // d0 = 32*db + 16*(grp%2).
  int vofs[L::DB];
#pragma unroll
  for (int db = 0; db < L::DB; ++db) {
    const int key = 4 * (grp >> 1) + (gi >> 2);
    const int c = 4 * db + 2 * (grp & 1) + ((gi & 3) >> 1);
    vofs[db] = key * L::ROWB + ((c ^ L::fv(gi >> 2)) << 4) + ((gi & 1) << 3);
  }

  f32x16 oacc[RB][L::DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < L::DB; ++db) oacc[rb][db] = f32x16{};
  float m_run[RB], l_run[RB];   // reference max (base-2 scaled units), this lane's row-sum share
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.0f;
  }
  const float c = p.scale_log2;
  typedef f32x16 Scores[RB];

  // S^T = K Q^T over the 32 keys of the tile in ring slot `slot`.
  auto qk = [&](int slot, Scores& sacc) {
    const char* Ks = smem + slot * L::STAGE_B;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sacc[rb] = f32x16{};
#pragma unroll
    for (int s = 0; s < L::DS; ++s) {
      const bf16x8 a =
          *reinterpret_cast<const bf16x8*>(Ks + k_row_off + (((2 * s + hh) ^ fkl) << 4));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        sacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[rb][s], sacc[rb], 0, 0, 0);
    }
  };

  // c * the row maximum of the scores `sc` of tile t (both lanes of a row hold
  // the same value): the first tile's sets the reference maximum, later ones
  // are formed only when a rescale is due.
  float mx_pend[RB];
  auto tile_max = [&](auto tail_tag, const Scores& sc, int t) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int key0 = t * BN;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mraw = POS_SCALE ? -INFINITY : INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = !TAIL || key0 + 8 * (r >> 2) + 4 * hh + (r & 3) < n_keys;
        const float v = ok ? sc[rb][r] : (POS_SCALE ? -INFINITY : INFINITY);
        mraw = POS_SCALE ? fmaxf(mraw, v) : fminf(mraw, v);
      }
      mx_pend[rb] = pair_max(mraw * c);
    }
  };

  // Online softmax of tile t's scores `sacc`, with the scores of the next
  // tile (K fragments kf, when DO_QK) computed in between: one MFMA of the
  // next tile's chain per slice of this tile's exponentials, so that the
  // matrix core and the vector ALU work at the same time.  The weights are
  // formed against the current reference maximum; when some lane's share of
  // a row's weights sums past kLazyLimit (a uniform branch, rarely taken
  // after the first tile), the accumulators are rescaled to the tile's
  // maximum and the weights formed again.  Produces the bf16 P fragments and
  // this lane's share of the tile's row sums.  The TAIL instantiation masks
  // the keys past the end of the sequence (only the last tile can need it).
  auto qk_softmax = [&](auto do_qk_tag, auto tail_tag, const Scores& sacc, int t,
                        const bf16x8 (&kf)[L::DS], const char* Ks, bf16x8 (&pf)[RB][2],
                        float (&tsum)[RB], Scores& snext) {
    constexpr bool DO_QK = decltype(do_qk_tag)::value;
    constexpr bool TAIL = decltype(tail_tag)::value;
    // Accumulator register r holds key 8*(r/4) + 4*hh + r%4 of the tile.
    const int key0 = t * BN;
    auto valid = [&](int r) { return !TAIL || key0 + 8 * (r >> 2) + 4 * hh + (r & 3) < n_keys; };
    // P = exp2(S*c - m) rounded to bf16, straight into MFMA B fragments; the
    // row sum adds exactly the bf16 weights that enter P.V (packed dot with 1).
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
    auto weights = [&](int rb, int r) {
      float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[rb][r], c, -m_run[rb]));
      float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[rb][r + 1], c, -m_run[rb]));
      if (!valid(r)) p0 = 0.0f;
      if (!valid(r + 1)) p1 = 0.0f;
      const bf16x2 pk = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
      pf[rb][r >> 3][r & 7] = pk[0];
      pf[rb][r >> 3][(r & 7) + 1] = pk[1];
      tsum[rb] = __builtin_amdgcn_fdot2_f32_bf16(pk, one2, tsum[rb], false);
    };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      snext[rb] = f32x16{};
      tsum[rb] = 0.0f;
    }
    constexpr int PER = 16 / L::DS;   // score registers per MFMA slice
#pragma unroll
    for (int s = 0; s < L::DS; ++s) {
      // 32-row waves take the K fragments read up front; 64-row waves read
      // each one just before its two MFMAs (fewer live registers).
      bf16x8 ks_frag;
      if (DO_QK)
        ks_frag = RB == 1 ? kf[s]
                          : *reinterpret_cast<const bf16x8*>(Ks + k_row_off + (((2 * s + hh) ^ fkl) << 4));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (DO_QK) snext[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ks_frag, qf[rb][s], snext[rb], 0, 0, 0);
#pragma unroll
        for (int r = s * PER; r < (s + 1) * PER; r += 2) weights(rb, r);
      }
    }
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) grow = grow || tsum[rb] > kLazyLimit;
    if (__builtin_expect(__any(grow), 0)) {
      tile_max(tail_tag, sacc, t);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float m_new = fmaxf(m_run[rb], mx_pend[rb]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < L::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[rb][db][r] *= alpha;
        m_run[rb] = m_new;
        tsum[rb] = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) weights(rb, r);
      }
    }
  };

  // Add the tile's row sums and O^T += V^T P^T for the tile in ring slot
  // `slot`: two 16-key k-steps per 32-wide block of output columns, each V^T
  // fragment shared by the row blocks.  Element j of the V^T operand of k-step
  // ks is key 16*ks + (j < 4 ? 4*hh + j : 8 + 4*hh + j - 4): the first
  // transposing read covers j < 4, the second (8 rows further) j >= 4.
  auto finish_pv = [&](const bf16x8 (&pf)[RB][2], const float (&tsum)[RB], int slot) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) l_run[rb] += tsum[rb];
    const char* Vs = smem + slot * L::STAGE_B + L::TILE_B;
    // With one key group, the two waves on a SIMD belong to different
    // workgroups and drift independently: the wave entering its MFMA-only
    // P.V run takes issue priority, so the matrix pipe stays fed while the
    // other wave's softmax fills the gaps (3-4% at the high-batch workload).
    if (KG == 1) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < L::DB; ++db) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const lds_char* vp = (const lds_char*)(Vs + vofs[db] + ks * 16 * L::ROWB);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 8 * L::ROWB));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[rb][ks], oacc[rb][db], 0, 0, 0);
      }
    }
    if (KG == 1) __builtin_amdgcn_s_setprio(0);
  };

  // Software pipeline over the key tiles: while the vector units run the
  // softmax of tile t, the matrix cores already compute the scores of tile
  // t + 1.  Ring occupancy during iteration t: tile t (its V is read), tile t+1
  // (its K is read), tiles t+2 .. t+NS-2 in flight; tile t+NS-1 is issued into
  // the slot of tile t-1, which every wave has finished with once it passes
  // the barrier of iteration t.
  static_assert((NS & (NS - 1)) == 0, "ring depth must be a power of two");
  // Iteration index i of a group refers to its tile t_begin + i.
  auto slot_of = [&](int i) { return i & (NS - 1); };
  // Wait until the group's tile i has landed for every wave, then refill the
  // slot of tile i-2 with tile i+NS-2.  Every wave of the workgroup runs the
  // same number of these (and so of barriers), also past the end of its
  // group's tiles.
  auto advance = [&](int i) {
    wait_tiles<2 * LOADS, NS>(max(0, min(NS - 3, cnt - 1 - i)));
    barrier();
    if (i + NS - 2 < cnt) issue(t_begin + i + NS - 2, slot_of(i + NS - 2));
  };
  // The same where the caller guarantees that tile i + NS - 2 exists for
  // this group (so NS - 3 tiles are still in flight behind tile i), with the
  // refilled slot a compile-time constant: no branch and no runtime wait
  // count in the steady state.
  auto advance_steady = [&](int i, auto slot) {
    wait_vmcnt<2 * LOADS * (NS - 3)>();
    barrier();
    issue(t_begin + i + NS - 2, slot);
  };
  // Tile i (in ring slot `slot`): softmax and P.V, with the scores of tile
  // i+1 when DO_QK.  `slot` is an int or, in the loop unrolled by the ring
  // depth, a compile-time constant, so that the slot offsets fold into the
  // LDS reads' immediate offsets.
  auto step = [&](auto do_qk_tag, auto tail_tag, int i, const Scores& s_in, Scores& s_out,
                  auto slot) {
    constexpr bool DO_QK = decltype(do_qk_tag)::value;
    const int v_slot = slot;
    const int k_slot = (v_slot + 1) & (NS - 1);
    bf16x8 kf[L::DS];
    const char* Ks = smem + k_slot * L::STAGE_B;
    if (DO_QK && RB == 1) {
#pragma unroll
      for (int s = 0; s < L::DS; ++s)
        kf[s] = *reinterpret_cast<const bf16x8*>(Ks + k_row_off + (((2 * s + hh) ^ fkl) << 4));
    }
    bf16x8 pf[RB][2];
    float tsum[RB];
    qk_softmax(do_qk_tag, tail_tag, s_in, t_begin + i, kf, Ks, pf, tsum, s_out);
    finish_pv(pf, tsum, v_slot);
  };
  const std::true_type yes{};
  const std::false_type no{};
#pragma unroll
  for (int s = 0; s < NS - 2; ++s)
    if (s < cnt) issue(t_begin + s, s);
  // The Q loads (issued first) and the first K/V tiles are now all in flight.
  // Consuming Q here makes its (conservative, full) load wait overlap the K/V
  // latency and keeps it out of the pipelined loop.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int s = 0; s < L::DS; ++s) consume(qf[rb][s]);
  // Waves whose rows all lie past M run the same instruction stream on zero Q
  // rows (no branch in the loop) and store nothing.
  advance(0);
  Scores s_a, s_b;
  if (cnt > 0) {
    qk(slot_of(0), s_a);
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s_a[rb] = f32x16{};
  }
  // The first tile's row maximum is the reference maximum (finite: the tile
  // holds at least one key; a group without tiles takes its zero scores).
  if ((t_begin + 1) * BN > n_keys)
    tile_max(yes, s_a, t_begin);
  else
    tile_max(no, s_a, t_begin);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) m_run[rb] = mx_pend[rb];
  // Steady state, unrolled by two so that the score registers alternate
  // instead of being copied: both groups have tiles i and i+1 (group 0 has at
  // least nit - 1 tiles).
  int i = 0;
  if constexpr (NS == 4) {
    // Unrolled by the ring depth: i stays a multiple of 4, so tile i + j
    // lives in slot j.
    // i + 7 < nit: tiles up to i + 6 exist for both key groups (group 0 has
    // at least nit - 1 tiles), so every refill of this loop is unconditional.
    static_assert(NS == 4, "the steady-state slots below assume a 4-deep ring");
    for (; i + 7 < nit; i += 4) {
      advance_steady(i + 1, std::integral_constant<int, 3>{});
      step(yes, no, i, s_a, s_b, std::integral_constant<int, 0>{});
      advance_steady(i + 2, std::integral_constant<int, 0>{});
      step(yes, no, i + 1, s_b, s_a, std::integral_constant<int, 1>{});
      advance_steady(i + 3, std::integral_constant<int, 1>{});
      step(yes, no, i + 2, s_a, s_b, std::integral_constant<int, 2>{});
      advance_steady(i + 4, std::integral_constant<int, 2>{});
      step(yes, no, i + 3, s_b, s_a, std::integral_constant<int, 3>{});
    }
  }
  for (; i + 3 < nit; i += 2) {
    advance(i + 1);
    step(yes, no, i, s_a, s_b, slot_of(i));
    advance(i + 2);
    step(yes, no, i + 1, s_b, s_a, slot_of(i + 1));
  }
  if (i + 2 < nit) {
    advance(i + 1);
    step(yes, no, i, s_a, s_b, slot_of(i));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s_a[rb] = s_b[rb];
    ++i;
  }
  if (nit >= 2) {   // tile nit-2; group 0 may lack tile nit-1
    advance(nit - 1);
    if (nit - 1 < cnt)
      step(yes, no, nit - 2, s_a, s_b, slot_of(nit - 2));
    else
      step(no, no, nit - 2, s_a, s_b, slot_of(nit - 2));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s_a[rb] = s_b[rb];
  }
  // Only the last tile of the whole key sequence can run past its end; it is
  // always the group's tile nit-1.
  if (nit - 1 < cnt) {
    if (t_end * BN > n_keys)
      step(no, yes, nit - 1, s_a, s_b, slot_of(nit - 1));
    else
      step(no, no, nit - 1, s_a, s_b, slot_of(nit - 1));
  }

  float l_tot[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) l_tot[rb] = l_run[rb] + __shfl_xor(l_run[rb], 32);
  // Staging tile for the output: each wave writes a normalised 32 x D row
  // block to LDS (fp32, 16-byte chunk c of row r at chunk position c ^ (r & 7),
  // so that both the accumulator-order writes and the row-order reads spread
  // over all banks) and reads it back row by row, so that the global stores
  // cover whole contiguous rows.
  float* stg;
  if (KG == 2) {
    // Merge group 1's (max, sum, O) into group 0 through LDS (the rings are
    // free once every wave is past its last tile).  Lanes of the two groups
    // with the same (wave, lane) hold the same row and columns.
    float* xbuf = reinterpret_cast<float*>(smem_all) + wave * (L::DB * 16 + 2) * 64;
    barrier();
    if (kgrp == 1) {
#pragma unroll
      for (int db = 0; db < L::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xbuf[(db * 16 + r) * 64 + lane] = oacc[0][db][r];
      xbuf[(L::DB * 16) * 64 + lane] = m_run[0];
      xbuf[(L::DB * 16 + 1) * 64 + lane] = l_tot[0];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier();
    if (kgrp == 1) return;
    const float m1 = xbuf[(L::DB * 16) * 64 + lane];
    const float l1 = xbuf[(L::DB * 16 + 1) * 64 + lane];
    const float m_new = fmaxf(m_run[0], m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run[0] - m_new);   // 0 for an empty group
    const float a1 = __builtin_amdgcn_exp2f(m1 - m_new);
#pragma unroll
    for (int db = 0; db < L::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        oacc[0][db][r] = oacc[0][db][r] * a0 + xbuf[(db * 16 + r) * 64 + lane] * a1;
    l_tot[0] = l_tot[0] * a0 + l1 * a1;
    m_run[0] = m_new;
    // This wave alone reads and then rewrites its own exchange area (LDS
    // operations of one wave complete in order).
    stg = xbuf;
  } else {
    barrier();   // every wave is done with the ring
    stg = reinterpret_cast<float*>(smem_all) + wave * 32 * D;
  }
  static_assert(32 * D <= (L::DB * 16 + 2) * 64, "staging tile fits the exchange area");
  static_assert(NW * 32 * D * 4 <= sizeof(smem_all), "staging tiles fit the ring");
  if (!wave_active) return;
  const size_t rows_total = (size_t)p.B * p.NB * p.Hq * p.L;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row0 = wave_row0 + 32 * rb;           // first packed row of this block
    const int rows_here = min(32, p.M - row0);      // valid rows of this block
    if (rows_here <= 0) break;
    const float inv = 1.0f / l_tot[rb];
    // The previous block's row reads are complete before these writes: the
    // same wave's LDS operations complete in order.
#pragma unroll
    for (int db = 0; db < L::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int chunk = db * 8 + 2 * g + hh;
        *reinterpret_cast<f32x4*>(stg + lr * D + ((chunk ^ (lr & 7)) << 2)) =
            f32x4{oacc[rb][db][4 * g] * inv, oacc[rb][db][4 * g + 1] * inv,
                  oacc[rb][db][4 * g + 2] * inv, oacc[rb][db][4 * g + 3] * inv};
      }
    asm volatile("" ::: "memory");
    if (OUT_BF16) {
      // 8 values (16 bytes) per lane, D/8 lanes per row.
      constexpr int LPR = D / 8, RPI = 64 / LPR;
#pragma unroll
      for (int i2 = 0; i2 < 32 / RPI; ++i2) {
        const int row = i2 * RPI + lane / LPR, c8 = lane % LPR;
        const f32x4 a = *reinterpret_cast<const f32x4*>(stg + row * D + (((2 * c8) ^ (row & 7)) << 2));
        const f32x4 bq = *reinterpret_cast<const f32x4*>(stg + row * D + (((2 * c8 + 1) ^ (row & 7)) << 2));
        u32x4 pk;
        pk.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a.x) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a.y) << 16);
        pk.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a.z) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a.w) << 16);
        pk.z = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)bq.x) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)bq.y) << 16);
        pk.w = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)bq.z) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)bq.w) << 16);
        if (row < rows_here) {
          const size_t orow = it.q_head0 + attn_row_off(p, row0 + row);
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + orow * D + 8 * c8) = pk;
        }
      }
    } else {
      // 4 values (16 bytes) per lane, D/4 lanes per row: the final fp32 output,
      // or this split's partial.
      constexpr int LPR = D / 4, RPI = 64 / LPR;
      float* part = p.part_o + ((size_t)split * rows_total + prow_base + row0) * D;
#pragma unroll
      for (int i2 = 0; i2 < 32 / RPI; ++i2) {
        const int row = i2 * RPI + lane / LPR, c4 = lane % LPR;
        const f32x4 v = *reinterpret_cast<const f32x4*>(stg + row * D + ((c4 ^ (row & 7)) << 2));
        if (row < rows_here) {
          float* dst = p.splits == 1
                           ? static_cast<float*>(p.out) + (it.q_head0 + attn_row_off(p, row0 + row)) * D
                           : part + (size_t)row * D;
          *reinterpret_cast<f32x4*>(dst + 4 * c4) = v;
        }
      }
      if (p.splits > 1 && hh == 0 && lr < rows_here)
        p.part_lse[(size_t)split * rows_total + prow_base + row0 + lr] = m_run[rb] + __log2f(l_tot[rb]);
    }
    asm volatile("" ::: "memory");
  }
}

constexpr int kStages = 4;

template <int D, bool OUT_BF16, bool POS>
hipError_t launch_typed(const AttnParams& p, hipStream_t stream) {
  const int rows_wg = (p.rows_per_wave == 64 || p.stream_waves == 8) ? 2 * BM : BM;
  const int m_tiles = (p.M + rows_wg - 1) / rows_wg;
  const long long n = (long long)m_tiles * p.splits * p.B * p.NB * p.Hkv;
  if (n <= 0 || n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // The non-temporal form is built for the 4-wave plans with a non-negative
  // scale (where the streaming shapes run); elsewhere the hint is dropped.
  const bool nt = POS && p.nt_loads != 0;
  if (p.rows_per_wave == 64 || p.stream_waves == 8) {
    if constexpr (D == 128) {
      if (p.kgroups != 1 || (p.rows_per_wave == 64 && p.stream_waves == 8)) return hipErrorInvalidValue;
      if (p.rows_per_wave == 64)
        hipLaunchKernelGGL((attn_mfma_kernel<D, kStages, 1, 2, 1, OUT_BF16, POS, false>),
                           dim3((unsigned)n), dim3(kThreads), 0, stream, p, m_tiles, (int)n);
      else
        hipLaunchKernelGGL((attn_mfma_kernel<D, kStages, 1, 1, 2, OUT_BF16, POS, false>),
                           dim3((unsigned)n), dim3(2 * kThreads), 0, stream, p, m_tiles, (int)n);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (p.kgroups == 2) {
    if (nt)
      hipLaunchKernelGGL((attn_mfma_kernel<D, kStages, 2, 1, 1, OUT_BF16, POS, POS>),
                         dim3((unsigned)n), dim3(2 * kThreads), 0, stream, p, m_tiles, (int)n);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<D, kStages, 2, 1, 1, OUT_BF16, POS, false>),
                         dim3((unsigned)n), dim3(2 * kThreads), 0, stream, p, m_tiles, (int)n);
  } else {
    if (nt)
      hipLaunchKernelGGL((attn_mfma_kernel<D, kStages, 1, 1, 1, OUT_BF16, POS, POS>),
                         dim3((unsigned)n), dim3(kThreads), 0, stream, p, m_tiles, (int)n);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<D, kStages, 1, 1, 1, OUT_BF16, POS, false>),
                         dim3((unsigned)n), dim3(kThreads), 0, stream, p, m_tiles, (int)n);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t stream) {
  const bool ob = p.out_bf16 && p.splits == 1;
  const bool pos = p.scale_log2 >= 0.0f;
  if (ob) return pos ? launch_typed<D, true, true>(p, stream) : launch_typed<D, true, false>(p, stream);
  return pos ? launch_typed<D, false, true>(p, stream) : launch_typed<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams& p, hipStream_t stream) {
  switch (p.D) {
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tt
