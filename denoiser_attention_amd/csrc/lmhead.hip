// Fused LM-head projection and vocabulary statistics of the unmask step.
//
// Operation: TwoTower paper §2.2 "Sampling" / Algorithm 2.  The denoiser's
// distribution at a still-masked position is the softmax of the logits its
// LM head forms from the position's hidden state, logits = hidden . W^T with W
// the [vocab, d_model] projection.  The unmask step needs, per masked
// position, only (max logit, lowest id attaining it, sum of exp(logit - max)),
// so the projection is fused with that reduction and the logits never leave
// the chip.
//
// Kernels
//   lmhead_rows_kernel   -- one workgroup: the masked positions, in order,
//                           and their count (committed positions are never
//                           projected).
//   lmhead_stats_kernel  -- 8-wave workgroups over (256 masked rows,
//                           256-entry vocabulary slice) items: one per CU,
//                           each taking items in turn and requesting the
//                           next item's first tiles under the current one's
//                           last stages and statistics, when the ring
//                           schedule allows it; otherwise one workgroup
//                           per item.  Per item it computes S^T =
//                           W_slice . H^T with v_mfma_f32_32x32x16_bf16 (A =
//                           32 vocabulary rows, B = 32 hidden rows, both read
//                           as 16-byte runs along d_model), so that in the
//                           accumulator layout each lane owns one hidden row
//                           and 16 of a tile's 32 vocabulary entries: the
//                           per-row statistics are formed inside the lane,
//                           then with lane ^ 32, then across the 4 vocabulary
//                           waves of its row half through LDS.  Wave w covers
//                           vocabulary entries 64(w%4)..+63 of the slice
//                           against rows 128(w/4)..+127 (8 accumulator
//                           tiles).  W and H tiles of 64 d_model columns
//                           (whole 128-byte weight lines) stream with 16-byte
//                           direct-to-LDS loads (rows XOR-swizzled at 16-byte
//                           granularity) into a 3-stage weight ring and a
//                           2-stage hidden ring (160 KB, one workgroup per
//                           CU): the weight stream from HBM runs two tiles
//                           ahead, the hidden rows (from L2) one; one barrier
//                           per 64 columns, and each weight tile feeds 256
//                           rows.  A d_model that is an odd multiple of 32
//                           ends with a 32-column stage.
//   lmhead_merge_kernel  -- one wavefront per masked row: merges the row's
//                           slice partials into one.
// The confidence-ranking and commit step then runs on the merged partials.
#include <algorithm>
#include <climits>
#include <type_traits>
#include <utility>

#include "tt_internal.h"

namespace tt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 8;                          // 4 vocabulary ranges x 2 row halves
constexpr int kThreads = 64 * kWaves;
constexpr int NSW = 3;                              // weight ring stages
constexpr int NSH = 2;                              // hidden ring stages
constexpr int KS = 64;                              // d_model columns per stage
constexpr int ROWB = KS * 2;                        // bytes of one row of a stage (128)
constexpr int W_TILE = kLmVocab * ROWB;             // 32 KB
constexpr int H_TILE = kLmRows * ROWB;              // 32 KB
constexpr int W_LOADS = W_TILE / 16 / kThreads;     // 4 direct loads per thread
constexpr int H_LOADS = H_TILE / 16 / kThreads;     // 4
static_assert(W_LOADS == 4 && H_LOADS == 4, "one four-load DMA group per tile and thread");
static_assert(kLmVocab == 64 * 4, "four 64-entry vocabulary ranges per workgroup");
static_assert(kLmRows == 256 && KS == 64, "tile shape");
constexpr int RING = NSW * W_TILE + NSH * H_TILE;   // 160 KB: one workgroup per CU
static_assert(RING <= 160 * 1024, "rings fit the LDS");

// Chunk q (16 bytes) of stage row r lives in slot q ^ f(r).  A 16-byte LDS
// read is served 16 lanes (256 bytes) at a time; those lanes read 16
// consecutive 128-byte rows at the same chunk, which f spreads over all 16
// 16-byte bank groups (rows r and r + 1 differ in their 128-byte base, pairs
// of rows in f).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

struct Triple {
  float m;
  int arg;
  float s;
};

__device__ __forceinline__ Triple combine(Triple a, Triple b) {
  Triple r;
  r.m = fmaxf(a.m, b.m);
  const float sa = a.m == -INFINITY ? 0.0f : a.s * __builtin_amdgcn_exp2f((a.m - r.m) * kLog2e);
  const float sb = b.m == -INFINITY ? 0.0f : b.s * __builtin_amdgcn_exp2f((b.m - r.m) * kLog2e);
  r.s = sa + sb;
  r.arg = a.m > b.m ? a.arg : (b.m > a.m ? b.arg : min(a.arg, b.arg));
  return r;
}

__device__ __forceinline__ Triple shfl_xor_triple(Triple t, int mask) {
  return Triple{__shfl_xor(t.m, mask), __shfl_xor(t.arg, mask), __shfl_xor(t.s, mask)};
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier that leaves outstanding loads in flight (unlike
// __syncthreads, which also drains them).
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Four 16-byte direct-to-LDS loads per lane from one wave-uniform base: load
// j adds per-lane offset off[j], and lane i's bytes land at LDS address
// lds[j] + 16*i.  Issued from asm (no register outputs) so that the compiler
// does not drain them before unrelated LDS reads; the explicit vmcnt waits
// and barriers order them.  The compiler cannot see the asm's operands when
// it inserts hazard wait states: a vector instruction that wrote the scalar
// base (a spill reload, a readfirstlane) needs 5 wait states before a memory
// instruction reads it, given by the leading s_nop; M0 written by a scalar
// instruction needs one before a load into LDS reads it.  M0 is restored on
// the way out (the compiler does not expect an asm statement to change it).
__device__ __forceinline__ void dma16x4_s(const char* base, const uint32_t (&off)[4],
                                          const uint32_t (&lds)[4]) {
  uint32_t saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %9\n\t"
      "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %9\n\t"
      "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %9\n\t"
      "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %9\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(lds[0]), "s"(lds[1]),
        "s"(lds[2]), "s"(lds[3]), "s"(base)
      : "memory");
}

__global__ __launch_bounds__(1024) void lmhead_rows_kernel(LmParams p) {
  __shared__ int s_wave[16];
  __shared__ int s_base;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int i0 = 0; i0 < p.n_pos; i0 += 1024) {
    const int i = i0 + tid;
    const bool f = i < p.n_pos && p.mask_state[i] != 0;
    const unsigned long long bal = __ballot(f);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    int off = s_base;
    for (int w = 0; w < wave; ++w) off += s_wave[w];
    if (f) p.row_ids[off + below] = i;
    __syncthreads();
    if (tid == 0) {
      int t = 0;
      for (int w = 0; w < 16; ++w) t += s_wave[w];
      s_base += t;
    }
    __syncthreads();
  }
  if (tid == 0) *p.n_rows = s_base;
}

// A pointer every lane holds the same value of, moved to scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* q) {
  const uint64_t u = (uint64_t)(uintptr_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const char*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

// One (row tile, vocabulary slice) item: values every lane shares.
struct LmItem {
  const char* wbase;          // weight row vocab0, column 0
  int rt, slice, vocab0, rows_here;
};

// Persistent workgroups: workgroup lw takes items lw, lw + G, lw + 2G, ...
// of the n_rt x n_slices (row tile, vocabulary slice) items, item i being row
// tile i % n_rt of slice i / n_rt (n_rt from the masked-row count the rows
// kernel left).  Consecutive items on one XCD share a weight slice.  When
// the ring schedule wraps to slot 0 at an item boundary (a d_model that is a
// multiple of 6 x 64 columns), the next item's first tiles are requested
// during the current item's last two stages, so they stream in under its last
// matrix work and its statistics.
__global__ __launch_bounds__(kThreads, 1) void lmhead_stats_kernel(LmParams p) {
  __shared__ __attribute__((aligned(1024))) char ring[RING];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int vw = wave & 3, rw = wave >> 2;         // vocabulary range, row half
  const int G = gridDim.x;
  const int lw = xcd_remap(blockIdx.x, G);
  const int n_rows = *p.n_rows;
  const int n_rt = (n_rows + kLmRows - 1) / kLmRows;
  const int total = n_rt * p.n_slices;
  if (lw >= total) return;                         // whole workgroup
  const int d = p.d;
  const size_t rowb = (size_t)d * 2;

  // Thread tid fills 16-byte slot i = tid + kThreads*j of each stage (row
  // r = i / 8, slot q = i % 8), holding the row's global chunk q ^ swz(r).
  // Since kThreads / 8 is a multiple of 16, that chunk, qc, is the same for
  // every j; lo_half: it lies in the first 32 columns of the stage.
  const int qc = (tid & 7) ^ swz(tid >> 3);
  const bool lo_half = qc < 4;
  const char* hbase = static_cast<const char*>(p.hidden);
  const uint32_t ring_u32 = (uint32_t)(uintptr_t)(lds_char*)ring;

  auto set_item = [&](int item, LmItem& it) {
    it.rt = item % n_rt;
    it.slice = item / n_rt;
    it.vocab0 = it.slice * kLmVocab;
    it.rows_here = min(kLmRows, n_rows - it.rt * kLmRows);
    it.wbase = static_cast<const char*>(p.weight) + (size_t)it.vocab0 * rowb;
  };
  // Hidden-row load offsets (bytes from the hidden matrix + the stage's
  // column base) and the masked position of hidden row tid, for row tile rt.
  uint32_t hoff[H_LOADS];
  int out_row;
  auto set_rows = [&](const LmItem& it) {
    const int row0 = it.rt * kLmRows;
#pragma unroll
    for (int j = 0; j < H_LOADS; ++j) {
      const int r = (tid + kThreads * j) >> 3;
      const int row = p.row_ids[row0 + min(r, it.rows_here - 1)];
      hoff[j] = (uint32_t)((size_t)row * rowb) + (qc << 4);
    }
    out_row = tid < it.rows_here ? p.row_ids[row0 + tid] : 0;
  };

  // Column tile kt; the last tile of a d_model that is an odd multiple of 32
  // holds 32 columns.
  const int nfull = d / KS;
  const int ntile = nfull + (d % KS != 0 ? 1 : 0);
  // Weight tile kt goes to weight slot kt % 3, hidden tile kt to hidden slot
  // kt % 2 (the hidden rows come from L2 and need less lead).  In a 32-column
  // weight stage, a thread whose chunk lies in the second 32 columns (past the
  // row end) loads its row's chunk 64 bytes earlier into its own slot instead,
  // which no read of that stage uses: every thread issues W_LOADS loads per
  // weight tile, as the wait counts below assume.
  // Rows past the vocabulary load its last row (masked later).
  auto issue_w = [&](int kt, int wslot, const LmItem& it) {
    const uint32_t st = ring_u32 + wslot * W_TILE;
    const char* wk = uniform_ptr(it.wbase + (size_t)kt * ROWB);
    const int vlast = p.V - 1 - it.vocab0;
    const uint32_t col = (uint32_t)(qc << 4) - ((kt >= nfull && !lo_half) ? 64u : 0u);
    uint32_t off[W_LOADS], lds[W_LOADS];
#pragma unroll
    for (int j = 0; j < W_LOADS; ++j) {
      const int r = min((tid + kThreads * j) >> 3, vlast);
      off[j] = (uint32_t)r * (uint32_t)rowb + col;
      lds[j] = st + (kThreads * j + wave * 64) * 16;
    }
    dma16x4_s(wk, off, lds);
  };
  // The hidden tile of a 32-column stage loads only the first 32 columns; it
  // is always the item's last tile, waited for with no loads left in flight.
  auto issue_h = [&](int kt, int hslot) {
    const uint32_t st = ring_u32 + NSW * W_TILE + hslot * H_TILE;
    const char* hk = hbase + (size_t)kt * ROWB;
    if (kt < nfull || lo_half) {
      uint32_t lds[H_LOADS];
#pragma unroll
      for (int j = 0; j < H_LOADS; ++j) lds[j] = st + (kThreads * j + wave * 64) * 16;
      dma16x4_s(hk, hoff, lds);
    }
  };

  // Operand rows of this lane: vocabulary rows 64*vw + 32*vt + (lane & 31),
  // hidden rows 128*rw + 32*t + (lane & 31); the lane half picks the 8-column
  // run.
  const int lr = lane & 31, hh = lane >> 5;
  int a_row[2], b_row[4];
#pragma unroll
  for (int vt = 0; vt < 2; ++vt) a_row[vt] = 64 * vw + 32 * vt + lr;
#pragma unroll
  for (int t = 0; t < 4; ++t) b_row[t] = 128 * rw + 32 * t + lr;

  f32x16 acc[2][4];

  auto compute = [&](auto wslot_c, auto hslot_c, int n_halves) {
    const int wslot = wslot_c, hslot = hslot_c;
    const char* sw = ring + wslot * W_TILE;
    const char* sh = ring + NSW * W_TILE + hslot * H_TILE;
#pragma unroll
    for (int half = 0; half < KS / 32; ++half) {
      if (half >= n_halves) break;
      bf16x8 a[2][2], bq[2][4];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int c = 2 * (2 * half + s2) + hh;
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
          a[s2][vt] = *reinterpret_cast<const bf16x8*>(sw + a_row[vt] * ROWB + ((c ^ swz(a_row[vt])) << 4));
#pragma unroll
        for (int t = 0; t < 4; ++t)
          bq[s2][t] = *reinterpret_cast<const bf16x8*>(sh + b_row[t] * ROWB +
                                                       ((c ^ swz(b_row[t])) << 4));
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[vt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s2][vt], bq[s2][t], acc[vt][t], 0, 0, 0);
    }
  };

  // The next item's tiles 0 and 1 land in weight slots 0 and 1 and hidden
  // slot 0 exactly when ntile is a multiple of both ring periods.
  const bool chain = d % KS == 0 && ntile % (NSW * NSH) == 0;
  int item = lw;
  LmItem cur, nxt;
  set_item(item, cur);
  set_rows(cur);
  // Issue order: W0 H0 W1, then after the barrier of step t: H(t+1) W(t+2).
  // At step t the loads still allowed in flight are those of W(t+1) only, so
  // the weight stream runs two tiles ahead and the hidden stream one; past an
  // item's end, t+1 and t+2 continue into the next item's tiles 0 and 1.
  issue_w(0, 0, cur);
  issue_h(0, 0);
  if (ntile > 1) issue_w(1, 1, cur);
  using std::integral_constant;
  for (;;) {
    const int nitem = item + G;
    const bool more = nitem < total;
    if (more) set_item(nitem, nxt);
    // The next item's first tiles are requested early only when it has the
    // same row tile (always when G is a multiple of n_rt): its hidden rows are
    // this item's.
    const bool pre = chain && more && nxt.rt == cur.rt;
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[vt][t] = f32x16{};

    // Stage t: wait for tiles W(t), H(t), then request the tiles two and one
    // stages ahead, then the matrix work.  Kind (compile-time):
    //   0  tiles t+1 and t+2 exist in this item (the steady state);
    //   1  generic: requests only this item's tiles, when they exist;
    //   2  t = ntile-2 with chaining: H(t+1), then the next item's W0 if `pre`;
    //   3  t = ntile-1 with chaining: the next item's H0 and W1 if `pre`.
    auto step = [&](int t, auto ws, auto hs, int n_halves, auto kind) {
      constexpr int K = decltype(kind)::value;
      if constexpr (K == 0 || K == 2) {
        wait_vmcnt<W_LOADS>();
      } else if constexpr (K == 1) {
        if (t + 1 < ntile) wait_vmcnt<W_LOADS>(); else wait_vmcnt<0>();
      } else {
        if (pre) wait_vmcnt<W_LOADS>(); else wait_vmcnt<0>();
      }
      barrier();
      if constexpr (K == 0) {
        issue_h(t + 1, (t + 1) % NSH);
        issue_w(t + 2, (t + 2) % NSW, cur);
      } else if constexpr (K == 1) {
        if (t + 1 < ntile) issue_h(t + 1, (t + 1) % NSH);
        if (t + 2 < ntile) issue_w(t + 2, (t + 2) % NSW, cur);
      } else if constexpr (K == 2) {
        issue_h(t + 1, (t + 1) % NSH);
        if (pre) issue_w(0, 0, nxt);
      } else {
        if (pre) {
          issue_h(0, 0);
          issue_w(1, 1, nxt);
        }
      }
      compute(ws, hs, n_halves);
    };
    using C0 = integral_constant<int, 0>;
    using C1 = integral_constant<int, 1>;
    using C2 = integral_constant<int, 2>;
    using K0 = integral_constant<int, 0>;
    int i = 0;
    if (chain) {
      // ntile is a multiple of 6 (both rings' periods): every slot is a
      // constant; the last round hands over to the next item.
      for (; i + 6 < ntile; i += 6) {
        step(i, C0{}, C0{}, 2, K0{});
        step(i + 1, C1{}, C1{}, 2, K0{});
        step(i + 2, C2{}, C0{}, 2, K0{});
        step(i + 3, C0{}, C1{}, 2, K0{});
        step(i + 4, C1{}, C0{}, 2, K0{});
        step(i + 5, C2{}, C1{}, 2, K0{});
      }
      step(i, C0{}, C0{}, 2, K0{});
      step(i + 1, C1{}, C1{}, 2, K0{});
      step(i + 2, C2{}, C0{}, 2, K0{});
      step(i + 3, C0{}, C1{}, 2, K0{});
      step(i + 4, C1{}, C0{}, 2, integral_constant<int, 2>{});
      step(i + 5, C2{}, C1{}, 2, integral_constant<int, 3>{});
    } else {
      // Steady state unrolled by 6 with constant slots; the generic loop
      // takes the last nfull % 6 full stages and a 32-column last stage.
      const integral_constant<int, 1> K1{};
      for (; i + 6 <= nfull; i += 6) {
        step(i, C0{}, C0{}, 2, K1);
        step(i + 1, C1{}, C1{}, 2, K1);
        step(i + 2, C2{}, C0{}, 2, K1);
        step(i + 3, C0{}, C1{}, 2, K1);
        step(i + 4, C1{}, C0{}, 2, K1);
        step(i + 5, C2{}, C1{}, 2, K1);
      }
      for (; i < ntile; ++i) step(i, i % NSW, i % NSH, i < nfull ? 2 : 1, K1);
    }

    // Statistics of each hidden row over this wave's 64 entries.  Accumulator
    // register r of tile (vt, t) holds entry 64*vw + 32*vt + 8*(r/4) + 4*hh +
    // r%4 of row 128*rw + 32*t + lr; they are visited in increasing id order,
    // so a strict '>' keeps the lowest id among equal maxima.
    Triple tr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float m = -INFINITY;
      int arg = INT_MAX;
#pragma unroll
      for (int vt = 0; vt < 2; ++vt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int v = cur.vocab0 + 64 * vw + 32 * vt + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (v < p.V && acc[vt][t][r] > m) {
            m = acc[vt][t][r];
            arg = v;
          }
        }
      float s = 0.0f;
      if (m != -INFINITY) {
        const float mb = m * kLog2e;
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int v = cur.vocab0 + 64 * vw + 32 * vt + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (v < p.V) s += __builtin_amdgcn_exp2f(fmaf(acc[vt][t][r], kLog2e, -mb));
          }
      }
      tr[t] = combine(Triple{m, arg, s}, shfl_xor_triple(Triple{m, arg, s}, 32));
    }

    // Across the 4 vocabulary ranges, through weight slot 2: it held the
    // item's last tile (or nothing is in flight), never a prefetched one.
    // The waits here cover LDS operations only, so the next item's tiles stay
    // in flight.
    barrier();
    Triple* xt = reinterpret_cast<Triple*>(ring + 2 * W_TILE);   // [vocabulary range][256 rows]
    if (hh == 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) xt[vw * kLmRows + 128 * rw + 32 * t + lr] = tr[t];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier();
    if (tid < cur.rows_here) {
      Triple r = xt[tid];
#pragma unroll
      for (int w = 1; w < 4; ++w) r = combine(r, xt[w * kLmRows + tid]);
      VocabPartial out;
      out.m = r.m;
      out.arg = r.arg;
      out.s = r.s;
      out.pad = 0;
      p.slices[(size_t)out_row * p.n_slices + cur.slice] = out;
    }
    if (!more) break;
    item = nitem;
    const bool new_rows = nxt.rt != cur.rt;
    cur = nxt;
    if (!pre) {
      // Every wave is past its reads of xt (weight slot 2) before it reaches
      // the next stage's barrier, and these loads go to slots 0 and 1.
      if (new_rows) set_rows(cur);
      issue_w(0, 0, cur);
      issue_h(0, 0);
      if (ntile > 1) issue_w(1, 1, cur);
    }
  }
}

// One wavefront per masked row: lane i merges slices i, i+64, ..., then the
// wavefront combines (max and lowest argmax do not depend on the order; the
// sum is formed in one fixed order).
constexpr int kMergeBatch = 8;

__global__ __launch_bounds__(64) void lmhead_merge_kernel(LmParams p) {
  const int i = blockIdx.x;
  if (i >= *p.n_rows) return;
  const int lane = threadIdx.x;
  const int row = p.row_ids[i];
  const VocabPartial* src = p.slices + (size_t)row * p.n_slices;
  Triple t{-INFINITY, INT_MAX, 0.0f};
  for (int c0 = 0; c0 < p.n_slices; c0 += 64 * kMergeBatch) {
    VocabPartial q[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int c = c0 + 64 * j + lane;
      if (c < p.n_slices) q[j] = src[c];
    }
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      if (c0 + 64 * j + lane < p.n_slices) t = combine(t, Triple{q[j].m, q[j].arg, q[j].s});
  }
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) t = combine(t, shfl_xor_triple(t, mask));
  if (lane == 0) {
    VocabPartial out;
    out.m = t.m;
    out.arg = t.arg;
    out.s = t.s;
    out.pad = 0;
    p.merged[row] = out;
  }
}

}  // namespace

hipError_t launch_lmhead(const LmParams& p, hipStream_t stream) {
  if (p.n_pos <= 0 || p.d % kLmK != 0 || p.d <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lmhead_rows_kernel, dim3(1), dim3(1024), 0, stream, p);
  // Items: at most n_pos / 256 row tiles (rounded up) x n_slices.  When the
  // ring schedule lets an item hand over to the next (d_model a multiple of
  // 6 x 64), one persistent workgroup per CU takes them in turn; otherwise
  // each workgroup takes one item (a persistent workgroup would only wait
  // for its next item's first tiles, where a new workgroup does the same).
  const long long n_rt = (p.n_pos + kLmRows - 1) / kLmRows;
  const long long n = n_rt * p.n_slices;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const bool chain = p.d % KS == 0 && (p.d / KS) % (NSW * NSH) == 0;
  const unsigned grid = (unsigned)(chain ? std::min<long long>(n, kLmWorkgroups) : n);
  hipLaunchKernelGGL(lmhead_stats_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL(lmhead_merge_kernel, dim3((unsigned)p.n_pos), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tt
