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
//   lmhead_stats_kernel  -- one workgroup of 8 waves per (256 masked rows,
//                           256-entry vocabulary slice).  Computes S^T =
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

// One 16-byte direct-to-LDS load per lane from a wave-uniform base plus a
// per-lane offset: lane i's bytes land at LDS address lds + 16*i.  Issued from
// asm (no register outputs) so that the compiler does not drain it before
// unrelated LDS reads; the explicit vmcnt waits and barriers order it.
__device__ __forceinline__ void dma16_s(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
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

__global__ __launch_bounds__(kThreads, 1) void lmhead_stats_kernel(LmParams p, int n_rt) {
  __shared__ __attribute__((aligned(1024))) char ring[RING];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int vw = wave & 3, rw = wave >> 2;         // vocabulary range, row half
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = logical % n_rt, slice = logical / n_rt;
  const int n_rows = *p.n_rows;
  const int row0 = rt * kLmRows;
  if (row0 >= n_rows) return;                      // whole workgroup
  const int rows_here = min(kLmRows, n_rows - row0);
  const int vocab0 = slice * kLmVocab;
  const int d = p.d;
  const size_t rowb = (size_t)d * 2;

  // Per-thread direct-load offsets (bytes from the stage's column base).
  uint32_t woff[W_LOADS], hoff[H_LOADS];
  bool wlo[W_LOADS], hlo[H_LOADS];   // the load's global chunk lies in the first 32 columns
#pragma unroll
  for (int j = 0; j < W_LOADS; ++j) {
    const int i = tid + kThreads * j, r = i >> 3, q = i & 7;
    const int v = min(vocab0 + r, p.V - 1);        // past the vocabulary: a valid row, masked later
    woff[j] = (uint32_t)((size_t)(v - vocab0) * rowb) + ((q ^ swz(r)) << 4);
    wlo[j] = (q ^ swz(r)) < 4;
  }
#pragma unroll
  for (int j = 0; j < H_LOADS; ++j) {
    const int i = tid + kThreads * j, r = i >> 3, q = i & 7;
    const int row = p.row_ids[row0 + min(r, rows_here - 1)];
    hoff[j] = (uint32_t)((size_t)row * rowb) + ((q ^ swz(r)) << 4);
    hlo[j] = (q ^ swz(r)) < 4;
  }
  const char* wbase = static_cast<const char*>(p.weight) + (size_t)vocab0 * rowb;
  const char* hbase = static_cast<const char*>(p.hidden);
  const uint32_t ring_u32 = (uint32_t)(uintptr_t)(lds_char*)ring;

  // Column tile kt; the last tile of a d_model that is an odd multiple of 32
  // holds 32 columns, and only the loads of those columns are issued.
  const int nfull = d / KS;
  const int ntile = nfull + (d % KS != 0 ? 1 : 0);
  // Weight tile kt goes to weight slot kt % 3, hidden tile kt to hidden slot
  // kt % 2 (the hidden rows come from L2 and need less lead).
  auto issue_w = [&](int kt, int wslot) {
    const uint32_t st = ring_u32 + wslot * W_TILE;
    const char* wk = wbase + (size_t)kt * ROWB;
    const bool half = kt >= nfull;
#pragma unroll
    for (int j = 0; j < W_LOADS; ++j)
      if (!half || wlo[j]) dma16_s(wk, woff[j], st + (kThreads * j + wave * 64) * 16);
  };
  auto issue_h = [&](int kt, int hslot) {
    const uint32_t st = ring_u32 + NSW * W_TILE + hslot * H_TILE;
    const char* hk = hbase + (size_t)kt * ROWB;
    const bool half = kt >= nfull;
#pragma unroll
    for (int j = 0; j < H_LOADS; ++j)
      if (!half || hlo[j]) dma16_s(hk, hoff[j], st + (kThreads * j + wave * 64) * 16);
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
#pragma unroll
  for (int vt = 0; vt < 2; ++vt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[vt][t] = f32x16{};

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

  // Issue order: W0 H0 W1, then after the barrier of step t: H(t+1) W(t+2).
  // At step t the loads still allowed in flight are those of W(t+1) only, so
  // the weight stream runs two tiles ahead and the hidden stream one.
  issue_w(0, 0);
  issue_h(0, 0);
  if (ntile > 1) issue_w(1, 1);
  using std::integral_constant;
  auto step = [&](int t, auto ws, auto hs, int n_halves) {
    if (t + 1 < ntile) wait_vmcnt<W_LOADS>(); else wait_vmcnt<0>();
    barrier();
    if (t + 1 < ntile) issue_h(t + 1, (t + 1) % NSH);
    if (t + 2 < ntile) issue_w(t + 2, (t + 2) % NSW);
    compute(ws, hs, n_halves);
  };
  int i = 0;
  // Steady state, unrolled by 6 (both rings' periods): constant slots.  The
  // generic loop below takes only the last nfull % 6 full stages and a
  // 32-column last stage.
  for (; i + 6 <= nfull; i += 6) {
    step(i, integral_constant<int, 0>{}, integral_constant<int, 0>{}, 2);
    step(i + 1, integral_constant<int, 1>{}, integral_constant<int, 1>{}, 2);
    step(i + 2, integral_constant<int, 2>{}, integral_constant<int, 0>{}, 2);
    step(i + 3, integral_constant<int, 0>{}, integral_constant<int, 1>{}, 2);
    step(i + 4, integral_constant<int, 1>{}, integral_constant<int, 0>{}, 2);
    step(i + 5, integral_constant<int, 2>{}, integral_constant<int, 1>{}, 2);
  }
  for (; i < ntile; ++i) step(i, i % NSW, i % NSH, i < nfull ? 2 : 1);

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
        const int v = vocab0 + 64 * vw + 32 * vt + 8 * (r >> 2) + 4 * hh + (r & 3);
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
          const int v = vocab0 + 64 * vw + 32 * vt + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (v < p.V) s += __builtin_amdgcn_exp2f(fmaf(acc[vt][t][r], kLog2e, -mb));
        }
    }
    tr[t] = combine(Triple{m, arg, s}, shfl_xor_triple(Triple{m, arg, s}, 32));
  }

  // Across the 4 vocabulary ranges (LDS; the ring is free once every wave is
  // past it).
  barrier();
  Triple* xt = reinterpret_cast<Triple*>(ring);   // [vocabulary range][256 rows]
  if (hh == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) xt[vw * kLmRows + 128 * rw + 32 * t + lr] = tr[t];
  }
  __syncthreads();
  if (tid < rows_here) {
    Triple r = xt[tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) r = combine(r, xt[w * kLmRows + tid]);
    const int row = p.row_ids[row0 + tid];
    VocabPartial out;
    out.m = r.m;
    out.arg = r.arg;
    out.s = r.s;
    out.pad = 0;
    p.slices[(size_t)row * p.n_slices + slice] = out;
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
  const long long n_rt = (p.n_pos + kLmRows - 1) / kLmRows;
  const long long n = n_rt * p.n_slices;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(lmhead_stats_kernel, dim3((unsigned)n), dim3(kThreads), 0, stream, p,
                     (int)n_rt);
  hipLaunchKernelGGL(lmhead_merge_kernel, dim3((unsigned)p.n_pos), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tt
