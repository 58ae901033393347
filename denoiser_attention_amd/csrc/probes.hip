// Roof probes for gfx950: the rates this chip sustains for the two resources
// the denoising step is bound by, measured beside the datasheet figures.
//
//   tt_probe_hbm_read   streams a buffer from HBM with 16-byte non-temporal
//                       loads (the vocabulary pass's access pattern: one
//                       256-thread workgroup per 16 KB chunk, every load issued
//                       up front) and folds it into one word per workgroup.
//   tt_probe_mfma_bf16  back-to-back v_mfma_f32_32x32x16_bf16 on register
//                       operands: four independent accumulator chains per wave,
//                       four waves per workgroup, no memory traffic in the loop;
//                       operands random bf16 values (as attention tiles feed the
//                       matrix cores) or low-entropy ones (the rate the matrix
//                       cores reach when their power draw is low).
//
// Both kernels run a fixed amount of work and exit normally.  Their results are
// written only when they equal a value the inputs never produce, which keeps
// every load and every MFMA live without storing anything in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tt_probes.h"

#define TT_PROBE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kLoads = 4;                                   // 16-byte loads per thread
constexpr uint32_t kChunk = kThreads * kLoads * 16;         // bytes per workgroup
constexpr uint32_t kNever = 0x9e3779b9u;

__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4* buf, uint32_t* sink) {
  const u32x4* base = buf + (size_t)blockIdx.x * (kChunk / 16) + threadIdx.x;
  u32x4 v[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) v[i] = __builtin_nontemporal_load(base + i * kThreads);
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (acc == kNever) sink[blockIdx.x & 1023] = acc;
}

// A 32-bit integer hash (a murmur-style finalizer), for operand bits that look
// random to the multipliers.
__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// A bf16 value of magnitude 0.25..4 with a random sign and mantissa.
__device__ __forceinline__ __bf16 rand_bf16(uint32_t h) {
  const uint32_t bits = (h & 0x8000u) | ((125u + (h >> 16) % 5u) << 7) | ((h >> 8) & 0x7fu);
  return __builtin_bit_cast(__bf16, (uint16_t)bits);
}

// RANDOM = true: every MFMA takes a different pair of operand registers
// filled with random bf16 values (what an attention tile feeds the matrix
// cores); false: one pair of low-entropy operands (mostly zero bits) reused.
template <bool RANDOM>
__global__ __launch_bounds__(kThreads, 2) void mfma_bf16_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  constexpr int NR = RANDOM ? 4 : 1;
  bf16x8 a[NR], b[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (RANDOM) {
        const uint32_t seed = (blockIdx.x * kThreads + threadIdx.x) * 64u + j * 8u + i;
        a[j][i] = rand_bf16(mix(2u * seed + 1u));
        b[j][i] = rand_bf16(mix(2u * seed + 2u));
      } else {
        a[j][i] = (__bf16)(0.001f * (float)((lane + i) & 7));
        b[j][i] = (__bf16)(0.002f * (float)((lane * 3 + i) & 7));
      }
    }
  f32x16 c0{}, c1{}, c2{}, c3{};
  for (int it = 0; it < iters; it += NR) {
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[u], a[(u + 1) % NR], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(u + 2) % NR], b[(u + 3) % NR], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[(u + 1) % NR], a[(u + 3) % NR], c3, 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (s == -1.0f) sink[(blockIdx.x * kThreads + threadIdx.x) & 1023] = s;
}

}  // namespace

TT_PROBE_EXPORT int tt_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink,
                                      hipStream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % kChunk != 0) return 1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0) return 1;
  const size_t n = bytes / kChunk;
  if (n > 0x7fffffffu) return 1;
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)n), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(buf), sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

TT_PROBE_EXPORT int tt_probe_mfma_bf16(int n_workgroups, int iters, int random_operands,
                                       float* sink, hipStream_t stream) {
  if (!sink || n_workgroups < 1 || iters < 1 || iters % 4 != 0) return 1;
  if (random_operands)
    hipLaunchKernelGGL(mfma_bf16_kernel<true>, dim3((unsigned)n_workgroups), dim3(kThreads), 0,
                       stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_bf16_kernel<false>, dim3((unsigned)n_workgroups), dim3(kThreads), 0,
                       stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

TT_PROBE_EXPORT double tt_probe_mfma_bf16_flops(int n_workgroups, int iters) {
  // 4 waves x 4 MFMAs per iteration, each 32 x 32 x 16 multiply-adds.
  return (double)n_workgroups * 4.0 * 4.0 * (double)iters * 2.0 * 32.0 * 32.0 * 16.0;
}
