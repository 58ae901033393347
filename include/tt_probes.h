/*
 * tt_probes.h -- roof probes of libtt_probes (measurement only, not part of the
 * denoising step).  They measure what an MI355X (gfx950) sustains for the two
 * resources the step is bound by, so that each kernel's time can be put against
 * both the datasheet roof and the measured one.
 *
 * Conventions: device pointers on the current HIP device; calls only enqueue on
 * `stream`; return 0 on success, 1 for an invalid argument (nothing enqueued),
 * 4 for a failed launch.  Neither probe stores anything in practice: `sink`
 * receives a value only if a reduction equals one the inputs never produce.
 */
#ifndef TT_PROBES_H_
#define TT_PROBES_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streams `bytes` of `buf` from memory once with 16-byte non-temporal loads,
 * one 256-thread workgroup per 16 KB (every load issued up front).
 *   buf   16-byte aligned; bytes a positive multiple of 16384
 *   sink  uint32_t[1024] scratch */
int tt_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/* n_workgroups 256-thread workgroups, each wave issuing `iters` x 4 independent
 * v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic in the loop).
 *   iters            a positive multiple of 4
 *   random_operands  1: each MFMA reads a different register pair of random
 *                    bf16 values (magnitudes 0.25..4); 0: one pair of
 *                    low-entropy values (mostly zero bits), reused
 *   sink             float[1024] scratch */
int tt_probe_mfma_bf16(int n_workgroups, int iters, int random_operands, float* sink,
                       hipStream_t stream);

/* Floating-point operations of one tt_probe_mfma_bf16 call. */
double tt_probe_mfma_bf16_flops(int n_workgroups, int iters);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* TT_PROBES_H_ */
