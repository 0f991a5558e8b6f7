/* libfa_probe: a measurement probe for gfx950, not part of the attention
 * interface (libfa does not contain it and does not depend on it).
 *
 * fa_probe_mfma_bf16 runs nothing but bf16 matrix-core instructions
 * (v_mfma_f32_32x32x16_bf16, 32768 FLOPs each): every wave of 256-thread
 * workgroups issues `iters` rounds of four independent accumulator chains on
 * operands held in registers. Launched with two workgroups per compute unit
 * (two waves per SIMD), it measures the matrix-core rate the device sustains
 * at its current clock, the practical ceiling beside the published dense
 * bf16 peak against which the attention kernels are compared.
 *
 * Arguments:
 *   workgroups  number of 256-thread workgroups (> 0)
 *   iters       rounds per wave (> 0); one round = 4 MFMAs
 *   sink        device pointer to at least one float; written only if the
 *               accumulated sum equals -1, which cannot happen (every
 *               operand is non-negative): it keeps the work from being
 *               optimised away
 *   stream      HIP stream the launch is enqueued on (0 = null stream)
 * Returns 0, -1 for a bad argument (nothing is launched) or -3 when the
 * launch fails. The call is asynchronous and allocates nothing.
 *
 * fa_probe_mfma_bf16_flops returns the FLOPs one such launch performs:
 * workgroups * 4 waves * iters * 4 * 32768. */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#include <hip/hip_runtime.h>

#ifdef __cplusplus
extern "C" {
#endif

int fa_probe_mfma_bf16(int workgroups, int iters, float* sink, hipStream_t stream);
double fa_probe_mfma_bf16_flops(int workgroups, int iters);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
