// Matrix-core rate probe for gfx950 (libfa_probe.so): bf16 32x32x16 MFMAs
// only, four independent accumulator chains per wave, operands in registers.
// It measures the sustained matrix-core ceiling the attention kernels are
// measured beside; the attention library neither contains nor uses it.
#include <hip/hip_runtime.h>

#include "fa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256, 2) void mfma_peak_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // Small non-negative values: the sums stay finite and non-negative.
    a[i] = (__bf16)(0.0009765625f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.0009765625f * (float)((3 * lane + i) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (s == -1.0f) sink[0] = s;  // never true: keeps the chains live
}

}  // namespace

extern "C" int fa_probe_mfma_bf16(int workgroups, int iters, float* sink, hipStream_t stream) {
  if (workgroups <= 0 || iters <= 0 || sink == nullptr) return -1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, iters,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" double fa_probe_mfma_bf16_flops(int workgroups, int iters) {
  if (workgroups <= 0 || iters <= 0) return 0.0;
  return (double)workgroups * 4.0 * (double)iters * 4.0 * 32768.0;
}
