// Measurement probes for gfx950 (libfa_probe.so): the matrix-core rate
// (bf16 32x32x16 MFMAs only, four independent accumulator chains per wave,
// operands in registers) and the HBM -> LDS streaming rate (the forward's
// load path alone). They measure the sustained ceilings the attention
// kernels are measured beside; the attention library neither contains nor
// uses them.
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

// HBM -> LDS streaming: each workgroup reads `blocks` consecutive 32 KB
// blocks through two LDS stages with 16-byte buffer loads into LDS (the path
// and the one-block-ahead ring of the attention forward), 8 loads of 1 KB per
// wave per block. Wave 0 reads one element of every lane's 16 bytes of each
// landed block back from LDS and sums them; thread 0 writes the sum.
constexpr int kStreamBlock = 32768;

__global__ __launch_bounds__(256, 2) void stream_lds_kernel(const char* src, int blocks,
                                                             float* sums) {
  __shared__ __attribute__((aligned(1024))) char stage0[kStreamBlock];
  __shared__ __attribute__((aligned(1024))) char stage1[kStreamBlock];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* base = src + (size_t)blockIdx.x * blocks * kStreamBlock;
  auto issue = [&](int j, char* dst) {
    if (j >= blocks) return;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base + (size_t)j * kStreamBlock), 0, kStreamBlock, 0x00020000);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kb = wave * 8 + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + kb * 1024),
                                               16, kb * 1024 + lane * 16, 0, 0, 0);
    }
  };
  float s = 0.0f;
  auto consume = [&](const char* stage) {
    if (wave != 0) return;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      s += (float)*(const __bf16*)(stage + i * 1024 + lane * 16 + 2 * (i & 7));
    }
  };
  issue(0, stage0);
  for (int j = 0; j < blocks; j += 2) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of block j
    __syncthreads();
    issue(j + 1, stage1);
    consume(stage0);
    if (j + 1 >= blocks) break;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    issue(j + 2, stage0);
    consume(stage1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no load may still target LDS at exit
  if (threadIdx.x == 0) sums[blockIdx.x] = s;
}

}  // namespace

extern "C" int fa_probe_stream_lds(const void* src, int workgroups, int blocks, float* sums,
                                   hipStream_t stream) {
  if (src == nullptr || sums == nullptr || workgroups <= 0 || blocks <= 0 ||
      workgroups > (1 << 20) || blocks > (1 << 16))
    return -1;
  hipLaunchKernelGGL(stream_lds_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream,
                     (const char*)src, blocks, sums);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" double fa_probe_stream_lds_bytes(int workgroups, int blocks) {
  if (workgroups <= 0 || blocks <= 0) return 0.0;
  return (double)workgroups * (double)blocks * 32768.0;
}

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
