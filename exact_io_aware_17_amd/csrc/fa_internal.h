// Internal interface between the host entry points (fa_api.cpp) and the
// gfx950 kernels. Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;              // may be null
  const int32_t* kv_lens;  // may be null
  int B, H, N, d;
  float scale;             // multiplies Q K^T
  float scale_log2;        // scale * log2(e), rounded once to float
  int causal;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;            // workspace: D_i = sum_c dO_ic O_ic, [B, H, N] float32
  float* lse2;             // workspace: lse_i * log2(e) (+inf for an empty row), [B, H, N]
  const int32_t* kv_lens;
  int B, H, N, d;
  float scale;
  float scale_log2;
  int causal;
};

// Each launcher enqueues on `stream` and returns hipGetLastError().
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream);

size_t bwd_workspace_bytes(int B, int H, int N, int d);

}  // namespace fa
