// Internal interface between the host entry points (fa_api.cpp) and the
// gfx950 kernels. Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Element types of q, k, v, o (and of the gradients).
enum { DTYPE_BF16 = 0, DTYPE_F16 = 1, DTYPE_F32 = 2 };

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;              // may be null
  const int32_t* kv_lens;  // may be null
  int B, H, N, d;          // N: query rows per head
  int Hkv, Nk;             // K/V heads (a divisor of H) and key rows per head
  int dtype;               // DTYPE_*
  int bn;                  // keys per streamed block (fwd_block_keys), 16-bit paths
  float scale;             // multiplies Q K^T
  float scale_log2;        // scale * log2(e), rounded once to float
  int causal;              // key j visible to query i only if j <= i + Nk - N - diag
  int diag;                // 0: causal (j <= i), 1: strict causal (j < i)
  // Split work items (used only with a plan of nitems > 0): per (b, h)
  // nslots partial states, each BM rows of unnormalised O (fp32) plus the
  // row max and both row sums, and one arrival counter per query tile.
  int nslots;
  int* counters;           // FWD_COUNTERS ints, zero between calls; [B*H, ntiles] used
  float* part_ml;          // [B*H, nslots, FWD_ML_FLOATS]
  float* part_o;           // [B*H, nslots, FWD_BM * d]
};

// Forward tiling shared by the kernel and the host planner.
constexpr int FWD_BM = 128;                 // query rows per workgroup
// Keys per streamed block of a forward launch (the planner counts these
// blocks): 64 for head dimensions up to 64; at d = 128, 64 (two workgroups
// per CU) without the causal mask or for long causal rows on at most two
// waves of workgroups, else 32 (three per CU); 32 at d = 96 and 256.
int fwd_block_keys(int d, int Nq, int Nk, int BH, bool causal, int cus);
// Compute units of the current device (0 if unknown; cached).
int fwd_device_cus();
constexpr int FWD_ML_FLOATS = 4 * 2 * FWD_BM;  // {m, l, l_bf, 0} for each of 2*BM lanes
constexpr int FWD_PLAN_MAX = 512;
constexpr int FWD_MAX_PARTS = 16;  // key-range parts of one split tile
// Arrival counters occupy a fixed region at the start of every forward
// workspace, whatever the shape, so a workspace reused for another shape
// still finds them zero: plans are made only when B*H*ntiles fits.
constexpr int FWD_COUNTERS = 16384;

// Work items of the forward, in dispatch order (the same list for every
// (b, h)). Item: tile | part << 12 | (nparts - 1) << 16 | slot_base << 20
// (tile < 4096, nparts <= FWD_MAX_PARTS, slot_base < 4096).
// Part `part` of `nparts` covers key blocks [part*nb/nparts, (part+1)*nb/nparts)
// of the tile's nb nominal blocks; split parts use partial-state slots
// slot_base + part.
struct FwdPlan {
  int nitems;  // 0: one item per tile, heaviest first (no split)
  int nslots;  // partial-state slots per (b, h)
  uint32_t item[FWD_PLAN_MAX];
};

// Balancing plan for N query rows against Nk keys, BH query heads, `cus`
// compute units and `occ` resident workgroups per compute unit (cached; the
// reference stays valid).
// Blocks are of bn keys (fwd_block_keys(d)).
const FwdPlan& fwd_plan(int N, int Nk, int BH, bool causal, int bn, int cus, int occ);
// Nominal key blocks of query tile t (causal: bottom-right aligned).
int fwd_tile_blocks(int N, int Nk, int t, bool causal, int bn);
// Workspace layout for a plan: byte offsets of counters, part_ml, part_o and the total.
struct FwdWorkspace {
  size_t counters, part_ml, part_o, total;
};
FwdWorkspace fwd_workspace_layout(const FwdPlan& plan, int BH, int N, int d);
// Resident forward workgroups per compute unit of the instance for head
// dimension d, block size bn and element type dtype (0 if unknown; cached).
int fwd_occupancy(int d, int bn, bool causal, int dtype);

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
  int B, H, N, d;          // N: query rows per head
  int Hkv, Nk;             // as FwdParams
  int dtype;               // DTYPE_BF16 or DTYPE_F16
  float scale;
  float scale_log2;
  int causal;
  int diag;                // as FwdParams
};

// Each launcher enqueues on `stream` and returns hipGetLastError().
// launch_fwd and launch_bwd take bf16 or fp16 tensors (p.dtype).
hipError_t launch_fwd(const FwdParams& p, const FwdPlan& plan, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);

size_t bwd_workspace_bytes(int B, int H, int N, int d);

}  // namespace fa
