// Internal interface between the host entry points (fa_api.cpp) and the
// gfx950 kernels. Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <memory>

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
  int bn;                  // keys per streamed block (FWD_BN), 16-bit paths
  float scale;             // multiplies Q K^T
  float scale_log2;        // scale * log2(e), rounded once to float
  int causal;              // key j visible to query i only if j <= i + Nk - N - diag
  int diag;                // 0: causal (j <= i), 1: strict causal (j < i)
  // Causal without a split plan: 1 if each workgroup takes the pair of
  // query tiles (ntiles-1-r, r) (fwd_pair_tiles), 0 for one tile each.
  int pair;
  // One tile per workgroup, no split plan: 1 if each XCD runs its heads one
  // after another (fwd_head_sequential), 0 for the item-major order.
  int seq;
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
constexpr int BWD_BT = 128;                 // rows per gradient workgroup (queries in dQ, keys in dK/dV)
// Keys per streamed block of the 16-bit forward (the planner counts these
// blocks): 64 at every head dimension and shape.
constexpr int FWD_BN = 64;
// Compute units of the current device (0 if unknown; cached).
int fwd_device_cus();
constexpr int FWD_ML_FLOATS = 4 * 2 * FWD_BM;  // {m, l, l_bf, 0} for each of 2*BM lanes
constexpr int FWD_PLAN_MAX = 512;
// Key-range parts of one split tile: up to 16 when the plan splits several
// tiles, up to 64 when the rows are a single query tile (decode), whose
// parts are then the whole grid of a head.
constexpr int FWD_MAX_PARTS = 16;
constexpr int FWD_MAX_PARTS_ONE_TILE = 64;
// Arrival counters occupy a fixed region at the start of every forward
// workspace, whatever the shape, so a workspace reused for another shape
// still finds them zero: plans are made only when B*H*ntiles fits.
constexpr int FWD_COUNTERS = 16384;

// Work items of the forward, in dispatch order (the same list for every
// (b, h)). Item: tile | part << 9 | (nparts - 1) << 15 | slot_base << 21
// (tile < 512 and slot_base < 2048, as a plan has at most FWD_PLAN_MAX
// items; nparts <= FWD_MAX_PARTS_ONE_TILE).
// Part `part` of `nparts` covers key blocks [part*nb/nparts, (part+1)*nb/nparts)
// of the tile's nb nominal blocks; split parts use partial-state slots
// slot_base + part.
struct FwdPlan {
  int nitems;  // 0: one item per tile, heaviest first (no split)
  int nslots;  // partial-state slots per (b, h)
  uint32_t item[FWD_PLAN_MAX];
};

// Balancing plan for N query rows against Nk keys, BH query heads, `cus`
// compute units and `occ` resident workgroups per compute unit, in blocks of
// bn keys. Plans depend only on the tiles' block counts (so a decode loop
// whose key count grows by one per step reuses a plan for bn steps) and are
// kept in a bounded, least-recently-used cache; the returned plan stays
// valid while the caller holds it.
std::shared_ptr<const FwdPlan> fwd_plan(int N, int Nk, int BH, bool causal, int bn, int cus,
                                        int occ);
// Plans held by the cache (for tests of its bound) and its capacity.
size_t fwd_plan_cache_size();
constexpr size_t FWD_PLAN_CACHE_MAX = 128;
// Nominal key blocks of query tile t (causal: bottom-right aligned).
int fwd_tile_blocks(int N, int Nk, int t, bool causal, int bn);
// L2 cache of one XCD of the target device (gfx950: 4 MB per XCD).
constexpr long long FWD_L2_BYTES = 4ll << 20;
// Whether an unsplit causal forward pairs its query tiles: tile ntiles-1-r
// (keys ascending) then tile r (keys descending) in one workgroup, so that
// every workgroup streams ntiles+1 tiles' worth of blocks and the workgroups
// of a head read two key positions at a time. Chosen when one head's K and
// V (2 * Nk * d 16-bit elements) are at least one XCD's L2, where streaming
// every tile from key 0 re-fetches K and V in proportion to N, and the
// paired grid still fills every resident slot (BH * ceil(ntiles / 2) >=
// cus * occ).
bool fwd_pair_tiles(int N, int Nk, int d, int BH, bool causal, int cus, int occ);
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
  // Work order of each gradient kernel (head_sequential): 0 tile-major
  // (every XCD starts with the heaviest tiles of all its heads), 1 each XCD
  // runs its heads one after another.
  int seq_dq, seq_dkdv;
};

// Each launcher enqueues on `stream` and returns hipGetLastError().
// launch_fwd and launch_bwd take bf16 or fp16 tensors (p.dtype).
hipError_t launch_fwd(const FwdParams& p, const FwdPlan& plan, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);

size_t bwd_workspace_bytes(int B, int H, int N, int d);
// Whether a kernel with `items` workgroups over heads (a multiple of 8)
// should run each XCD's heads one after another: when the grid is at least
// 16 rounds of the cus * occ resident slots. The tile-major order then keeps
// every head of an XCD streaming its operands at once, past the L2 and the
// Infinity Cache, while the longest-first balance that the sequential order
// gives up within an XCD matters little over that many rounds. Measured on
// the backward: 2 rounds -13 %, 4 rounds -4 %, 8 rounds -1 to -4 %,
// 16 rounds +4 to +13 %, 32 rounds +13 to +31 %. On the forward at d = 128:
// 4 to 8 causal rounds -3 to -21 %, non-causal +-1 %; 16 rounds +10 to
// +36 %, 32 rounds +27 %.
bool head_sequential(long long items, int cus, int occ);

// The forward's order for one tile per workgroup and no split plan: each
// XCD runs its heads one after another (head_sequential on BH * ntiles
// workgroups, BH a multiple of 8) unless the causal tiles are paired.
bool fwd_head_sequential(int N, int Nk, int d, int BH, bool causal, int cus, int occ);

// fa_fwd_ex_noalloc's workspace: a device array of this many bytes per GPU
// (fa_noalloc.hip). noalloc_scratch() returns the current device's copy
// (nullptr if its address cannot be obtained); clear_ints() enqueues a
// kernel that zeroes n ints.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
void* noalloc_scratch();
hipError_t clear_ints(int* p, int n, hipStream_t stream);

}  // namespace fa
