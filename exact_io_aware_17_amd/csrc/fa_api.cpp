// Host entry points of libfa: argument validation, then one launch per step on
// the caller's stream. Validation happens before any HIP call, so every
// argument error is reported without touching the device.
#include "../../include/fa.h"

#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

static_assert(fa::NOALLOC_SCRATCH_BYTES == FA_NOALLOC_SCRATCH_BYTES,
              "the header states the scratch size the library holds");

namespace {

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  if (!a || !b) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shared checks of the shape, scale and mask arguments: H query heads of Nq
// rows, Hkv K/V heads (H a multiple of Hkv) of Nk rows.
int check_common(int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int mask_kind) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL &&
      mask_kind != FA_MASK_CAUSAL_STRICT)
    return FA_ERR_INVALID_ARG;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  // Row indices (b*H + h)*Nq + i and (b*Hkv + h)*Nk + j are formed in 32-bit
  // arithmetic.
  if ((long long)B * H * Nq > 0x7fffffffLL || (long long)B * Hkv * Nk > 0x7fffffffLL)
    return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Decode with grouped K/V heads: with one query row per head the G = H / Hkv
// query heads that share a K/V head are G adjacent rows of q and o (a
// [B, H, 1, d] tensor is laid out as [B, Hkv, G, d]) and of lse, and that
// one query sees every key under the non-strict causal mask (it sits at the
// last key's position). Launched as Hkv heads of G query rows without the
// mask, each K/V head is streamed once instead of once per query head; the
// rows, their keys and their results are the same. Rewrites the launch
// shape in place (16-bit paths only; the strict mask hides the last key, so
// it keeps the per-head launch).
void pack_decode(int& H, int Hkv, int& Nq, int& mask_kind) {
  if (Nq != 1 || H == Hkv || mask_kind == FA_MASK_CAUSAL_STRICT) return;
  Nq = H / Hkv;
  H = Hkv;
  mask_kind = FA_MASK_NONE;
}

bool valid_dtype(int dtype) {
  return dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F16 || dtype == FA_DTYPE_F32;
}

float scale_log2(float scale) {
  return (float)((double)scale * 1.4426950408889634073599246810019);
}

const fa::FwdPlan& no_plan() {
  static const fa::FwdPlan plan = [] {
    fa::FwdPlan p{};
    p.nitems = 0;
    p.nslots = 0;
    return p;
  }();
  return plan;
}

// Where a forward's split-KV workspace comes from: the caller, or the
// library's per-device scratch (fa_fwd_ex_noalloc).
enum WorkspaceSource { WS_CALLER, WS_SCRATCH };

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Hkv, int Nq, int Nk, int d, int dtype, float scale, int mask_kind,
               const int32_t* kv_lens, void* workspace, size_t workspace_bytes, hipStream_t stream,
               WorkspaceSource source = WS_CALLER) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!workspace && workspace_bytes) return FA_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return FA_ERR_INVALID_ARG;
  int st = check_common(B, H, Hkv, Nq, Nk, d, scale, mask_kind);
  if (st != FA_OK) return st;
  const bool f32 = (dtype == FA_DTYPE_F32);
  const size_t elem = f32 ? 4 : 2;
  const size_t qbytes = (size_t)B * H * Nq * d * elem;    // q, o
  const size_t kbytes = (size_t)B * Hkv * Nk * d * elem;  // k, v
  const size_t lbytes = (size_t)B * H * Nq * sizeof(float);
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) ||
      overlaps(o, qbytes, v, kbytes))
    return FA_ERR_INVALID_ARG;
  if (lse && (overlaps(lse, lbytes, q, qbytes) || overlaps(lse, lbytes, k, kbytes) ||
              overlaps(lse, lbytes, v, kbytes) || overlaps(lse, lbytes, o, qbytes)))
    return FA_ERR_INVALID_ARG;
  if (workspace) {
    const void* others[5] = {q, k, v, o, lse};
    const size_t osz[5] = {qbytes, kbytes, kbytes, qbytes, lbytes};
    for (int i = 0; i < 5; ++i)
      if (overlaps(workspace, workspace_bytes, others[i], osz[i])) return FA_ERR_INVALID_ARG;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_UNSUPPORTED;
  if (lse && ((uintptr_t)lse & 3u)) return FA_ERR_UNSUPPORTED;
  if (kv_lens && ((uintptr_t)kv_lens & 3u)) return FA_ERR_UNSUPPORTED;
  if (workspace && !aligned16(workspace)) return FA_ERR_UNSUPPORTED;

  fa::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.kv_lens = kv_lens;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.N = Nq;
  p.Nk = Nk;
  p.d = d;
  p.dtype = f32 ? fa::DTYPE_F32 : (dtype == FA_DTYPE_F16 ? fa::DTYPE_F16 : fa::DTYPE_BF16);
  p.scale = scale;
  p.scale_log2 = scale_log2(scale);
  p.causal = (mask_kind != FA_MASK_NONE);
  p.diag = (mask_kind == FA_MASK_CAUSAL_STRICT) ? 1 : 0;
  p.pair = 0;
  p.seq = 0;
  p.nslots = 0;
  p.counters = nullptr;
  p.part_ml = nullptr;
  p.part_o = nullptr;
  p.bn = 0;
  if (f32) {
    hipError_t e = fa::launch_fwd_f32(p, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  pack_decode(H, Hkv, Nq, mask_kind);
  p.H = H;
  p.N = Nq;
  p.causal = (mask_kind != FA_MASK_NONE);
  const int BH = B * H;
  const int cus = fa::fwd_device_cus();
  p.bn = fa::FWD_BN;
  const int occ = fa::fwd_occupancy(d, p.bn, p.causal != 0, p.dtype);
  std::shared_ptr<const fa::FwdPlan> held;  // keeps the plan alive until the launch
  const fa::FwdPlan* plan = &no_plan();
  if (source == WS_SCRATCH) {
    // Every argument is valid: take the plan, check that its workspace fits
    // the scratch, then find this device's scratch and clear the counters
    // the plan uses (the scratch keeps whatever the last call left).
    held = fa::fwd_plan(Nq, Nk, BH, p.causal != 0, p.bn, cus, occ);
    const fa::FwdWorkspace w = fa::fwd_workspace_layout(*held, BH, Nq, d);
    if (w.total > fa::NOALLOC_SCRATCH_BYTES) return FA_ERR_UNSUPPORTED;
    if (held->nitems > 0) {
      char* ws = (char*)fa::noalloc_scratch();
      if (!ws) return FA_ERR_HIP;
      plan = held.get();
      p.nslots = held->nslots;
      p.counters = (int*)(ws + w.counters);
      p.part_ml = (float*)(ws + w.part_ml);
      p.part_o = (float*)(ws + w.part_o);
      const int ntiles = (Nq + fa::FWD_BM - 1) / fa::FWD_BM;
      if (fa::clear_ints(p.counters, BH * ntiles, stream) != hipSuccess)
        return FA_ERR_HIP;
    }
  } else if (workspace) {
    held = fa::fwd_plan(Nq, Nk, BH, p.causal != 0, p.bn, cus, occ);
    const fa::FwdWorkspace w = fa::fwd_workspace_layout(*held, BH, Nq, d);
    if (held->nitems > 0 && workspace_bytes >= w.total) {
      plan = held.get();
      p.nslots = held->nslots;
      p.counters = (int*)((char*)workspace + w.counters);
      p.part_ml = (float*)((char*)workspace + w.part_ml);
      p.part_o = (float*)((char*)workspace + w.part_o);
    }
  }
  if (plan->nitems == 0 && fa::fwd_pair_tiles(Nq, Nk, d, BH, p.causal != 0, cus, occ)) p.pair = 1;
  if (plan->nitems == 0 && fa::fwd_head_sequential(Nq, Nk, d, BH, p.causal != 0, cus, occ))
    p.seq = 1;
  hipError_t e = fa::launch_fwd(p, *plan, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Resident workgroups per compute unit of both gradient kernels (their
// launch bounds: two, one at d = 256).
int bwd_occupancy(int d) { return d == 256 ? 1 : 2; }

// Work order of the two gradient kernels (head_sequential per kernel).
void bwd_orders(int B, int H, int Hkv, int Nq, int Nk, int d, int cus, int occ, int& seq_dq,
                int& seq_dkdv) {
  (void)d;
  const long long bt = fa::BWD_BT;
  const long long dq_items = (long long)B * H * ((Nq + bt - 1) / bt);
  const long long dkdv_items = (long long)B * Hkv * ((Nk + bt - 1) / bt);
  seq_dq = ((B * H) % 8 == 0 && fa::head_sequential(dq_items, cus, occ)) ? 1 : 0;
  seq_dkdv = ((B * Hkv) % 8 == 0 && fa::head_sequential(dkdv_items, cus, occ)) ? 1 : 0;
}

int bwd_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, void* workspace, int B, int H,
               int Hkv, int Nq, int Nk, int d, int dtype, float scale, int mask_kind,
               const int32_t* kv_lens, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
    return FA_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return FA_ERR_INVALID_ARG;
  int st = check_common(B, H, Hkv, Nq, Nk, d, scale, mask_kind);
  if (st != FA_OK) return st;
  if (dtype == FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
  const size_t qbytes = (size_t)B * H * Nq * d * 2;    // q, o, dout, dq
  const size_t kbytes = (size_t)B * Hkv * Nk * d * 2;  // k, v, dk, dv
  const size_t lbytes = (size_t)B * H * Nq * sizeof(float);
  const size_t wbytes = fa::bwd_workspace_bytes(B, H, Nq, d);
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t insz[6] = {qbytes, kbytes, kbytes, qbytes, qbytes, lbytes};
  void* outs[4] = {dq, dk, dv, workspace};
  const size_t outsz[4] = {qbytes, kbytes, kbytes, wbytes};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return FA_ERR_INVALID_ARG;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
      ((uintptr_t)lse & 3u) || (kv_lens && ((uintptr_t)kv_lens & 3u)))
    return FA_ERR_UNSUPPORTED;

  fa::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = (float*)workspace;
  p.lse2 = (float*)((char*)workspace + wbytes / 2);
  p.kv_lens = kv_lens;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.N = Nq;
  p.Nk = Nk;
  p.d = d;
  p.dtype = (dtype == FA_DTYPE_F16) ? fa::DTYPE_F16 : fa::DTYPE_BF16;
  p.scale = scale;
  p.scale_log2 = scale_log2(scale);
  p.causal = (mask_kind != FA_MASK_NONE);
  p.diag = (mask_kind == FA_MASK_CAUSAL_STRICT) ? 1 : 0;
  bwd_orders(B, H, Hkv, Nq, Nk, d, fa::fwd_device_cus(), bwd_occupancy(d), p.seq_dq, p.seq_dkdv);
  hipError_t e = fa::launch_bwd(p, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK:
      return "FA_OK";
    case FA_ERR_INVALID_ARG:
      return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: unsupported head dimension, alignment or size";
    case FA_ERR_HIP:
      return "FA_ERR_HIP: kernel launch failed";
    default:
      return "unknown fa_status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int mask_kind, const int32_t* kv_lens, hipStream_t stream) {
  return fwd_common(q, k, v, o, lse, B, H, H, N, N, d, FA_DTYPE_BF16, scale, mask_kind, kv_lens,
                    nullptr, 0, stream);
}

size_t fa_fwd_ex_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d, int dtype,
                                 int mask_kind) {
  if (check_common(B, H, Hkv, Nq, Nk, d, 1.f, mask_kind) != FA_OK) return 0;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return 0;  // fp32: never split
  pack_decode(H, Hkv, Nq, mask_kind);  // the launch shape fa_fwd_ex plans for
  const bool causal = (mask_kind != FA_MASK_NONE);
  const int cus = fa::fwd_device_cus();
  const int bn = fa::FWD_BN;
  const int occ = fa::fwd_occupancy(d, bn, causal, dtype == FA_DTYPE_F16 ? fa::DTYPE_F16 : fa::DTYPE_BF16);
  const auto plan = fa::fwd_plan(Nq, Nk, B * H, causal, bn, cus, occ);
  return fa::fwd_workspace_layout(*plan, B * H, Nq, d).total;
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Hkv, int Nq, int Nk, int d, int dtype, float scale, int mask_kind,
              const int32_t* kv_lens, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fwd_common(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, dtype, scale, mask_kind, kv_lens,
                    workspace, workspace_bytes, stream);
}

int fa_fwd_ex_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Hkv, int Nq, int Nk, int d, int dtype, float scale, int mask_kind,
                      const int32_t* kv_lens, hipStream_t stream) {
  return fwd_common(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, dtype, scale, mask_kind, kv_lens,
                    nullptr, 0, stream, WS_SCRATCH);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
               int N, int d, float scale, int mask_kind, const int32_t* kv_lens, hipStream_t stream) {
  return fwd_common(q, k, v, o, lse, B, H, H, N, N, d, FA_DTYPE_F32, scale, mask_kind, kv_lens,
                    nullptr, 0, stream);
}

int fa_fwd_schedule(int Nq, int Nk, int BH, int d, int mask_kind, int cus, int occ,
                    uint32_t* items, int max_items, int* nslots) {
  if (Nq <= 0 || Nk <= 0 || BH <= 0 || d <= 0 || cus < 0 || occ < 0 || max_items < 0 ||
      (max_items > 0 && !items))
    return FA_ERR_INVALID_ARG;
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL &&
      mask_kind != FA_MASK_CAUSAL_STRICT)
    return FA_ERR_INVALID_ARG;
  const bool causal = mask_kind != FA_MASK_NONE;
  (void)d;  // every head dimension streams FWD_BN-key blocks
  const auto plan = fa::fwd_plan(Nq, Nk, BH, causal, fa::FWD_BN, cus, occ);
  for (int i = 0; i < plan->nitems && i < max_items; ++i) items[i] = plan->item[i];
  if (nslots) *nslots = plan->nslots;
  return plan->nitems;
}

int fa_fwd_tile_order(int Nq, int Nk, int BH, int d, int dtype, int mask_kind, int cus, int occ) {
  if (Nq <= 0 || Nk <= 0 || BH <= 0 || d <= 0 || cus < 0 || occ < 0) return FA_ERR_INVALID_ARG;
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL &&
      mask_kind != FA_MASK_CAUSAL_STRICT)
    return FA_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return FA_ERR_INVALID_ARG;
  if (dtype == FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
  const bool causal = mask_kind != FA_MASK_NONE;
  if (cus == 0 && occ == 0) {
    cus = fa::fwd_device_cus();
    occ = fa::fwd_occupancy(d, fa::FWD_BN, causal,
                            dtype == FA_DTYPE_F16 ? fa::DTYPE_F16 : fa::DTYPE_BF16);
  }
  if (fa::fwd_pair_tiles(Nq, Nk, d, BH, causal, cus, occ)) return FA_FWD_ORDER_PAIRED;
  if (fa::fwd_head_sequential(Nq, Nk, d, BH, causal, cus, occ))
    return FA_FWD_ORDER_HEAD_SEQUENTIAL;
  return FA_FWD_ORDER_HEAVY_FIRST;
}

int fa_bwd_tile_order(int B, int H, int Hkv, int Nq, int Nk, int d, int cus, int occ) {
  if (cus < 0 || occ < 0) return FA_ERR_INVALID_ARG;
  const int st = check_common(B, H, Hkv, Nq, Nk, d, 1.f, FA_MASK_NONE);
  if (st != FA_OK) return st;
  if (cus == 0 && occ == 0) {
    cus = fa::fwd_device_cus();
    occ = bwd_occupancy(d);
  }
  int seq_dq = 0, seq_dkdv = 0;
  bwd_orders(B, H, Hkv, Nq, Nk, d, cus, occ, seq_dq, seq_dkdv);
  return (seq_dq ? FA_BWD_DQ_HEAD_SEQUENTIAL : 0) | (seq_dkdv ? FA_BWD_DKDV_HEAD_SEQUENTIAL : 0);
}

int fa_fwd_block_keys(int B, int H, int Nq, int Nk, int d, int mask_kind) {
  const int st = check_common(B, H, H, Nq, Nk, d, 1.f, mask_kind);
  if (st != FA_OK) return st;
  return fa::FWD_BN;
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  return fa::bwd_workspace_bytes(B, H, N, d);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, void* workspace, int B, int H, int N,
           int d, float scale, int mask_kind, const int32_t* kv_lens, hipStream_t stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, H, N, N, d, FA_DTYPE_BF16,
                    scale, mask_kind, kv_lens, stream);
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv, void* workspace, int B, int H,
              int Hkv, int Nq, int Nk, int d, int dtype, float scale, int mask_kind,
              const int32_t* kv_lens, hipStream_t stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, Hkv, Nq, Nk, d, dtype,
                    scale, mask_kind, kv_lens, stream);
}

}  // extern "C"
