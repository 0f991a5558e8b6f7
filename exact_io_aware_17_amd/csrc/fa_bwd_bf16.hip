// Exact attention backward for gfx950: P recomputed from the saved logsumexp.
//
// The pages say only that the backward pass recomputes S and P from Q, K, V
// instead of storing them ("Question bank", the recomputation answers); the
// formulas are the standard derivative of softmax attention:
//   P = exp(S - lse) (0 where hidden or lse = -inf),  D_i = sum_c dO_ic O_ic,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,
//   dK = scale dS^T Q.
// Three kernels, no atomics:
//   delta  D_i for every row (fp32, into the caller's workspace);
//   dq     one workgroup per 32*NW query rows streams the visible key blocks:
//          S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T (the forward's
//          transposed layout: one query per lane pair);
//   dkdv   one workgroup per 32*NW keys streams the query blocks that see
//          them: S = Q K^T, dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS
//          (one key per lane pair).
// Operands that feed an MFMA contraction over the streamed index are staged
// in LDS twice: row-major (16-byte chunks XOR-swizzled by row) and
// transposed with the streamed index permuted by swap23, matching the order
// in which a 32x32 accumulator holds its rows.
#include "fa_internal.h"
#include "fa_device.h"

#include <math.h>

namespace fa {
namespace {

using namespace dev;

constexpr int BS = 64;  // streamed rows (keys in dq, queries in dkdv) per block

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// ---- a7: D_i = sum_c dO_ic O_ic ----
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const long long rows = (long long)p.B * p.H * p.N;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)((const __bf16*)p.o + row * D + c * 8);
    const u32x4 g = *(const u32x4*)((const __bf16*)p.dout + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf_lo(a[e]), bf_lo(g[e]), acc);
      acc = fmaf(bf_hi(a[e]), bf_hi(g[e]), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) p.delta[row] = acc;
}

// Stage rows [r0, r0 + BS) of a row-major [N, D] bf16 matrix into LDS, as a
// row-major copy (`rm`, may be null) and a transposed copy (`tr`, may be
// null) whose row index is permuted by swap23. Rows past N repeat row N-1.
template <int D, int NT>
__device__ __forceinline__ void stage_rows(const __bf16* __restrict__ X, int r0, int N, char* rm,
                                           char* tr, int tid) {
  constexpr int KCH = D / 8;
  constexpr int UNITS = (BS / 2) * KCH;
  static_assert(UNITS % NT == 0, "staging units must divide evenly");
#pragma unroll
  for (int i = 0; i < UNITS / NT; ++i) {
    const int u = tid + NT * i;
    const int dc = u % KCH, rp = u / KCH;
    const int ra = min(r0 + 2 * rp, N - 1);
    const int rb = min(r0 + 2 * rp + 1, N - 1);
    const u32x4 xa = *(const u32x4*)(X + (size_t)ra * D + dc * 8);
    const u32x4 xb = *(const u32x4*)(X + (size_t)rb * D + dc * 8);
    if (rm) {
      *(u32x4*)(rm + (2 * rp) * (D * 2) + row_slot<D>(2 * rp, dc) * 16) = xa;
      *(u32x4*)(rm + (2 * rp + 1) * (D * 2) + row_slot<D>(2 * rp + 1, dc) * 16) = xb;
    }
    if (tr) {
      const int pos = swap23(2 * rp);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = dc * 8 + e;
        const unsigned lo = (e & 1) ? hi16(xa[e >> 1]) : lo16(xa[e >> 1]);
        const unsigned hi = (e & 1) ? hi16(xb[e >> 1]) : lo16(xb[e >> 1]);
        *(unsigned*)(tr + d * (BS * 2) + t64_slot(d, pos >> 3) * 16 + (pos & 7) * 2) =
            lo | (hi << 16);
      }
    }
  }
}

// Work id with the XCD-contiguous remap (workgroups go round-robin over 8 XCDs).
__device__ __forceinline__ int work_id() {
  const int G = gridDim.x, bid = blockIdx.x;
  return (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
}

// Store a transposed 32x32-tiled accumulator (lane = one row of the output,
// registers = D columns in groups of 4) as bf16, times `mul`.
template <int D>
__device__ __forceinline__ void store_rowT(__bf16* dst, const f32x16* acc, float mul, int h) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[t][4 * g] * mul, acc[t][4 * g + 1] * mul);
      w[1] = pack_bf16x2(acc[t][4 * g + 2] * mul, acc[t][4 * g + 3] * mul);
      *(u32x2*)(dst + t * 32 + 8 * g + 4 * h) = w;
    }
}

// ---- dQ: one workgroup per 32*NW query rows ----
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_kernel(BwdParams p) {
  constexpr int BM = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int TB = BS * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[3 * TB];
  char* ks = smem;           // K block, row-major
  char* vs = smem + TB;      // V block, row-major
  char* kts = smem + 2 * TB; // K block, transposed (keys permuted)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int N = p.N;
  const int ntiles = (N + BM - 1) / BM;
  const int lid = work_id();
  const int bh = lid / ntiles;
  int tile = lid % ntiles;
  if (CAUSAL) tile = ntiles - 1 - tile;
  const int b = bh / p.H;
  const int q0 = tile * BM;
  int kvlen = N;
  if (p.kv_lens) kvlen = min(max(p.kv_lens[b], 0), N);
  int kend = kvlen;
  if (CAUSAL) kend = min(kend, q0 + BM);
  const int nblk = (kend + BS - 1) / BS;

  const size_t head = (size_t)bh * N * D;
  const __bf16* Q = (const __bf16*)p.q + head;
  const __bf16* K = (const __bf16*)p.k + head;
  const __bf16* V = (const __bf16*)p.v + head;
  const __bf16* dO = (const __bf16*)p.dout + head;

  const int qa = q0 + wave * 32;
  const int qrow = qa + n;
  const int qrow_c = min(qrow, N - 1);
  bf16x8 qf[D / 16], of[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    qf[c] = *(const bf16x8*)(Q + (size_t)qrow_c * D + 16 * c + 8 * h);
    of[c] = *(const bf16x8*)(dO + (size_t)qrow_c * D + 16 * c + 8 * h);
  }
  const float lse = p.lse[(size_t)bh * N + qrow_c];
  const float lse2 = (lse == NEG_INF) ? POS_INF : lse * LOG2E;  // empty row: P = 0
  const float dl = p.delta[(size_t)bh * N + qrow_c];
  const float scl = p.scale_log2;

  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) zero(acc[t]);

  for (int j = 0; j < nblk; ++j) {
    const int key0 = j * BS;
    __syncthreads();
    stage_rows<D, NT>(K, key0, N, ks, kts, tid);
    stage_rows<D, NT>(V, key0, N, vs, nullptr, tid);
    __syncthreads();
    if (CAUSAL && key0 > qa + 31) continue;  // wholly in this wave's future

    f32x16 s[2], dp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      zero(s[t]);
      zero(dp[t]);
    }
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = t * 32 + n;
        const int off = row * (D * 2) + row_slot<D>(row, 2 * c + h) * 16;
        s[t] = mfma32(*(const bf16x8*)(ks + off), qf[c], s[t]);
        dp[t] = mfma32(*(const bf16x8*)(vs + off), of[c], dp[t]);
      }
    const bool need_mask = (key0 + BS > kvlen) || (CAUSAL && key0 + BS - 1 > qa);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = exp2f(fmaf(s[t][r], scl, -lse2));
        if (need_mask) {
          const int key = key0 + t * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= kvlen || (CAUSAL && key > qrow)) pv = 0.f;
        }
        s[t][r] = pv * (dp[t][r] - dl);  // dS^T
      }
    bf16x8 df[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pack_bf16x2(s[kc >> 1][8 * (kc & 1) + 2 * e], s[kc >> 1][8 * (kc & 1) + 2 * e + 1]);
      df[kc] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const int drow = t * 32 + n;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16x8 a = *(const bf16x8*)(kts + drow * (BS * 2) + t64_slot(drow, 2 * kc + h) * 16);
        acc[t] = mfma32(a, df[kc], acc[t]);
      }
    }
  }

  if (qrow < N) store_rowT<D>((__bf16*)p.dq + head + (size_t)qrow * D, acc, p.scale, h);
}

// ---- dK, dV: one workgroup per 32*NW keys ----
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int BK = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int TB = BS * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[4 * TB];
  __shared__ __attribute__((aligned(16))) float lse2s[BS];
  __shared__ __attribute__((aligned(16))) float dls[BS];
  char* qs = smem;            // Q block, row-major
  char* os = smem + TB;       // dO block, row-major
  char* qts = smem + 2 * TB;  // Q block, transposed (queries permuted)
  char* ots = smem + 3 * TB;  // dO block, transposed (queries permuted)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int N = p.N;
  const int ntiles = (N + BK - 1) / BK;
  const int lid = work_id();
  const int bh = lid / ntiles;
  const int tile = lid % ntiles;  // low key tiles see the most queries: they go first
  const int b = bh / p.H;
  const int kb0 = tile * BK;
  int kvlen = N;
  if (p.kv_lens) kvlen = min(max(p.kv_lens[b], 0), N);

  const size_t head = (size_t)bh * N * D;
  const __bf16* Q = (const __bf16*)p.q + head;
  const __bf16* K = (const __bf16*)p.k + head;
  const __bf16* V = (const __bf16*)p.v + head;
  const __bf16* dO = (const __bf16*)p.dout + head;
  const float* lse = p.lse + (size_t)bh * N;
  const float* delta = p.delta + (size_t)bh * N;

  const int kw0 = kb0 + wave * 32;
  const int key = kw0 + n;
  const int key_c = min(key, N - 1);
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    kf[c] = *(const bf16x8*)(K + (size_t)key_c * D + 16 * c + 8 * h);
    vf[c] = *(const bf16x8*)(V + (size_t)key_c * D + 16 * c + 8 * h);
  }
  const float scl = p.scale_log2;

  f32x16 dva[D / 32], dka[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    zero(dva[t]);
    zero(dka[t]);
  }

  const int nqb = (N + BS - 1) / BS;
  const int qstart = CAUSAL ? kb0 / BS : 0;
  const bool active = kb0 < kvlen;  // otherwise every key of the tile is hidden
  for (int ib = active ? qstart : nqb; ib < nqb; ++ib) {
    const int qb0 = ib * BS;
    __syncthreads();
    stage_rows<D, NT>(Q, qb0, N, qs, qts, tid);
    stage_rows<D, NT>(dO, qb0, N, os, ots, tid);
    if (tid < BS) {
      const int qi = min(qb0 + tid, N - 1);
      const float l = lse[qi];
      lse2s[tid] = (l == NEG_INF) ? POS_INF : l * LOG2E;
      dls[tid] = delta[qi];
    }
    __syncthreads();
    if (kw0 >= kvlen) continue;                    // all of this wave's keys are hidden
    if (CAUSAL && kw0 > qb0 + BS - 1) continue;    // every query of the block precedes them

    const bool need_mask =
        (kw0 + 31 >= kvlen) || (qb0 + BS > N) || (CAUSAL && kw0 + 31 > qb0);
    f32x16 pt[2], dst[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      f32x16 s, dp;
      zero(s);
      zero(dp);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const int row = qt * 32 + n;
        const int off = row * (D * 2) + row_slot<D>(row, 2 * c + h) * 16;
        s = mfma32(*(const bf16x8*)(qs + off), kf[c], s);
        dp = mfma32(*(const bf16x8*)(os + off), vf[c], dp);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ql = qt * 32 + 8 * g + 4 * h;  // four consecutive queries
        const f32x4 l4 = *(const f32x4*)(lse2s + ql);
        const f32x4 d4 = *(const f32x4*)(dls + ql);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pv = exp2f(fmaf(s[r], scl, -l4[e]));
          if (need_mask) {
            const int query = qb0 + ql + e;
            if (key >= kvlen || query >= N || (CAUSAL && key > query)) pv = 0.f;
          }
          pt[qt][r] = pv;
          dst[qt][r] = pv * (dp[r] - d4[e]);
        }
      }
    }
    bf16x8 pf[4], df[4];
#pragma unroll
    for (int qc = 0; qc < 4; ++qc) {
      u32x4 wp, wd;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * (qc & 1) + 2 * e;
        wp[e] = pack_bf16x2(pt[qc >> 1][r], pt[qc >> 1][r + 1]);
        wd[e] = pack_bf16x2(dst[qc >> 1][r], dst[qc >> 1][r + 1]);
      }
      pf[qc] = __builtin_bit_cast(bf16x8, wp);
      df[qc] = __builtin_bit_cast(bf16x8, wd);
    }
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const int drow = t * 32 + n;
#pragma unroll
      for (int qc = 0; qc < 4; ++qc) {
        const int off = drow * (BS * 2) + t64_slot(drow, 2 * qc + h) * 16;
        dva[t] = mfma32(*(const bf16x8*)(ots + off), pf[qc], dva[t]);
        dka[t] = mfma32(*(const bf16x8*)(qts + off), df[qc], dka[t]);
      }
    }
  }

  if (key < N) {
    store_rowT<D>((__bf16*)p.dk + head + (size_t)key * D, dka, p.scale, h);
    store_rowT<D>((__bf16*)p.dv + head + (size_t)key * D, dva, 1.f, h);
  }
}

template <int D, int NW>
hipError_t launch_d(const BwdParams& p, hipStream_t stream) {
  const long long rows = (long long)p.B * p.H * p.N;
  const long long rpb = 256 / (D / 8);
  const long long g0 = (rows + rpb - 1) / rpb;
  const long long BM = 32 * NW;
  const long long g1 = (long long)p.B * p.H * ((p.N + BM - 1) / BM);
  if (g0 > 0x7fffffffLL || g1 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)g0), dim3(256), 0, stream, p);
  if (p.causal) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, true>), dim3((unsigned)g1), dim3(NW * 64), 0,
                       stream, p);
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, true>), dim3((unsigned)g1), dim3(NW * 64), 0, stream,
                       p);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, false>), dim3((unsigned)g1), dim3(NW * 64), 0,
                       stream, p);
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, false>), dim3((unsigned)g1), dim3(NW * 64), 0,
                       stream, p);
  }
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  const size_t bytes = (size_t)B * H * N * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  if (p.d == 128) return launch_d<128, 4>(p, stream);
  if (p.d == 64) return launch_d<64, 4>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
