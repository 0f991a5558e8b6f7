// Exact attention backward for gfx950 (bf16 or fp16 tensors, fp32
// accumulation): P recomputed from the saved logsumexp.
//
// The pages say only that the backward pass recomputes S and P from Q, K, V
// instead of storing them ("Question bank", the recomputation answers); the
// formulas are the standard derivative of softmax attention:
//   P = exp(S - lse) (0 where hidden or lse = -inf),  D_i = sum_c dO_ic O_ic,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,
//   dK = scale dS^T Q.
// Two kernels, no atomics, in this order:
//   dq     one workgroup per 128 query rows first forms D_i and
//          lse_i*log2(e) (+inf for an empty row, so that P = 0) for its rows
//          and stores them in the caller's workspace, then streams the
//          visible key blocks (64 keys, 32 at D = 256): S^T = K Q^T,
//          dP^T = V dO^T, dS^T, dQ^T += K^T dS^T (the forward's transposed
//          layout: one query per lane pair);
//   dkdv   one workgroup per 128 keys streams the blocks of 32 queries that
//          see them, with their D and lse*log2(e) from the workspace:
//          S = Q K^T, dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS
//          (one key per lane pair).
// Streamed blocks go from HBM to LDS with direct 16-byte loads into a double
// buffer, stored once, row-major. The same copy is read two ways: as rows
// (ds_read_b128, the A operand of the S / dP products) and transposed
// (ds_read_b64_tr_b16, the A operand of the products that contract over the
// streamed rows). The 16-byte chunks of a row are XOR-swizzled with a pattern
// that keeps both kinds of read free of bank conflicts. Contraction slots over
// the streamed rows follow the order in which a 32x32 accumulator holds its
// rows (bits 2 and 3 swapped), as in the forward kernel.
#include "fa_internal.h"
#include "fa_device.h"

#include <math.h>

#include <type_traits>

namespace fa {
namespace {

using namespace dev;

constexpr int BS = 32;   // streamed query rows per block in dkdv
constexpr int NWB = 4;   // waves per workgroup
constexpr int BT = 32 * NWB;  // rows owned by a workgroup (queries in dq, keys in dkdv)
static_assert(BT == BWD_BT, "workgroup rows match the host's work-order rule");

// Waves per SIMD each kernel's register budget is sized for.
#ifndef FA_BWD_DQ_OCC
#define FA_BWD_DQ_OCC 2
#endif
#ifndef FA_BWD_DKDV128_OCC
#define FA_BWD_DKDV128_OCC 2
#endif

// 16-byte chunk c of row `row` of a streamed tile is stored at slot
// tslot(row, c): 16 consecutive rows read at one chunk, and 8 consecutive
// rows read 4 chunks each by the transpose reads, both spread evenly over the
// LDS banks. An XOR of the chunk index, except for the 12-chunk rows of
// D = 96, which rotate by (row / 4) mod 4 instead.
template <int D>
__device__ __forceinline__ int tslot(int row, int c) {
  static_assert(D == 32 || D == 64 || D == 96 || D == 128 || D == 256, "head dimension");
  if constexpr (D >= 128) {  // rows of 256 or 512 bytes: every row starts at bank 0
    return c ^ (4 * (row & 3) + ((row >> 2) & 3));
  } else if constexpr (D == 64) {
    return c ^ (((row >> 1) & 1) | (((row >> 2) & 1) << 2) | (((row >> 3) & 1) << 1));
  } else if constexpr (D == 32) {
    return c ^ ((row >> 2) & 3);
  } else {
    return (c + ((row >> 2) & 3)) % 12;
  }
}
// The chunk stored at slot s of row `row` (the inverse permutation).
template <int D>
__device__ __forceinline__ int tchunk(int row, int s) {
  if constexpr (D == 96) {
    return (s + 12 - ((row >> 2) & 3)) % 12;
  } else {
    return tslot<D>(row, s);
  }
}


// Work order. Workgroups are dispatched in id order, round-robin over the 8
// XCDs (id % 8). Tile-major (seq = 0): workgroup id w takes tile rank
// w / (B*H) of head w % (B*H), so each XCD starts with the heaviest tiles
// and, when B*H is a multiple of 8, keeps to a fixed set of heads (x, x+8,
// ...). Head-sequential (seq = 1, B*H a multiple of 8): XCD x takes the same
// heads but runs them one after another, rank-major within a head, so that
// few heads' streamed operands share its L2 at a time.
__device__ __forceinline__ int tile_rank(int BH, int nt, int seq) {
  if (seq && (BH & 7) == 0) return (blockIdx.x >> 3) % nt;
  return blockIdx.x / BH;
}
__device__ __forceinline__ int tile_head(int BH, int nt, int seq) {
  if (seq && (BH & 7) == 0) return (blockIdx.x & 7) + 8 * ((blockIdx.x >> 3) / nt);
  return blockIdx.x % BH;
}

// DMA of rows [r0, r0 + ROWS) of two row-major [N, D] 16-bit matrices X0, X1
// into LDS tiles dst0, dst1 (rows past N repeat row N-1; they are masked by
// the callers; r0 < N). Each DMA fills 1 KB (64 lanes x 16 bytes) of a tile
// with a buffer load into LDS from a resource based at row r0 (a 32-bit
// per-lane offset, no vector address arithmetic; the compiler counts these
// only in vmcnt, so LDS operand reads are still waited for by count). Where
// a tile splits into whole rows per DMA and evenly over the waves (D = 64,
// 128, 256, and D = 32 for 64 rows), every wave loads its share of both
// tiles; otherwise (D = 96, D = 32 for 32 rows) the DMAs of both tiles form
// one list dealt round-robin over the waves,
// lane l of DMA b covering slot 64 b + l of its tile in row-major order.
template <int D, int ROWS = BS>
__device__ __forceinline__ void issue_tiles(const void* __restrict__ X0v,
                                            const void* __restrict__ X1v, int r0, int N,
                                            char* dst0, char* dst1, int wave, int lane) {
  constexpr int ROWB = D * 2;
  constexpr int CPR = ROWB / 16;
  constexpr int DMA_PER_TILE = ROWS * ROWB / 1024;
  static_assert((2 * DMA_PER_TILE) % NWB == 0, "the DMAs of two tiles split evenly over the waves");
  const buffer_rsrc b0 = make_rsrc((const char*)X0v + (size_t)r0 * ROWB);
  const buffer_rsrc b1 = make_rsrc((const char*)X1v + (size_t)r0 * ROWB);
  const int last = N - 1 - r0;  // last row of the matrix, relative to r0
  if constexpr (1024 % ROWB == 0 && DMA_PER_TILE % NWB == 0) {
    constexpr int DPW = DMA_PER_TILE / NWB;
    constexpr int ROWS_PER_DMA = 1024 / ROWB;
#pragma unroll
    for (int e = 0; e < DPW; ++e) {
      const int blk = wave * DPW + e;
      const int row = blk * ROWS_PER_DMA + lane / CPR;
      const int off = min(row, last) * ROWB + tchunk<D>(row, lane % CPR) * 16;
      dma16_buf(b0, off, dst0 + blk * 1024);
      dma16_buf(b1, off, dst1 + blk * 1024);
    }
  } else {
#pragma unroll
    for (int m = 0; m < 2 * DMA_PER_TILE / NWB; ++m) {
      const int e = wave + NWB * m;  // wave-uniform
      const bool second = e >= DMA_PER_TILE;
      const int blk = second ? e - DMA_PER_TILE : e;
      const int g = 64 * blk + lane;
      const int row = g / CPR;
      const int off = min(row, last) * ROWB + tchunk<D>(row, g % CPR) * 16;
      dma16_buf(second ? b1 : b0, off, (second ? dst1 : dst0) + blk * 1024);
    }
  }
}

// Per-lane offsets of the two kinds of operand read of a streamed tile.
//  row read:  A operand rows n (of 32), logical chunk 2c + h     -> roff[c]
//  tr read:   A operand d rows dt*32 + (lane%32), slots over the streamed rows
//             16*kc + 8*r + 4*h + (lane%16)/4                     -> toff[dt][r]
//             (+ kc*16 rows, an immediate offset)
template <int D>
struct TileOffsets {
  int roff[D / 16];
  int toff[D / 32][2];
  __device__ __forceinline__ TileOffsets(int lane) {
    constexpr int ROWB = D * 2;
    const int n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) roff[c] = n * ROWB + tslot<D>(n, 2 * c + h) * 16;
    const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int vrow = 4 * h + ((lane & 15) >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = 8 * r + vrow;
        const int col = dt * 32 + vcol;
        toff[dt][r] = row * ROWB + tslot<D>(row, col >> 3) * 16 + (col & 7) * 2;
      }
  }
};

// Transposed A operand (d rows dt*32.., streamed-row chunk kc) of a tile.
template <typename X8, int D>
__device__ __forceinline__ X8 tr_operand(const char* tile, const TileOffsets<D>& o, int dt,
                                             int kc) {
  constexpr int ROWB = D * 2;
  const i16x4 lo = lds_read_tr16(tile + kc * 16 * ROWB + o.toff[dt][0]);
  const i16x4 hi = lds_read_tr16(tile + kc * 16 * ROWB + o.toff[dt][1]);
  return __builtin_bit_cast(X8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Store a transposed accumulator (lane = one output row, registers = D
// columns in groups of 4) as T, times `mul`.
template <typename T, int D>
__device__ __forceinline__ void store_rowT(T* dst, const f32x16* acc, float mul, int h) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = Elem<T>::pack(acc[t][4 * g] * mul, acc[t][4 * g + 1] * mul);
      w[1] = Elem<T>::pack(acc[t][4 * g + 2] * mul, acc[t][4 * g + 3] * mul);
      *(u32x2*)(dst + t * 32 + 8 * g + 4 * h) = w;
    }
}

// ---- dQ: one workgroup per 128 query rows ----
// Keys stream in blocks of BN (64 at D <= 128, 32 at D = 256, where the
// registers would not hold two score tiles).
constexpr int dq_block_keys(int D) { return D <= 128 ? 64 : 32; }

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(NWB * 64, D == 256 ? 1 : FA_BWD_DQ_OCC) void bwd_dq_kernel(BwdParams p) {
  typedef Elem<T> E;
  typedef typename E::x8 x8;
  constexpr int BN = dq_block_keys(D);
  constexpr int KT = BN / 32;  // 32-key tiles per block
  constexpr int KC = BN / 16;  // 16-key contraction chunks per block
  constexpr int ROWB = D * 2;
  constexpr int TB = BN * ROWB;
  constexpr int DC = D / 16, DT = D / 32;
  // K and V blocks, row-major, one LDS object per stage (so that the
  // compiler sees that the next block's DMA cannot alias this block's reads
  // and does not wait for it before them).
  __shared__ __attribute__((aligned(1024))) char kbuf0[TB];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TB];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TB];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
  const int n = lane & 31, h = lane >> 5;
  const int N = p.N;
  const int ntiles = (N + BT - 1) / BT;
  const int bh = tile_head(p.B * p.H, ntiles, p.seq_dq);
  int tile = tile_rank(p.B * p.H, ntiles, p.seq_dq);
  if (CAUSAL) tile = ntiles - 1 - tile;  // the latest query rows see the most keys
  const int b = bh / p.H;
  const int q0 = tile * BT;
  const int Nk = p.Nk;
  const int shift = CAUSAL ? Nk - N - p.diag : 0;  // causal: key visible iff key <= query + shift
  int kvlen = Nk;
  if (p.kv_lens) kvlen = min(max(p.kv_lens[b], 0), Nk);
  int kend = kvlen;
  if (CAUSAL) kend = max(min(kend, q0 + BT + shift), 0);
  const int nblk = (kend + BN - 1) / BN;

  const size_t head = (size_t)bh * N * D;
  const size_t kvhead = ((size_t)b * p.Hkv + (bh % p.H) / (p.H / p.Hkv)) * Nk * D;
  const T* Q = (const T*)p.q + head;
  const T* K = (const T*)p.k + kvhead;
  const T* V = (const T*)p.v + kvhead;
  const T* dO = (const T*)p.dout + head;
  const T* O = (const T*)p.o + head;

  const int qa = q0 + wave * 32;
  const int qrow = qa + n;
  const int qrow_c = min(qrow, N - 1);
  x8 qf[DC], of[DC];
  float dpart = 0.f;  // this lane's half of D_i = sum_c dO_ic O_ic
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    qf[c] = *(const x8*)(Q + (size_t)qrow_c * D + 16 * c + 8 * h);
    of[c] = *(const x8*)(dO + (size_t)qrow_c * D + 16 * c + 8 * h);
    const u32x4 a = __builtin_bit_cast(u32x4, *(const x8*)(O + (size_t)qrow_c * D + 16 * c + 8 * h));
    const u32x4 g = __builtin_bit_cast(u32x4, of[c]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dpart = fmaf(E::lo(a[e]), E::lo(g[e]), dpart);
      dpart = fmaf(E::hi(a[e]), E::hi(g[e]), dpart);
    }
  }
  const float dl = dpart + __shfl_xor(dpart, 32);  // lanes n and n + 32 hold the two halves
  const float lse_row = p.lse[(size_t)bh * N + qrow_c];
  const float lse2 = (lse_row == NEG_INF) ? POS_INF : lse_row * LOG2E;  // empty row: P = 0
  if (h == 0 && qrow < N) {  // for the dK/dV kernel, which runs next
    p.delta[(size_t)bh * N + qrow] = dl;
    p.lse2[(size_t)bh * N + qrow] = lse2;
  }
  __builtin_amdgcn_sched_barrier(0);
  const float scl = p.scale_log2;
  const TileOffsets<D> off(lane);

  f32x16 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) zero(acc[t]);

  // Block j lives in stage j % 2; the loop is unrolled by the two stages so
  // that every buffer is a compile-time choice.
  auto issue = [&](int j, auto stage) {
    constexpr int SD = decltype(stage)::value;
    if (j >= nblk) return;
    issue_tiles<D, BN>(K, V, j * BN, Nk, SD == 0 ? kbuf0 : kbuf1, SD == 0 ? vbuf0 : vbuf1, wave,
                       lane);
  };
  auto step = [&](int j, auto stage) {
    constexpr int ST = decltype(stage)::value;
    wait_vmem();
    __syncthreads();
    issue(j + 1, std::integral_constant<int, 1 - ST>());
    const int key0 = j * BN;
    if (CAUSAL && key0 > qa + 31 + shift) return;  // wholly in this wave's future
    const char* ks = ST == 0 ? kbuf0 : kbuf1;
    const char* vs = ST == 0 ? vbuf0 : vbuf1;

    __builtin_amdgcn_s_setprio(1);
    f32x16 s[KT], dp[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      zero(s[t]);
      zero(dp[t]);
    }
    if constexpr (KT == 2) {
      // Two key tiles: the operands of both would not fit the registers, so
      // the reads roll one chunk ahead over the 2 * DC chunks (K, then V):
      // the reads of chunk c+1 go out before the MFMAs of chunk c.
#pragma unroll
      for (int c = 0; c < DC; ++c)
#pragma unroll
        for (int t = 0; t < KT; ++t) s[t] = E::mfma(*(const x8*)(ks + t * 32 * ROWB + off.roff[c]), qf[c], s[t]);
#pragma unroll
      for (int c = 0; c < DC; ++c)
#pragma unroll
        for (int t = 0; t < KT; ++t) dp[t] = E::mfma(*(const x8*)(vs + t * 32 * ROWB + off.roff[c]), of[c], dp[t]);
      __builtin_amdgcn_sched_group_barrier(0x100, KT, 0);
#pragma unroll
      for (int c = 0; c < 2 * DC; ++c) {
        if (c + 1 < 2 * DC) __builtin_amdgcn_sched_group_barrier(0x100, KT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, KT, 0);
      }
    } else {
      // One tile at D = 256, where the operands would not fit the registers.
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        s[0] = E::mfma(*(const x8*)(ks + off.roff[c]), qf[c], s[0]);
        dp[0] = E::mfma(*(const x8*)(vs + off.roff[c]), of[c], dp[0]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // Hidden keys (only in blocks that straddle the diagonal or kv_len): the
    // score becomes -inf, so its P is exactly 0. A uniform branch of its own,
    // so unmasked blocks pay nothing for it.
    const bool need_mask = (key0 + BN > kvlen) || (CAUSAL && key0 + BN - 1 > qa + shift);
    if (need_mask) {
      int lim = kvlen - 1;  // key visible iff key <= lim
      if (CAUSAL) lim = min(lim, qrow + shift);
      lim -= key0 + 4 * h;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t * 32 + 8 * (r >> 2) + (r & 3) > lim) s[t][r] = NEG_INF;
    }
    x8 df[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 8 * (kc & 1) + 2 * e + u;
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[kc >> 1][r], scl, -lse2));
          v2[u] = pv * (dp[kc >> 1][r] - dl);  // dS^T
        }
        w[e] = E::pack(v2[0], v2[1]);
      }
      df[kc] = __builtin_bit_cast(x8, w);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) acc[dt] = E::mfma(tr_operand<x8, D>(ks, off, dt, kc), df[kc], acc[dt]);
    {
      // Transposed operand reads (two per product) two products ahead.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < DT * KC; ++i) {
        if (i + 2 < DT * KC) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  issue(0, std::integral_constant<int, 0>());
  for (int j = 0; j < nblk; j += 2) {
    step(j, std::integral_constant<int, 0>());
    if (j + 1 < nblk) step(j + 1, std::integral_constant<int, 1>());
  }
  wait_vmem();

  if (qrow < N) store_rowT<T, D>((T*)p.dq + head + (size_t)qrow * D, acc, p.scale, h);
}

// ---- dK, dV: one workgroup per 128 keys of a K/V head, summed over the
// query heads that share it ----
// OUT selects the gradients computed: DKDV_V | DKDV_K in one pass, or (at
// D = 256, where both sets of accumulators and both operand sets exceed the
// register file) one of them per pass; the dV pass skips dP and dS.
constexpr int DKDV_V = 1, DKDV_K = 2;
constexpr int dkdv_waves_per_simd(int D) { return D == 256 ? 1 : (D == 128 ? FA_BWD_DKDV128_OCC : 2); }

template <typename T, int D, bool CAUSAL, int OUT>
__global__ __launch_bounds__(NWB * 64, dkdv_waves_per_simd(D)) void bwd_dkdv_kernel(BwdParams p) {
  typedef Elem<T> E;
  typedef typename E::x8 x8;
  constexpr int TB = BS * D * 2;
  constexpr int DC = D / 16, DT = D / 32;
  // Q and dO blocks (row-major) and their lse*log2(e), then D values: one
  // LDS object per stage, as in the dQ kernel.
  __shared__ __attribute__((aligned(1024))) char qbuf0[TB];
  __shared__ __attribute__((aligned(1024))) char qbuf1[TB];
  __shared__ __attribute__((aligned(1024))) char obuf0[TB];
  __shared__ __attribute__((aligned(1024))) char obuf1[TB];
  __shared__ __attribute__((aligned(16))) float stat0[64];
  __shared__ __attribute__((aligned(16))) float stat1[64];
  // At D = 128 the K operand fragments of this workgroup's keys wait in LDS
  // (32 KB; each lane reads back its own 16-byte slots, free of bank
  // conflicts) rather than in 32 registers: with them in registers the
  // kernel exceeds the 256 registers of two waves per SIMD, and the spill
  // reload waits for every outstanding load, the next block's DMA included.
  constexpr bool KF_LDS = (D == 128) && (OUT == (DKDV_V | DKDV_K));
  __shared__ __attribute__((aligned(1024))) char kfl[KF_LDS ? NWB * DC * 1024 : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
  const int n = lane & 31, h = lane >> 5;
  const int N = p.N, Nk = p.Nk;
  const int G = p.H / p.Hkv;  // query heads per K/V head
  const int ntk = (p.Nk + BT - 1) / BT;
  const int bkv = tile_head(p.B * p.Hkv, ntk, p.seq_dkdv);
  const int tile = tile_rank(p.B * p.Hkv, ntk, p.seq_dkdv);  // the earliest keys are seen by the most queries
  const int b = bkv / p.Hkv;
  const int kb0 = tile * BT;
  const int shift = CAUSAL ? Nk - N - p.diag : 0;  // causal: key visible iff key <= query + shift
  int kvlen = Nk;
  if (p.kv_lens) kvlen = min(max(p.kv_lens[b], 0), Nk);

  const size_t kvhead = (size_t)bkv * Nk * D;
  const size_t qhead0 = (size_t)bkv * G;  // first query head of the group (b * H + hk * G)
  const T* K = (const T*)p.k + kvhead;
  const T* V = (const T*)p.v + kvhead;

  const int kw0 = kb0 + wave * 32;
  const int key = kw0 + n;
  const int key_c = min(key, Nk - 1);
  x8 kf[KF_LDS ? 1 : DC], vf[(OUT & DKDV_K) ? DC : 1];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    const x8 kc = *(const x8*)(K + (size_t)key_c * D + 16 * c + 8 * h);
    if constexpr (KF_LDS)
      *(x8*)(kfl + (wave * DC + c) * 1024 + lane * 16) = kc;  // read back by this lane only
    else
      kf[c] = kc;
    if constexpr ((OUT & DKDV_K) != 0) vf[c] = *(const x8*)(V + (size_t)key_c * D + 16 * c + 8 * h);
  }
  __builtin_amdgcn_sched_barrier(0);
  const float scl = p.scale_log2;
  const TileOffsets<D> off(lane);

  f32x16 dva[DT], dka[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    zero(dva[t]);
    zero(dka[t]);
  }

  // Query blocks [qstart, nqb) of each of the G query heads, one stream:
  // step u is block qstart + u % nq of group head u / nq.
  const int nqb = (N + BS - 1) / BS;
  const int qstart = CAUSAL ? min(max(kb0 - shift, 0) / BS, nqb) : 0;
  const int nq = nqb - qstart;
  const int nsteps = (kb0 < kvlen) ? G * nq : 0;  // every key of the tile hidden: nothing to do
  // Step u streams query block i of group head g (u = g * nq + i - qstart);
  // (i, g) advance with u, so no step divides by nq.
  auto issue = [&](int u, int i, int g, auto stage) {
    constexpr int SD = decltype(stage)::value;
    if (u >= nsteps) return;
    const size_t qh = qhead0 + g;
    issue_tiles<D>((const T*)p.q + qh * N * D, (const T*)p.dout + qh * N * D, i * BS, N,
                   SD == 0 ? qbuf0 : qbuf1, SD == 0 ? obuf0 : obuf1, wave, lane);
    if (wave == 0) {  // 32 lse*log2(e) then 32 D values, 4 bytes per lane
      const size_t row0 = qh * N + (size_t)i * BS;  // the block's first row
      const int off = min(lane & 31, N - 1 - i * BS) * 4;
      float* dst = SD == 0 ? stat0 : stat1;
      if (lane < 32)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(p.lse2 + row0), (lds_void*)dst, 4, off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(p.delta + row0), (lds_void*)dst, 4, off, 0, 0, 0);
    }
  };
  // Step u uses stage u % 2; unrolled by the two stages as in the dQ kernel.
  int cur_i = qstart, cur_g = 0;  // block of the current step
  auto step = [&](int u, auto stage) {
    constexpr int ST = decltype(stage)::value;
    wait_vmem();
    __syncthreads();
    const int qb0 = cur_i * BS;
    int ni = cur_i + 1, ng = cur_g;
    if (ni == nqb) {
      ni = qstart;
      ++ng;
    }
    issue(u + 1, ni, ng, std::integral_constant<int, 1 - ST>());
    cur_i = ni;
    cur_g = ng;
    if (kw0 >= kvlen) return;                         // all of this wave's keys are hidden
    if (CAUSAL && kw0 > qb0 + BS - 1 + shift) return;  // every query of the block precedes them
    const char* qs = ST == 0 ? qbuf0 : qbuf1;
    const char* os = ST == 0 ? obuf0 : obuf1;
    const float* st = ST == 0 ? stat0 : stat1;

    if constexpr (OUT == (DKDV_V | DKDV_K)) {
      // Both gradients: the two products that need only the streamed rows
      // (S and dP) first, then P and dS on the VALU, then the two products
      // that need them (dV^T and dK^T). Two matrix phases per block, so the
      // other wave of the SIMD has long stretches of matrix work to overlap
      // with this wave's exponentials.
      __builtin_amdgcn_s_setprio(1);
      f32x16 s, dp;
      zero(s);
      zero(dp);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        x8 kc;
        if constexpr (KF_LDS)
          kc = *(const x8*)(kfl + (wave * DC + c) * 1024 + lane * 16);
        else
          kc = kf[c];
        s = E::mfma(*(const x8*)(qs + off.roff[c]), kc, s);
      }
#pragma unroll
      for (int c = 0; c < DC; ++c) dp = E::mfma(*(const x8*)(os + off.roff[c]), vf[c], dp);
      {
        // Operand reads two products ahead: an S product reads a Q row chunk
        // (and, from LDS, its K fragment), a dP product a dO row chunk.
        constexpr int RS = KF_LDS ? 2 : 1;  // reads per S product
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * RS, 0);
#pragma unroll
        for (int i = 0; i < 2 * DC; ++i) {
          const int nxt = i + 2;  // the product whose operands are read now
          const int r = nxt < DC ? RS : (nxt < 2 * DC ? 1 : 0);
          if (r == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          if (r == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      const bool need_mask = (kw0 + 31 >= kvlen) || (qb0 + BS > N) || (CAUSAL && kw0 + 31 > qb0 + shift);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int query = qb0 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= kvlen || query >= N || (CAUSAL && key > query + shift)) s[r] = NEG_INF;
        }
      }
      x8 pf[2], df[2];
#pragma unroll
      for (int qc = 0; qc < 2; ++qc) {
        u32x4 wp, wd;
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int g = 2 * qc + g2;
          const f32x4 l4 = *(const f32x4*)(st + 8 * g + 4 * h);
          const f32x4 d4 = *(const f32x4*)(st + 32 + 8 * g + 4 * h);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 4 * g + 2 * e;
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[r], scl, -l4[2 * e]));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], scl, -l4[2 * e + 1]));
            wp[2 * g2 + e] = E::pack(p0, p1);
            wd[2 * g2 + e] = E::pack(p0 * (dp[r] - d4[2 * e]), p1 * (dp[r + 1] - d4[2 * e + 1]));
          }
        }
        pf[qc] = __builtin_bit_cast(x8, wp);
        df[qc] = __builtin_bit_cast(x8, wd);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qc = 0; qc < 2; ++qc)
          dva[dt] = E::mfma(tr_operand<x8, D>(os, off, dt, qc), pf[qc], dva[dt]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) dka[dt] = E::mfma(tr_operand<x8, D>(qs, off, dt, qc), df[qc], dka[dt]);
      {
        // Transposed operand reads (two per product) two products ahead.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 4 * DT; ++i) {
          if (i + 2 < 4 * DT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      return;
    }
    // One gradient per pass (D = 256): phases in order, each value dead as
    // soon as it is consumed: S, P, dV^T (needs P), dP, dS (needs P and dP),
    // dK^T.
    __builtin_amdgcn_s_setprio(1);
    f32x16 s;
    zero(s);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      x8 kc;
      if constexpr (KF_LDS)
        kc = *(const x8*)(kfl + (wave * DC + c) * 1024 + lane * 16);
      else
        kc = kf[c];
      s = E::mfma(*(const x8*)(qs + off.roff[c]), kc, s);
    }
    __builtin_amdgcn_s_setprio(0);
    // Hidden pairs (only in blocks that straddle the diagonal, kv_len or the
    // last query row): the score becomes -inf, so its P is exactly 0. A
    // uniform branch of its own, so unmasked blocks pay nothing for it.
    const bool need_mask = (kw0 + 31 >= kvlen) || (qb0 + BS > N) || (CAUSAL && kw0 + 31 > qb0 + shift);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int query = qb0 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key >= kvlen || query >= N || (CAUSAL && key > query + shift)) s[r] = NEG_INF;
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int ql = 8 * g + 4 * h;  // four consecutive queries of this lane
      const f32x4 l4 = *(const f32x4*)(st + ql);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], scl, -l4[e]));  // P, fp32
      }
    }
    x8 pf[2];
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = E::pack(s[8 * qc + 2 * e], s[8 * qc + 2 * e + 1]);
      pf[qc] = __builtin_bit_cast(x8, w);
    }
    __builtin_amdgcn_s_setprio(1);
    if constexpr ((OUT & DKDV_V) != 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qc = 0; qc < 2; ++qc)
          dva[dt] = E::mfma(tr_operand<x8, D>(os, off, dt, qc), pf[qc], dva[dt]);
    }
    if constexpr ((OUT & DKDV_K) == 0) {
      __builtin_amdgcn_s_setprio(0);
      return;
    }
    f32x16 dp;
    zero(dp);
#pragma unroll
    for (int c = 0; c < DC; ++c) dp = E::mfma(*(const x8*)(os + off.roff[c]), vf[c], dp);
    __builtin_amdgcn_s_setprio(0);
    x8 df[2];
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
      u32x4 w;
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const int g = 2 * qc + g2;
        const f32x4 d4 = *(const f32x4*)(st + 32 + 8 * g + 4 * h);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 4 * g + 2 * e;
          w[2 * g2 + e] = E::pack(s[r] * (dp[r] - d4[2 * e]), s[r + 1] * (dp[r + 1] - d4[2 * e + 1]));
        }
      }
      df[qc] = __builtin_bit_cast(x8, w);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int qc = 0; qc < 2; ++qc) dka[dt] = E::mfma(tr_operand<x8, D>(qs, off, dt, qc), df[qc], dka[dt]);
    __builtin_amdgcn_s_setprio(0);
  };
  issue(0, qstart, 0, std::integral_constant<int, 0>());
  for (int u = 0; u < nsteps; u += 2) {
    step(u, std::integral_constant<int, 0>());
    if (u + 1 < nsteps) step(u + 1, std::integral_constant<int, 1>());
  }
  wait_vmem();

  if (key < Nk) {
    if constexpr ((OUT & DKDV_K) != 0)
      store_rowT<T, D>((T*)p.dk + kvhead + (size_t)key * D, dka, p.scale, h);
    if constexpr ((OUT & DKDV_V) != 0)
      store_rowT<T, D>((T*)p.dv + kvhead + (size_t)key * D, dva, 1.f, h);
  }
}

template <typename T, int D, bool CAUSAL>
void launch_grads(const BwdParams& p, long long g1, long long g2, hipStream_t stream) {
  const dim3 blk(NWB * 64);
  // dQ first: it stores the per-row D and lse*log2(e) the dK/dV kernel reads.
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL>), dim3((unsigned)g1), blk, 0, stream, p);
  if constexpr (D == 256) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, DKDV_V>), dim3((unsigned)g2), blk, 0, stream,
                       p);
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, DKDV_K>), dim3((unsigned)g2), blk, 0, stream,
                       p);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, DKDV_V | DKDV_K>), dim3((unsigned)g2), blk, 0,
                       stream, p);
  }
}

template <typename T, int D>
hipError_t launch_d(const BwdParams& p, hipStream_t stream) {
  const long long g1 = (long long)p.B * p.H * ((p.N + BT - 1) / BT);     // dQ: query tiles
  const long long g2 = (long long)p.B * p.Hkv * ((p.Nk + BT - 1) / BT);  // dK, dV: key tiles
  if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.causal)
    launch_grads<T, D, true>(p, g1, g2, stream);
  else
    launch_grads<T, D, false>(p, g1, g2, stream);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  const size_t rows = (size_t)B * H * N;
  const size_t one = (rows * sizeof(float) + 255) & ~(size_t)255;
  return 2 * one;  // D, then lse*log2(e)
}

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
#define FA_LAUNCH(DD)                                                     \
  if (p.d == DD) {                                                        \
    if (p.dtype == DTYPE_BF16) return launch_d<__bf16, DD>(p, stream);   \
    if (p.dtype == DTYPE_F16) return launch_d<_Float16, DD>(p, stream);  \
  }
  FA_LAUNCH(32) FA_LAUNCH(64) FA_LAUNCH(96) FA_LAUNCH(128) FA_LAUNCH(256)
#undef FA_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace fa
