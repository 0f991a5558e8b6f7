// Exact attention forward for gfx950: bf16 or fp16 matrix cores, fp32 online
// softmax.
//
// One workgroup of NW = 4 waves owns BM = 128 query rows of one (batch, head)
// and streams the visible keys in blocks of BN keys through LDS, carrying per
// query row a reference max m, the running normaliser l and the unnormalised
// output (the online recurrence of the interactive explainer "The Flash
// Attention"; "Exercises", the block merges). The score block and its
// probabilities live only in registers; only Q, K, V, O and lse touch device
// memory.
//
// Layout (each wave owns 32 queries, one per lane pair):
//  * Scores are produced transposed, S^T = K Q^T, with the 32x32x16 MFMA of
//    the input type (bf16 or fp16):
//    A = a 32-key x 16-dim slice of K (LDS), B = the wave's Q^T slice (held in
//    registers for the whole kernel). In the 32x32 accumulator lane l holds
//    query (l % 32) and 16 keys, so row max and row sum are in-lane
//    reductions plus one exchange between the two lane halves.
//  * The output is accumulated transposed too, O^T += V^T P^T. B = P^T comes
//    straight from the score registers after rounding to the input type; the contraction
//    slots of the A operand are assigned to keys in the order the accumulator
//    holds them (bits 2 and 3 of the key index swapped), which the contraction
//    permits. A = V^T is read from the row-major V tile with the gfx950
//    transpose read (ds_read_b64_tr_b16): four lanes reading four key rows
//    give each lane four keys of one d column.
//  * K and V tiles go from HBM to LDS with 16-byte buffer loads straight
//    into LDS (no register staging) into two buffers: block j+1 is in flight
//    while block j is used. The 16-byte chunks of a row are permuted per row so the operand
//    reads hit every LDS bank evenly. The loop is unrolled by two so that
//    each buffer's LDS offsets are immediates, and each lane's source offsets
//    within a block are computed once.
//  * Registers are kept low enough for several waves per SIMD: their
//    interleaving hides LDS and MFMA latency and overlaps one wave's softmax
//    with another's matrix work.
//  * The per-row rescale factor is a per-lane scalar. The reference max moves
//    only when a block's max exceeds it by more than TAU (log2 units), so the
//    accumulator rescale is skipped wave-wide in almost every block; any
//    reference gives the same O = acc / l and lse = m + ln l exactly, and the
//    lag bound keeps every exponential below 2^TAU.
//  * Exponentials are base 2 (v_exp_f32) with scale*log2(e) folded into one
//    FMA. Two row sums are kept: O is divided by the sum of the rounded
//    weights that P V actually used (each output row is then a convex
//    combination of V rows even where one weight dominates), and the
//    logsumexp uses the sum of the fp32 probabilities (fp32 accuracy for the
//    backward pass).
//  * Causal: key blocks wholly in a wave's future are skipped ("Question
//    bank": blocks entirely in the future are skipped); only blocks that
//    straddle the diagonal or the padding length apply a mask.
//  * A row with no visible key keeps l = 0 and is written as O = 0 and
//    lse = -inf ("Worked examples", Cell D2).
//  * Tile order (causal): by default one tile per workgroup, the tiles that
//    see the most keys first. When one head's K and V outgrow an XCD's L2,
//    the host selects the paired instance instead: a workgroup takes tile
//    ntiles-1-r with its keys ascending, then tile r with its keys
//    descending. The online recurrence is exact in any block order ("The
//    Flash Attention"; "Exercises", a common reference), every pair streams
//    about ntiles+1 tiles' worth of blocks, and the pairs of a head read the
//    same two blocks at a time, so K and V are fetched about once per XCD.
//    On grids of 16 or more rounds of resident workgroups (and B*H a
//    multiple of 8) each XCD instead runs its heads one after another, so
//    only a few heads' K and V share its L2 at a time; the outputs are
//    bitwise the same in every order.
//  * Load balance: a host plan may cut a tile's key range into up to 16
//    parts (64 when the query rows are a single tile) processed by
//    different workgroups. Each part stores its partial
//    state (unnormalised O, reference max, both sums; fp32) and counts its
//    arrival on the tile's counter; the last part to arrive merges all parts
//    in part order with the exact block merge ("Exercises", the block
//    merges), so the result does not depend on which part finished last,
//    and resets the counter to zero. No workgroup ever waits for another.
#include "fa_internal.h"
#include "fa_device.h"

#include <math.h>

#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>

namespace fa {
namespace {

using namespace dev;

constexpr int NW = 4;         // waves per workgroup
constexpr int BM = 32 * NW;   // queries per workgroup
static_assert(BM == FWD_BM, "workgroup tile matches the host planner");
// Allowed lag of the reference max (log2 units), per element type. While the
// lag holds every weight p is at most 2^TAU: fp16 weights must stay far below
// its largest finite value (65504 = 2^16 - 2^5), so TAU = 8 there; bf16 has
// fp32's exponent range, and with TAU = 32 no weight, lane sum (at most 64
// weights), row sum or accumulator (at most 2^31 keys of weight 2^32 times
// |V|) approaches the fp32 range, while rows of widely spread scores move
// their reference far less often.
template <typename T>
constexpr float lag_tau() { return std::is_same<T, _Float16>::value ? 8.0f : 32.0f; }

#ifndef FA_PRIO_MFMA
#define FA_PRIO_MFMA 1  // wave priority (s_setprio) during the MFMA phases
#endif
#ifndef FA_FWD_WG_PER_CU
#define FA_FWD_WG_PER_CU 3
#endif

// Resident workgroups per CU the register budget is sized for (a lower bound
// for the compiler: what fits decides the occupancy). At D = 256 the Q^T
// fragments and output accumulators alone take 192 registers per lane; with
// 64-key blocks D = 128 takes 190 (two workgroups per CU) and D = 96 160
// (three); D = 64 fits 128 (four) and D = 32 96 (five).
constexpr int fwd_wg_per_cu(int D, int BN) {
  return D == 256 ? 1 : ((D == 128 || D == 96) && BN == 64 ? 2 : FA_FWD_WG_PER_CU);
}

// Head dimensions with kernel instances.
#define FA_FOR_EACH_D(X) X(32) X(64) X(96) X(128) X(256)

// PAIRED (causal only): each workgroup takes a pair of query tiles (see the
// work item below) instead of one.
template <typename T, int D, int BN, bool CAUSAL, bool PAIRED>
__global__ __launch_bounds__(NW * 64, fwd_wg_per_cu(D, BN)) void fwd_kernel(FwdParams p, FwdPlan plan) {
  static_assert(CAUSAL || !PAIRED, "pairs balance causal tiles");
  typedef Elem<T> E;
  typedef typename E::x8 x8;
  constexpr float TAU = lag_tau<T>();
  constexpr float P_BOUND = (float)(1ull << (int)TAU);  // 2^TAU
  constexpr int ROWB = D * 2;                 // bytes per K/V row
  constexpr int TILE = BN * ROWB;             // bytes per K or V tile
  constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  constexpr int DMA_PER_TILE = TILE / 1024;   // 1 KB (64 lanes x 16 B) per DMA instruction
  // Whole rows per DMA and an equal share of the K and of the V DMAs per wave
  // (D = 64, 128, 256); otherwise (D = 32, 96) the K and V DMAs of a block
  // form one list dealt round-robin over the waves, each DMA covering 64
  // consecutive 16-byte slots of its tile in row-major order.
  constexpr bool ROWWISE = (1024 % ROWB == 0) && (DMA_PER_TILE % NW == 0);
  constexpr int DPW = ROWWISE ? DMA_PER_TILE / NW : 1;  // per wave per tile (row-wise)
  constexpr int ROWS_PER_DMA = ROWWISE ? 1024 / ROWB : 1;
  constexpr int MPW = 2 * DMA_PER_TILE / NW;  // per wave per block (dealt)
  constexpr int DC = D / 16;                  // 16-wide d chunks (S contraction)
  constexpr int DT = D / 32;                  // 32-row d tiles of O^T
  constexpr int KT = BN / 32;                 // 32-key MFMA tiles per block
  constexpr int KC = BN / 16;                 // 16-key contraction chunks per block
  static_assert((2 * DMA_PER_TILE) % NW == 0, "the DMAs of a block split evenly over the waves");
  static_assert(BN == 32 || BN == 64, "block of 32 or 64 keys");

  // One LDS object per stage and operand: the compiler then knows that the
  // DMA into one stage cannot alias the reads of the other, and the block's
  // first LDS read need not wait for the next block's DMA (with one array per
  // operand it waits for every outstanding DMA, serialising the prefetch).
  __shared__ __attribute__((aligned(1024))) char kbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TILE];
  __shared__ int s_arrival;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
  const int n = lane & 31;  // query of this lane within the wave / row within an MFMA tile
  const int h = lane >> 5;  // lane half

  // ---- work item ----
  const int N = p.N;
  const int ntiles = (N + BM - 1) / BM;
  const int BH = p.B * p.H;
  // Workgroups are dispatched in id order, round-robin over the 8 XCDs
  // (id % 8), each with its own L2.
  int bh, tile0, ntile = 1, part = 0, nparts = 1, slot_base = 0;
  if constexpr (PAIRED) {
    // Paired causal tiles: item r is tile ntiles-1-r (keys ascending) then,
    // if different, tile r (keys descending). Every item streams about
    // ntiles+1 tiles' worth of blocks, and the workgroups of one head read
    // only two key positions at any time: all heavy tiles are at block t,
    // all light tiles at the block t mirrors. When B*H is a multiple of 8,
    // XCD x takes the heads x, x+8, x+16, ... (the same heads as in the
    // item-major order, so per-batch key lengths load every XCD alike) and
    // runs their items head by head, keeping few heads' K and V in its L2.
    const int npairs = (ntiles + 1) / 2;
    int r;
    if ((BH & 7) == 0) {
      const int k = blockIdx.x >> 3;
      bh = (blockIdx.x & 7) + 8 * (k / npairs);
      r = k % npairs;
    } else {
      bh = blockIdx.x % BH;
      r = blockIdx.x / BH;
    }
    tile0 = ntiles - 1 - r;
    if (tile0 != r) ntile = 2;
  } else {
    // Item-major order: workgroup id w takes item w / (B*H) of head
    // w % (B*H), so every XCD sees the heaviest items first and, when B*H
    // is a multiple of 8, the items of a fixed set of heads, whose K and V
    // then share its L2.
    bh = blockIdx.x % BH;
    int rank = blockIdx.x / BH;
    if (p.seq && plan.nitems == 0 && (BH & 7) == 0) {
      // Head-sequential: XCD x takes the same heads (x, x+8, ...) but runs
      // them one after another, heaviest tile first within a head.
      bh = (blockIdx.x & 7) + 8 * ((blockIdx.x >> 3) / ntiles);
      rank = (blockIdx.x >> 3) % ntiles;
    }
    if (plan.nitems > 0) {
      const unsigned it = plan.item[rank];
      tile0 = (int)(it & 0x1ffu);
      part = (int)((it >> 9) & 63u);
      nparts = (int)((it >> 15) & 63u) + 1;
      slot_base = (int)(it >> 21);
    } else {
      tile0 = CAUSAL ? ntiles - 1 - rank : rank;  // causal: the latest rows see the most keys
    }
  }
  const int b = bh / p.H;
  const int Nk = p.Nk;
  // Causal: key visible iff key <= query + shift (queries are the last N of
  // the Nk positions; the strict mask also hides the query's own position).
  const int shift = CAUSAL ? Nk - N - p.diag : 0;
  int kvlen = Nk;
  if (p.kv_lens) kvlen = min(max(p.kv_lens[b], 0), Nk);

  const size_t head = (size_t)bh * N * D;  // Q, O rows of this head
  const size_t kvhead = ((size_t)b * p.Hkv + (bh % p.H) / (p.H / p.Hkv)) * Nk * D;
  const T* __restrict__ Q = (const T*)p.q + head;
  const T* __restrict__ K = (const T*)p.k + kvhead;
  const T* __restrict__ V = (const T*)p.v + kvhead;

  // Per-tile state, set at the start of each tile of the item.
  int tile, q0;        // query tile and its first row
  int jbeg, jend;      // this item's key blocks of the tile: [jbeg, jend)
  int qa, qrow;        // first query of this wave; query of this lane
  bool started;        // the wave has processed a block of this tile

  // ---- K/V block stream, HBM -> LDS ----
  // Per-lane source offsets inside a block (bytes), fixed for the kernel: a
  // block's DMA then needs only a scalar base. A block that runs past row
  // N-1 (the ragged end) takes the clamped path.
  int gk[DPW], gv[DPW];
  if constexpr (ROWWISE) {
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int row = (wave * DPW + i) * ROWS_PER_DMA + lane / CPR;
      const int pch = lane % CPR;
      gk[i] = row * ROWB + kchunk<D>(row, pch) * 16;
      gv[i] = row * ROWB + vchunk<D>(row, pch) * 16;
    }
  }
  // Dealt DMAs: the m-th of this wave is entry wave + NW*m of the block's list
  // (K tile DMAs first, then V); lane l covers slot 64*blk + l of its tile.
  int grow[MPW], gch[MPW], goff[MPW];
  if constexpr (!ROWWISE) {
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      const int e = wave + NW * m;
      const bool isv = e >= DMA_PER_TILE;
      const int g = 64 * (isv ? e - DMA_PER_TILE : e) + lane;
      grow[m] = g / CPR;
      gch[m] = isv ? vchunk<D>(grow[m], g % CPR) : kchunk<D>(grow[m], g % CPR);
      goff[m] = grow[m] * ROWB + gch[m] * 16;
    }
  }
  // DMAs are buffer loads with the LDS flag: a per-block buffer resource
  // (scalar base at the block's first row) and a 32-bit per-lane offset,
  // so a block costs no vector address arithmetic. Unlike the global form,
  // these count only in vmcnt for the compiler, which then waits for the
  // operand reads of the LDS by count while a DMA is in flight.
  auto issue_block = [&](int j, auto stage) {
    constexpr int SD = decltype(stage)::value;
    if ((PAIRED && j < jbeg) || j >= jend) return;  // only a descending stream runs below jbeg
    const int key0 = j * BN;
    char* ks = SD == 0 ? kbuf0 : kbuf1;
    char* vs = SD == 0 ? vbuf0 : vbuf1;
    const buffer_rsrc kr = make_rsrc(K + (size_t)key0 * D);
    const buffer_rsrc vr = make_rsrc(V + (size_t)key0 * D);
    const bool full = key0 + BN <= Nk;
    if constexpr (!ROWWISE) {
#pragma unroll
      for (int m = 0; m < MPW; ++m) {
        const int e = wave + NW * m;  // wave-uniform
        const bool isv = e >= DMA_PER_TILE;
        char* dst = (isv ? vs : ks) + (isv ? e - DMA_PER_TILE : e) * 1024;
        // a ragged last block re-reads row Nk - 1 for the rows past it
        const int off = full ? goff[m] : (min(grow[m], Nk - 1 - key0) * ROWB + gch[m] * 16);
        dma16_buf(isv ? vr : kr, off, dst);
      }
      return;
    }
    // One uniform branch per block: a full block issues its DMAs with the
    // precomputed offsets, straight through.
    if (full) {
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int blk = wave * DPW + i;
        dma16_buf(kr, gk[i], ks + blk * 1024);
        dma16_buf(vr, gv[i], vs + blk * 1024);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int blk = wave * DPW + i;
      const int row = blk * ROWS_PER_DMA + lane / CPR;
      const int pch = lane % CPR;
      const int r = min(row, Nk - 1 - key0);
      dma16_buf(kr, r * ROWB + kchunk<D>(row, pch) * 16, ks + blk * 1024);
      dma16_buf(vr, r * ROWB + vchunk<D>(row, pch) * 16, vs + blk * 1024);
    }
  };

  // Per-lane LDS offsets of the operand reads (the block-independent parts).
  int koff[DC];  // K row n (+32 per key tile), logical chunk 2c + h
#pragma unroll
  for (int c = 0; c < DC; ++c) koff[c] = n * ROWB + kslot<D>(n, 2 * c + h) * 16;
  // V^T transpose reads: row 16*kc + 8r + 4h + (lane%16)/4, column
  // dt*32 + 16*((lane/16)%2) + 4*(lane%4) (four elements = 8 bytes). The slot
  // permutation depends only on row % 8, which 16*kc + 8r leaves unchanged.
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int vrow = 4 * h + ((lane & 15) >> 2);
  int voff[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int col = dt * 32 + vcol;
    voff[dt] = vrow * ROWB + vslot<D>(vrow, col >> 3) * 16 + (col & 7) * 2;
  }

  x8 qf[DC];              // Q^T fragments: lane (n, h) holds query qrow, dims 16c + 8h .. +8
  f32x16 acc[DT];         // O^T, unnormalised
  float m_run;            // reference max (scaled log2 units)
  float l_run;            // this lane's share of sum p (fp32)
  float l_bf;             // the same over the rounded (16-bit) p used by P V
  const float scl = p.scale_log2;

  // One key block: the stage (LDS buffer) is a compile-time constant, so
  // every LDS operand offset is an immediate. The c-th block of a tile's
  // stream uses stage c % 2; block jnext, the one after it, goes to the
  // other stage.
  auto step = [&](int j, int jnext, auto stage) {
    constexpr int ST = decltype(stage)::value;
    // Block j has landed once this wave's DMAs are done (its only
    // outstanding vector-memory operations) and every wave has passed the
    // barrier, which also frees the other stage, read in the previous block.
    wait_vmem();
    __syncthreads();
    const int key0 = j * BN;
    // Blocks wholly in this wave's future (all its rows would be masked), and
    // every block of a wave whose rows all lie past the last query (decode,
    // a ragged last tile), are skipped; the wave still issues its share of
    // the next block's DMA.
    const bool skip = (CAUSAL && key0 > qa + 31 + shift) || qa >= N;
    const char* ks = ST == 0 ? kbuf0 : kbuf1;
    const char* vs = ST == 0 ? vbuf0 : vbuf1;

    // ---- S^T = K Q^T for BN keys x 32 queries ----
    // Waves in a matrix phase get issue priority over waves in their softmax,
    // so whichever wave has MFMAs ready keeps the matrix pipe fed while the
    // others' VALU work fills the gaps.
    f32x16 s[KT];
    if (!skip) {
      __builtin_amdgcn_s_setprio(FA_PRIO_MFMA);
#pragma unroll
      for (int t = 0; t < KT; ++t) zero(s[t]);
#pragma unroll
      for (int c = 0; c < DC; ++c)
#pragma unroll
        for (int t = 0; t < KT; ++t)
          s[t] = E::mfma(*(const x8*)(ks + t * 32 * ROWB + koff[c]), qf[c], s[t]);
      if constexpr (D == 128 && BN == 64) {
        // Rolling read-ahead: the K reads of chunk c+1 go out before the
        // MFMAs of chunk c, so each wait leaves two reads in flight.
        __builtin_amdgcn_sched_group_barrier(0x100, KT, 0);  // DS reads
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          if (c + 1 < DC) __builtin_amdgcn_sched_group_barrier(0x100, KT, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, KT, 0);  // MFMA
        }
      }
    }
    // The next block's DMA goes out after the S products are issued: its
    // issue overlaps their drain instead of delaying the first K read, and
    // with no LDS DMA in flight during the K reads the compiler waits for
    // each read by count (lgkmcnt(n)) rather than for all of them.
    issue_block(jnext, std::integral_constant<int, 1 - ST>());
    if (skip) return;
    __builtin_amdgcn_s_setprio(0);
    // ---- mask (only blocks that straddle the diagonal or kv_len) ----
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

    // ---- online softmax ----
    // Probabilities against the current reference max m_run. While the
    // block's row max stays within TAU of it every p is at most 2^TAU, so a
    // lane sum above 2^TAU (or not a number: a row whose keys were all
    // hidden so far) is the only case that needs the block max: then the
    // reference moves to the row's block max if that lies more than TAU above
    // it (rescaling the accumulators once), and the block's p are recomputed.
    x8 pf[KC];
    // rs: this block's fp32 sum (from -0, so the first addition is exact and
    // needs no instruction); lbf_new: l_bf with this block's rounded p added.
    float rs, lbf_new;
    auto probabilities = [&](float m_use) {
      rs = -0.f;
      lbf_new = l_bf;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * (kc & 1) + 2 * e;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kc >> 1][r], scl, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kc >> 1][r + 1], scl, -m_use));
          w[e] = E::pack(p0, p1);
          rs += p0 + p1;
          lbf_new = E::add_pair(w[e], lbf_new);
        }
        pf[kc] = __builtin_bit_cast(x8, w);
      }
    };
    // A descending stream's first blocks straddle the diagonal, so a wave may
    // skip some before its first; an ascending one starts at jbeg.
    if (PAIRED ? !started : j == jbeg) {
      // First block of the tile this wave processes: there is nothing to
      // rescale yet, so the reference max is simply the block's row max
      // (-inf for a row with no visible key, whose p are then 0) and the lag
      // check below passes.
      started = true;
      float mx = NEG_INF;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
      m_run = pair_max(mx) * scl;
      probabilities((m_run == NEG_INF) ? 0.f : m_run);
    } else {
      probabilities(m_run);
    }
    if (__any(!(rs <= P_BOUND))) {
      float mx = NEG_INF;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
      const float mt = pair_max(mx) * scl;  // block max, scaled (-inf if all hidden)
      const bool up = mt > m_run + TAU;
      // A sum above the bound with every block max still within TAU of its
      // reference (many weights near 2^TAU) moves no reference: the p just
      // computed stand. Only a moved reference, or a row with nothing
      // visible so far (its p are not numbers), needs the rescale and the
      // recompute.
      if (__any(up || m_run == NEG_INF)) {
        const float m_new = up ? mt : m_run;
        const float corr = up ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 if m_run = -inf
        l_run *= corr;
        l_bf *= corr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] *= corr;
        m_run = m_new;
        probabilities((m_run == NEG_INF) ? 0.f : m_run);  // nothing visible yet: p = 0
      }
    }
    l_run += rs;
    l_bf = lbf_new;

    __builtin_amdgcn_s_setprio(FA_PRIO_MFMA);
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const i16x4 lo = lds_read_tr16(vs + kc * 16 * ROWB + voff[dt]);
        const i16x4 hi = lds_read_tr16(vs + (kc * 16 + 8) * ROWB + voff[dt]);
        const x8 a = __builtin_bit_cast(x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = E::mfma(a, pf[kc], acc[dt]);
      }
    {
      // Rolling read-ahead: the four transpose reads of the next pair of
      // contraction chunks go out before the two MFMAs of the current pair,
      // so each pair's LDS latency overlaps the previous pair's matrix work.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads
#pragma unroll
      for (int g = 0; g < DT * KC / 2; ++g) {
        if (g + 1 < DT * KC / 2) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      }
    }
  };

  for (int it = 0; it < ntile; ++it) {
    tile = it ? ntiles - 1 - tile0 : tile0;
    q0 = tile * BM;
    int kend = kvlen;
    if (CAUSAL) kend = max(min(kend, q0 + BM + shift), 0);
    const int nblk = (kend + BN - 1) / BN;  // visible blocks
    // This item's block range: its share of the tile's nominal (unpadded)
    // blocks, clipped to the visible ones.
    const int nbn = (max(CAUSAL ? min(Nk, q0 + BM + Nk - N) : Nk, 0) + BN - 1) / BN;
    jbeg = part * nbn / nparts;
    jend = min((part + 1) * nbn / nparts, nblk);
    qa = q0 + wave * 32;
    qrow = qa + n;
    {
      const int qrow_c = min(qrow, N - 1);
#pragma unroll
      for (int c = 0; c < DC; ++c)
        qf[c] = *(const x8*)(Q + (size_t)qrow_c * D + 16 * c + 8 * h);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) zero(acc[dt]);
    m_run = NEG_INF;
    l_run = 0.f;
    l_bf = 0.f;
    started = false;
    // A second tile: every wave has finished reading both stages of the
    // first before stage 0 is refilled.
    if (it) __syncthreads();
    // The first tile streams its blocks in ascending order, the second in
    // descending order.
    const int dir = it ? -1 : 1;
    const int jfirst = it ? jend - 1 : jbeg;
    const int nb = jend - jbeg;
    issue_block(jfirst, std::integral_constant<int, 0>());
    __builtin_amdgcn_sched_barrier(0);
    for (int c = 0; c < nb; c += 2) {
      const int j = jfirst + c * dir;
      step(j, j + dir, std::integral_constant<int, 0>());
      if (c + 1 < nb) step(j + dir, j + 2 * dir, std::integral_constant<int, 1>());
    }
    __builtin_amdgcn_s_setprio(0);
    wait_vmem();  // no DMA may still target this workgroup's LDS at exit

    // ---- split item: publish the partial state; the last arrival merges ----
    if (nparts > 1) {
      // Slot layout (fp32): accumulators as [wave][dt][r/4][lane][r%4] (every
      // 16-byte access of a wave covers 1 KB contiguously), then per lane
      // {m, l, l_bf, 0}. Written and read with device-coherent 16-byte buffer
      // accesses (they bypass the per-XCD L2 caches), so no cache-wide
      // write-back or invalidation is needed; completing this wave's stores
      // before the barrier orders them before the arrival count.
      constexpr int SLOT_O = BM * D * 4;              // bytes of accumulators per slot
      constexpr int SLOT_ML = FWD_ML_FLOATS * 4;      // bytes of row statistics per slot
      const size_t slot0 = (size_t)bh * p.nslots + slot_base;
      const buffer_rsrc ro = make_rsrc(p.part_o + slot0 * (BM * D));
      const buffer_rsrc rm = make_rsrc(p.part_ml + slot0 * FWD_ML_FLOATS);
      const int vo = (wave * DT * 4 * 64 + lane) * 16;  // + ((dt * 4 + g) * 64) * 16
      const int vm = (wave * 64 + lane) * 16;
      // A wave whose rows all lie past the last query (a packed decode tile, a
      // ragged last tile) writes no output: it neither publishes nor merges.
      const bool live = qa < N;
      if (live) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v = {acc[dt][4 * g], acc[dt][4 * g + 1], acc[dt][4 * g + 2], acc[dt][4 * g + 3]};
            store_coherent16(v, ro, part * SLOT_O + vo + (dt * 4 + g) * 64 * 16);
          }
        const f32x4 st = {m_run, l_run, l_bf, 0.f};
        store_coherent16(st, rm, part * SLOT_ML + vm);
      }
      wait_vmem();
      __syncthreads();
      int* ctr = p.counters + (size_t)bh * ntiles + tile;
      if (tid == 0) s_arrival = atomicAdd(ctr, 1);
      __syncthreads();
      if (s_arrival != nparts - 1) return;  // another part will merge
      if (tid == 0) atomicExch(ctr, 0);     // ready for the next call
      if (N - q0 <= 32) {
        // Only wave 0 holds rows (a packed decode tile, a short last tile):
        // every wave merges a share of its d tiles (dt = wave, wave + NW,
        // ...), reading wave 0's slots, and writes those columns of its
        // rows. The part loops are unrolled so that the loads of several
        // parts are in flight at once (each costs a memory latency).
        // No barrier follows.
        constexpr int DTW = (DT + NW - 1) / NW;  // d tiles per wave
        if (wave >= DT) return;
        const int vm0 = lane * 16;
        float m_all = NEG_INF;
#pragma unroll 8
        for (int q = 0; q < nparts; ++q) m_all = fmaxf(m_all, load_coherent16(rm, q * SLOT_ML + vm0)[0]);
        float l_sum = 0.f, lbf_sum = 0.f;
        f32x16 mo[DTW];
#pragma unroll
        for (int i = 0; i < DTW; ++i) zero(mo[i]);
#pragma unroll 4
        for (int q = 0; q < nparts; ++q) {
          const f32x4 stat = load_coherent16(rm, q * SLOT_ML + vm0);
          const float c = (stat[0] == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(stat[0] - m_all);
          l_sum = fmaf(c, stat[1], l_sum);
          lbf_sum = fmaf(c, stat[2], lbf_sum);
#pragma unroll
          for (int i = 0; i < DTW; ++i) {
            const int dt = wave + NW * i;
            if (dt < DT) {
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const f32x4 v = load_coherent16(ro, q * SLOT_O + (lane + (dt * 4 + g) * 64) * 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) mo[i][4 * g + e] = fmaf(c, v[e], mo[i][4 * g + e]);
              }
            }
          }
        }
        const float l_tot = pair_sum(l_sum);
        const float l_o = pair_sum(lbf_sum);
        const bool empty = (l_tot == 0.f);
        const float inv = empty ? 0.f : 1.f / l_o;
        const int orow = q0 + n;  // wave 0's row in this lane
        if (orow < N) {
          T* O = (T*)p.o + head + (size_t)orow * D;
#pragma unroll
          for (int i = 0; i < DTW; ++i) {
            const int dt = wave + NW * i;
            if (dt < DT) {
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = E::pack(mo[i][4 * g] * inv, mo[i][4 * g + 1] * inv);
                w[1] = E::pack(mo[i][4 * g + 2] * inv, mo[i][4 * g + 3] * inv);
                *(u32x2*)(O + dt * 32 + 8 * g + 4 * h) = w;
              }
            }
          }
          if (wave == 0 && h == 0 && p.lse)
            p.lse[(size_t)bh * N + orow] = empty ? NEG_INF : (m_all + log2f(l_tot)) * LN2;
        }
        return;
      }
      if (!live) return;                    // no barrier follows

      // Every part, this one included, is read back and combined in part
      // order: the result does not depend on which part arrived last.
      // The row statistics are read twice (max first, then the sums), so any
      // number of parts merges in the same registers.
      float m_all = NEG_INF;
#pragma unroll 8
      for (int q = 0; q < nparts; ++q) m_all = fmaxf(m_all, load_coherent16(rm, q * SLOT_ML + vm)[0]);
      float l_sum = 0.f, lbf_sum = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) zero(acc[dt]);
      for (int q = 0; q < nparts; ++q) {
        const f32x4 stat = load_coherent16(rm, q * SLOT_ML + vm);
        const float m_q = stat[0];
        const float c = (m_q == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(m_q - m_all);
        l_sum = fmaf(c, stat[1], l_sum);
        lbf_sum = fmaf(c, stat[2], lbf_sum);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v = load_coherent16(ro, q * SLOT_O + vo + (dt * 4 + g) * 64 * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[dt][4 * g + e] = fmaf(c, v[e], acc[dt][4 * g + e]);
          }
      }
      m_run = m_all;
      l_run = l_sum;
      l_bf = lbf_sum;
    }

    // ---- finalize ----
    const float l_tot = pair_sum(l_run);
    const float l_o = pair_sum(l_bf);
    const bool empty = (l_tot == 0.f);
    const float inv = empty ? 0.f : 1.f / l_o;
    if (qrow < N) {
      T* O = (T*)p.o + head + (size_t)qrow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = E::pack(acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv);
          w[1] = E::pack(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv);
          *(u32x2*)(O + dt * 32 + 8 * g + 4 * h) = w;
        }
      if (h == 0 && p.lse) {
        p.lse[(size_t)bh * N + qrow] = empty ? NEG_INF : (m_run + log2f(l_tot)) * LN2;
      }
    }
  }  // tiles of the item
}

template <typename T, int D, int BN>
hipError_t launch_d(const FwdParams& p, const FwdPlan& plan, hipStream_t stream) {
  const long long ntiles = (p.N + BM - 1) / BM;
  const bool paired = p.causal && p.pair && plan.nitems == 0;
  const long long items = plan.nitems > 0 ? plan.nitems : (paired ? (ntiles + 1) / 2 : ntiles);
  const long long grid = (long long)p.B * p.H * items;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), blk(NW * 64);
  if (paired)
    hipLaunchKernelGGL((fwd_kernel<T, D, BN, true, true>), g, blk, 0, stream, p, plan);
  else if (p.causal)
    hipLaunchKernelGGL((fwd_kernel<T, D, BN, true, false>), g, blk, 0, stream, p, plan);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, BN, false, false>), g, blk, 0, stream, p, plan);
  return hipGetLastError();
}

template <typename T, int D, int BN, bool CAUSAL>
int occupancy() {
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per, reinterpret_cast<const void*>(&fwd_kernel<T, D, BN, CAUSAL, false>), NW * 64,
          0) != hipSuccess)
    return 0;
  return per;
}

// Calls f(std::integral_constant<int, BN>) for the block size instantiated
// (64 keys at every head dimension); returns `fallback` for any other bn.
template <int D, typename F, typename R>
R with_block_keys(int bn, F&& f, R fallback) {
  if (bn == 64) return f(std::integral_constant<int, 64>());
  return fallback;
}

template <typename T, int D>
int occupancy_of(int bn, bool causal) {
  return with_block_keys<D>(bn, [&](auto b) {
    constexpr int BN = decltype(b)::value;
    return causal ? occupancy<T, D, BN, true>() : occupancy<T, D, BN, false>();
  }, 0);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, const FwdPlan& plan, hipStream_t stream) {
#define FA_LAUNCH(DD)                                                                    \
  if (p.d == DD) {                                                                       \
    return with_block_keys<DD>(p.bn, [&](auto b) {                                       \
      constexpr int BN = decltype(b)::value;                                             \
      if (p.dtype == DTYPE_BF16) return launch_d<__bf16, DD, BN>(p, plan, stream);       \
      if (p.dtype == DTYPE_F16) return launch_d<_Float16, DD, BN>(p, plan, stream);      \
      return hipErrorInvalidValue;                                                       \
    }, hipErrorInvalidValue);                                                            \
  }
  FA_FOR_EACH_D(FA_LAUNCH)
#undef FA_LAUNCH
  return hipErrorInvalidValue;
}

int fwd_device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it == cache.end()) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 0)
      cus = 0;
    it = cache.emplace(dev, cus).first;
  }
  return it->second;
}

int fwd_occupancy(int d, int bn, bool causal, int dtype) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, bool, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(dev, d, bn, causal, dtype);
  auto it = cache.find(key);
  if (it == cache.end()) {
    int per = 0;
#define FA_OCC(DD)                                                      \
  if (d == DD) {                                                        \
    if (dtype == DTYPE_BF16) per = occupancy_of<__bf16, DD>(bn, causal);   \
    if (dtype == DTYPE_F16) per = occupancy_of<_Float16, DD>(bn, causal);  \
  }
    FA_FOR_EACH_D(FA_OCC)
#undef FA_OCC
    it = cache.emplace(key, per > 0 ? per : 0).first;
  }
  return it->second;
}

}  // namespace fa
