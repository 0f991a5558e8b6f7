// Exact attention forward for gfx950: bf16 matrix cores, fp32 online softmax.
//
// One workgroup owns BM = 32 * NW query rows of one (batch, head) and streams
// the visible keys in blocks of BN = 64 through LDS, carrying per query row the
// running max m, the running normaliser l and the unnormalised output (the
// online recurrence of the interactive explainer "The Flash Attention";
// "Exercises", the block merges). The score block and its probabilities live
// only in registers.
//
// Layout choices (each wave owns 32 queries, one per lane pair):
//  * Scores are produced transposed, S^T = K Q^T, with the 32x32x16 bf16 MFMA:
//    A = a 32-key x 16-dim slice of K (read from LDS), B = the wave's Q^T
//    slice (held in registers for the whole kernel). In the 32x32 accumulator
//    lane l holds query (l % 32) and 16 keys, so the row max and row sum are
//    in-lane reductions plus one exchange between the two lane halves.
//  * The output is accumulated transposed too, O^T += V^T P^T: B = P^T comes
//    straight from the score registers (after bf16 rounding), A = V^T is read
//    from a transposed copy of the V block in LDS whose key order is permuted
//    (bits 2 and 3 of the key index swapped) so that it matches the order in
//    which the accumulator registers hold the keys. The contraction index is
//    free to permute, so no data moves between lanes.
//  * The per-row rescale factor exp(m_old - m_new) is then a per-lane scalar.
//  * Exponentials are base 2 with scale*log2(e) folded into one FMA.
//  * K rows in LDS have their 16-byte chunks XOR-swizzled by row and the V^T
//    rows by d, so the MFMA operand reads of 32 consecutive rows spread over
//    all banks.
//  * Causal: key blocks wholly in a wave's future are skipped ("Question
//    bank": blocks entirely in the future are skipped); only blocks that
//    straddle the diagonal or the padding length apply a mask.
//  * A row with no visible key keeps l = 0 and is written as O = 0 and
//    lse = -inf ("Worked examples", Cell D2).
#include "fa_internal.h"
#include "fa_device.h"

#include <math.h>

namespace fa {
namespace {

using namespace dev;

constexpr int BN = 64;  // keys per streamed block

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(FwdParams p) {
  constexpr int BM = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int KT_BYTES = BN * D * 2;   // K tile
  constexpr int VT_BYTES = D * BN * 2;   // V^T tile
  constexpr int STAGE = KT_BYTES + VT_BYTES;
  constexpr int KCH = D / 8;             // 16-byte chunks per K row
  constexpr int K_PER_T = BN * KCH / NT; // K chunks staged per thread
  constexpr int V_PER_T = (BN / 2) * KCH / NT;  // (key pair, d chunk) units per thread
  static_assert(K_PER_T >= 1 && V_PER_T >= 1, "tile too small for the workgroup");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;   // query within the wave / row within an MFMA tile
  const int h = lane >> 5;   // lane half

  // ---- work assignment (a0: the tile schedule) ----
  const int N = p.N;
  const int ntiles = (N + BM - 1) / BM;
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of work ids so the tiles of one head share an L2.
  const int lid = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int bh = lid / ntiles;
  int tile = lid % ntiles;
  if (CAUSAL) tile = ntiles - 1 - tile;  // longest rows of a head first
  const int b = bh / p.H;
  const int q0 = tile * BM;

  int kvlen = N;
  if (p.kv_lens) kvlen = min(max(p.kv_lens[b], 0), N);
  int kend = kvlen;
  if (CAUSAL) kend = min(kend, q0 + BM);
  const int nblk = (kend + BN - 1) / BN;

  const size_t head = (size_t)bh * N * D;
  const __bf16* __restrict__ Q = (const __bf16*)p.q + head;
  const __bf16* __restrict__ K = (const __bf16*)p.k + head;
  const __bf16* __restrict__ V = (const __bf16*)p.v + head;

  // ---- Q^T fragments: lane (n, h) holds query qrow, dims 16c + 8h .. +8 ----
  const int qa = q0 + wave * 32;  // first query of this wave
  const int qrow = qa + n;
  const int qrow_c = min(qrow, N - 1);
  bf16x8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qf[c] = *(const bf16x8*)(Q + (size_t)qrow_c * D + 16 * c + 8 * h);

  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float m_run = NEG_INF;  // running max, in units of scale*log2(e)*score
  float l_run = 0.f;      // this lane's share of the running normaliser
  const float scl = p.scale_log2;

  // ---- staging registers for the next K/V block ----
  u32x4 kreg[K_PER_T];
  u32x4 vreg[V_PER_T][2];

  auto load_block = [&](int j) {
    const int key0 = j * BN;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int u = tid + NT * i;
      const int row = u / KCH, c = u % KCH;
      const int key = min(key0 + row, N - 1);
      kreg[i] = *(const u32x4*)(K + (size_t)key * D + c * 8);
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + NT * i;
      const int dc = u % KCH, kp = u / KCH;
      const int k0 = min(key0 + 2 * kp, N - 1);
      const int k1 = min(key0 + 2 * kp + 1, N - 1);
      vreg[i][0] = *(const u32x4*)(V + (size_t)k0 * D + dc * 8);
      vreg[i][1] = *(const u32x4*)(V + (size_t)k1 * D + dc * 8);
    }
  };
  auto store_block = [&](int buf) {
    char* ks = smem + buf * STAGE;
    char* vs = ks + KT_BYTES;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int u = tid + NT * i;
      const int row = u / KCH, c = u % KCH;
      *(u32x4*)(ks + row * (D * 2) + row_slot<D>(row, c) * 16) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + NT * i;
      const int dc = u % KCH, kp = u / KCH;
      const int pos = swap23(2 * kp);  // even; the odd key of the pair sits at pos + 1
      const unsigned* w0 = (const unsigned*)&vreg[i][0];
      const unsigned* w1 = (const unsigned*)&vreg[i][1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = dc * 8 + e;
        const unsigned lo = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xffffu);
        const unsigned hi = (e & 1) ? (w1[e >> 1] >> 16) : (w1[e >> 1] & 0xffffu);
        *(unsigned*)(vs + d * (BN * 2) + t64_slot(d, pos >> 3) * 16 + (pos & 7) * 2) =
            lo | (hi << 16);
      }
    }
  };

  if (nblk > 0) {
    load_block(0);
    store_block(0);
  }
  __syncthreads();

  for (int j = 0; j < nblk; ++j) {
    const int buf = j & 1;
    if (j + 1 < nblk) load_block(j + 1);

    const int key0 = j * BN;
    // Skip blocks wholly in this wave's future (all its rows would be masked).
    const bool wave_skip = CAUSAL && (key0 > qa + 31);
    if (!wave_skip) {
      const char* ks = smem + buf * STAGE;
      const char* vs = ks + KT_BYTES;

      // ---- a2: S^T = K Q^T for 64 keys x 32 queries ----
      f32x16 s[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int row = t * 32 + n;
          const bf16x8 a = *(const bf16x8*)(ks + row * (D * 2) + row_slot<D>(row, 2 * c + h) * 16);
          s[t] = mfma32(a, qf[c], s[t]);
        }
      }

      // ---- a3: mask (only on blocks that straddle the diagonal or kv_len) ----
      const bool need_mask = (key0 + BN > kvlen) || (CAUSAL && key0 + BN - 1 > qa);
      if (need_mask) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + t * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool hide = (key >= kvlen) || (CAUSAL && key > qrow);
            if (hide) s[t][r] = NEG_INF;
          }
      }

      // ---- a4: online softmax ----
      float mx = NEG_INF;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx * scl);
      const float m_use = (m_new == NEG_INF) ? 0.f : m_new;  // all hidden so far: keep p = 0
      const float corr = exp2f(m_run - m_use);               // 0 when m_run = -inf
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = exp2f(fmaf(s[t][r], scl, -m_use));
          s[t][r] = pv;
          rs += pv;
        }
      l_run = l_run * corr + rs;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= corr;

      // ---- P^T fragments (bf16): chunk kc = registers 8*(kc%2).. of tile kc/2 ----
      bf16x8 pf[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = pack_bf16x2(s[kc >> 1][8 * (kc & 1) + 2 * e], s[kc >> 1][8 * (kc & 1) + 2 * e + 1]);
        pf[kc] = __builtin_bit_cast(bf16x8, w);
      }

      // ---- a5: O^T += V^T P^T ----
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        const int drow = t * 32 + n;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const bf16x8 a = *(const bf16x8*)(vs + drow * (BN * 2) + t64_slot(drow, 2 * kc + h) * 16);
          acc[t] = mfma32(a, pf[kc], acc[t]);
        }
      }
    }

    if (j + 1 < nblk) store_block(buf ^ 1);
    __syncthreads();
  }

  // ---- a6: finalize ----
  const float l_tot = pair_sum(l_run);
  const bool empty = (l_tot == 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  if (qrow < N) {
    __bf16* O = (__bf16*)p.o + head + (size_t)qrow * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv);
        w[1] = pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv);
        *(u32x2*)(O + t * 32 + 8 * g + 4 * h) = w;
      }
    if (h == 0 && p.lse) {
      p.lse[(size_t)bh * N + qrow] =
          empty ? NEG_INF : (m_run + log2f(l_tot)) * LN2;
    }
  }
}

template <int D, int NW>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  constexpr int BM = 32 * NW;
  const long long ntiles = (p.N + BM - 1) / BM;
  const long long grid = (long long)p.B * p.H * ntiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.causal)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, true>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, false>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  if (p.d == 128) return launch_d<128, 4>(p, stream);
  if (p.d == 64) return launch_d<64, 4>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
