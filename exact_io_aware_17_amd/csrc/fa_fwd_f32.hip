// Exact attention forward in float32 (the reference-precision path).
//
// Same result as the bf16 path but with float32 inputs, float32 products and
// float32 exponentials, for parity checks at 1e-5. Two threads share one query
// row (each holds half of q and half of the output accumulator); a workgroup
// owns 128 query rows and streams keys in blocks of 32 through LDS. Per block
// it applies the online recurrence of the interactive explainer "The Flash
// Attention": block max m', m_new = max(m, m'), c = exp(m - m_new),
// l <- l c + sum exp(s - m_new), acc <- acc c + sum exp(s - m_new) v, with a
// single division by l at the end and the empty-row guard of "Worked
// examples", Cell D2. Throughput is not a goal here.
#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

constexpr int BQ = 128;  // query rows per workgroup
constexpr int BK = 32;   // keys per block
constexpr float NEG_INF = -__builtin_huge_valf();

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdParams p) {
  constexpr int HD = D / 2;
  __shared__ float ks[BK][D];
  __shared__ float vs[BK][D];

  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int N = p.N;
  const int ntiles = (N + BQ - 1) / BQ;
  const int bh = blockIdx.x / ntiles;
  const int tile = blockIdx.x % ntiles;
  const int b = bh / p.H;
  const int q0 = tile * BQ;
  const int qrow = q0 + (tid >> 1);
  const int qrow_c = min(qrow, N - 1);

  const int Nk = p.Nk;
  // Causal: key visible iff key <= query + shift (the queries are the last N
  // of the Nk positions; the strict mask also hides the query's own one).
  const int shift = CAUSAL ? Nk - N - p.diag : 0;

  int kvlen = Nk;
  if (p.kv_lens) kvlen = min(max(p.kv_lens[b], 0), Nk);
  int kend = kvlen;
  if (CAUSAL) kend = max(min(kend, q0 + BQ + shift), 0);
  const int nblk = (kend + BK - 1) / BK;

  const size_t head = (size_t)bh * N * D;
  const size_t kvhead = ((size_t)b * p.Hkv + (bh % p.H) / (p.H / p.Hkv)) * Nk * D;
  const float* Q = (const float*)p.q + head;
  const float* K = (const float*)p.k + kvhead;
  const float* V = (const float*)p.v + kvhead;

  float q[HD];
#pragma unroll
  for (int t = 0; t < HD; ++t) q[t] = Q[(size_t)qrow_c * D + half * HD + t];
  float acc[HD];
#pragma unroll
  for (int t = 0; t < HD; ++t) acc[t] = 0.f;
  float m = NEG_INF, l = 0.f;
  const float scale = p.scale;

  for (int j = 0; j < nblk; ++j) {
    const int key0 = j * BK;
    __syncthreads();
    for (int u = tid; u < BK * D; u += 256) {
      const int r = u / D, c = u % D;
      const int key = min(key0 + r, Nk - 1);
      ks[r][c] = K[(size_t)key * D + c];
      vs[r][c] = V[(size_t)key * D + c];
    }
    __syncthreads();

    float sc[BK];
    float bmax = NEG_INF;
#pragma unroll
    for (int jj = 0; jj < BK; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < HD; ++t) dot = fmaf(q[t], ks[jj][half * HD + t], dot);
      dot += __shfl_xor(dot, 1);
      const int key = key0 + jj;
      const bool vis = (key < kvlen) && (!CAUSAL || key <= qrow + shift);
      const float s = vis ? dot * scale : NEG_INF;
      sc[jj] = s;
      bmax = fmaxf(bmax, s);
    }
    const float m_new = fmaxf(m, bmax);
    if (m_new == NEG_INF) continue;  // nothing visible yet: the state stays empty
    const float c = (m == NEG_INF) ? 0.f : expf(m - m_new);
    l *= c;
#pragma unroll
    for (int t = 0; t < HD; ++t) acc[t] *= c;
#pragma unroll
    for (int jj = 0; jj < BK; ++jj) {
      const float pj = expf(sc[jj] - m_new);
      l += pj;
#pragma unroll
      for (int t = 0; t < HD; ++t) acc[t] = fmaf(pj, vs[jj][half * HD + t], acc[t]);
    }
    m = m_new;
  }

  if (qrow < N) {
    const bool empty = (l == 0.f);
    float* O = (float*)p.o + head + (size_t)qrow * D + half * HD;
#pragma unroll
    for (int t = 0; t < HD; ++t) O[t] = empty ? 0.f : acc[t] / l;
    if (half == 0 && p.lse) p.lse[(size_t)bh * N + qrow] = empty ? NEG_INF : m + logf(l);
  }
}

template <int D>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  const long long grid = (long long)p.B * p.H * ((p.N + BQ - 1) / BQ);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.causal)
    hipLaunchKernelGGL((fwd_f32_kernel<D, true>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, false>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
  if (p.d == 256) return launch_d<256>(p, stream);
  if (p.d == 128) return launch_d<128>(p, stream);
  if (p.d == 96) return launch_d<96>(p, stream);
  if (p.d == 64) return launch_d<64>(p, stream);
  if (p.d == 32) return launch_d<32>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
