// Forward routing statistics: per-expert share of the top-k picks f_e, mean
// router probability P_e, the load-balancing term N * sum_e f_e P_e and the
// router z term mean_t lse_t^2.
//
// Page "Mixture-of-Experts" (wiki), step 8 and "The load-balancing auxiliary
// loss" (f_e, P_e, N * sum f_e P_e, minimum 1 at uniform routing); page
// "Mixture of Experts (MoE): Architecture, Routing, and Scaling", "Auxiliary
// Load Balancing Loss" and "Importance Loss and Z-Loss" (the z term over the
// tokens' log-sum-exp). f_e counts the T*k top-k picks before capacity, so
// sum_e f_e = 1; the coefficients of the training losses are left to the
// caller.
//
// Evaluation: fp64 from the fp32 logits, as the router's rank keys. Pass 1:
// block b owns a contiguous token range; wave v of it takes tokens v, v+4, ...
// of the range (each token's loads issued one token ahead), a lane owning
// experts l, l+64, ...; per-lane fp64 sums of the softmax probabilities and
// integer pick counts (LDS integer adds, exact in any order), then the block's
// four waves are summed in wave order into per-block partials, stored
// expert-major. Pass 2: a wave per expert sums its row of partials (lane l:
// blocks l, l+64, ... in order, then an xor butterfly), 16 experts per block;
// pass 3 adds the blocks' f P sums and the z partials. Every floating-point
// sum has a fixed order, so results are bit-reproducible; no floating-point
// atomics.
#include "moe_common.h"

#include <math.h>

namespace moe {

namespace {

constexpr int kStatsBlocks = 256;  // pass-1 blocks at most
// NS: experts per lane (ceil(N / 64) rounded up to a power of two)
template <int NS>
__global__ __launch_bounds__(256) void stats_partial_kernel(const float* __restrict__ logits,
                                                           const int32_t* __restrict__ idx,
                                                           int T, int N, int k, int per_block,
                                                           double* __restrict__ psum,
                                                           int32_t* __restrict__ pcnt,
                                                           double* __restrict__ pz) {
  __shared__ double wsum[4][kMaxN];
  __shared__ int wcnt[4][kMaxN];
  __shared__ double wz[4];
  const int l = lane_id();
  const int wv = threadIdx.x / kWave;
  const int t0 = blockIdx.x * per_block;
  const int t1 = min(T, t0 + per_block);
  for (int e = l; e < N; e += kWave) wcnt[wv][e] = 0;
  __builtin_amdgcn_wave_barrier();
  double acc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) acc[i] = 0.0;
  double z = 0.0;
  // token t's row (lanes own experts l, l+64, ...) and pick l (lanes < k),
  // loaded one token ahead of their use
  float v[NS], vn[NS];
  int pick = -1, pickn = -1;
  auto load = [&](int t, float (&r)[NS], int& p) {
    const bool ok = t < t1;
    const float* row = logits + (size_t)(ok ? t : 0) * N;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int e = l + kWave * i;
      r[i] = (ok && e < N) ? row[e] : -INFINITY;
    }
    p = (ok && l < k) ? idx[(size_t)t * k + l] : -1;
  };
  load(t0 + wv, v, pick);
  for (int t = t0 + wv; t < t1; t += 4) {
    load(t + 4, vn, pickn);
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NS; ++i) m = fmaxf(m, v[i]);
    m = wave_max_f32(m);
    const double md = (double)m;
    double ex[NS];
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      ex[i] = (l + kWave * i < N) ? exp((double)v[i] - md) : 0.0;
      s += ex[i];
    }
    s = wave_sum_f64(s);
    const double lse = md + log(s);
    z += lse * lse;  // every lane holds the same lse
    // p = exp(L - m) / sum exp(L - m), the exponentials reused
    const double rs = 1.0 / s;
#pragma unroll
    for (int i = 0; i < NS; ++i) acc[i] += ex[i] * rs;
    // integer counts: the order of the additions does not matter
    if ((unsigned)pick < (unsigned)N) atomicAdd(&wcnt[wv][pick], 1);
#pragma unroll
    for (int i = 0; i < NS; ++i) v[i] = vn[i];
    pick = pickn;
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = l + kWave * i;
    if (e < N) wsum[wv][e] = acc[i];
  }
  if (l == 0) wz[wv] = z;
  __syncthreads();
  // partials expert-major ([N][nb]) so that pass 2 reads each expert's row
  // of block partials contiguously
  const int nb = gridDim.x;
  for (int e = threadIdx.x; e < N; e += 256) {
    psum[(size_t)e * nb + blockIdx.x] = ((wsum[0][e] + wsum[1][e]) + wsum[2][e]) + wsum[3][e];
    pcnt[(size_t)e * nb + blockIdx.x] = wcnt[0][e] + wcnt[1][e] + wcnt[2][e] + wcnt[3][e];
  }
  if (threadIdx.x == 0) pz[blockIdx.x] = ((wz[0] + wz[1]) + wz[2]) + wz[3];
}

// Pass 2: one wave per expert (block b, wave v: expert 16 b + v). Lane l sums
// the partials of pass-1 blocks l, l + 64, ... in order (loads batched four
// at a time), then an xor butterfly over the lanes. Each block also writes
// the sum of f_e * P_e over its 16 experts in expert order; with a single
// block it finishes the two scalars itself.
__global__ __launch_bounds__(1024) void stats_expert_kernel(const double* __restrict__ psum,
                                                           const int32_t* __restrict__ pcnt,
                                                           const double* __restrict__ pz,
                                                           int nb, int T, int N, int k,
                                                           double* __restrict__ fpb,
                                                           float* __restrict__ stats) {
  __shared__ double fpart[16];
  const int l = lane_id();
  const int wv = threadIdx.x / kWave;
  const int e = blockIdx.x * 16 + wv;
  double fp = 0.0;
  if (e < N) {
    const double* ps = psum + (size_t)e * nb;
    const int32_t* pc = pcnt + (size_t)e * nb;
    double s = 0.0;
    int c = 0;
    for (int b0 = 0; b0 < nb; b0 += 4 * kWave) {
      double sv[4];
      int cv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = b0 + u * kWave + l;
        sv[u] = b < nb ? ps[b] : 0.0;
        cv[u] = b < nb ? pc[b] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s += sv[u];
        c += cv[u];
      }
    }
    s = wave_sum_f64(s);
    c = wave_sum_i32(c);
    const double f = (double)c / ((double)T * (double)k);
    const double P = s / (double)T;
    if (l == 0) {
      stats[e] = (float)f;
      stats[N + e] = (float)P;
    }
    fp = f * P;
  }
  if (l == 0) fpart[wv] = fp;
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0;
    for (int q = 0; q < 16; ++q) a += fpart[q];
    if (gridDim.x == 1) {
      double z = 0.0;
      for (int b = 0; b < nb; ++b) z += pz[b];
      stats[2 * N] = (float)((double)N * a);
      stats[2 * N + 1] = (float)(z / (double)T);
    } else {
      fpb[blockIdx.x] = a;
    }
  }
}

// Pass 3 (more than 16 experts): the per-block sums of f_e * P_e and the
// z partials, each in order.
__global__ __launch_bounds__(64) void stats_final_kernel(const double* __restrict__ fpb, int nfb,
                                                         const double* __restrict__ pz, int nb,
                                                         int T, int N, float* __restrict__ stats) {
  if (threadIdx.x != 0) return;
  double a = 0.0;
  for (int q = 0; q < nfb; ++q) a += fpb[q];
  double z = 0.0;
  for (int b = 0; b < nb; ++b) z += pz[b];
  stats[2 * N] = (float)((double)N * a);
  stats[2 * N + 1] = (float)(z / (double)T);
}

int stats_blocks(int T) {
  const int want = cdiv(T, 16);  // up to 4 tokens per wave before the grid is full
  return want < kStatsBlocks ? (want > 0 ? want : 1) : kStatsBlocks;
}

}  // namespace

size_t stats_scratch_bytes(int T, int N) {
  const size_t nb = (size_t)stats_blocks(T);
  return align_up(nb * N * sizeof(double), 256) + align_up(nb * N * sizeof(int32_t), 256) +
         align_up(nb * sizeof(double), 256) + align_up((size_t)cdiv(N, 16) * sizeof(double), 256);
}

hipError_t launch_routing_stats(const float* logits, const int32_t* idx, int T, int N, int k,
                                float* stats, void* scratch, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int nb = stats_blocks(T);
  const int per_block = cdiv(T, nb);
  Carver c(scratch);
  double* psum = c.take<double>((size_t)nb * N);
  int32_t* pcnt = c.take<int32_t>((size_t)nb * N);
  double* pz = c.take<double>((size_t)nb);
  const int neb = cdiv(N, 16);
  double* fpb = c.take<double>((size_t)neb);
  const int ns = cdiv(N, kWave);
  if (ns <= 1)
    hipLaunchKernelGGL(stats_partial_kernel<1>, dim3(nb), dim3(256), 0, st, logits, idx, T, N, k,
                       per_block, psum, pcnt, pz);
  else if (ns <= 2)
    hipLaunchKernelGGL(stats_partial_kernel<2>, dim3(nb), dim3(256), 0, st, logits, idx, T, N, k,
                       per_block, psum, pcnt, pz);
  else if (ns <= 4)
    hipLaunchKernelGGL(stats_partial_kernel<4>, dim3(nb), dim3(256), 0, st, logits, idx, T, N, k,
                       per_block, psum, pcnt, pz);
  else if (ns <= 8)
    hipLaunchKernelGGL(stats_partial_kernel<8>, dim3(nb), dim3(256), 0, st, logits, idx, T, N, k,
                       per_block, psum, pcnt, pz);
  else
    hipLaunchKernelGGL(stats_partial_kernel<16>, dim3(nb), dim3(256), 0, st, logits, idx, T, N,
                       k, per_block, psum, pcnt, pz);
  hipLaunchKernelGGL(stats_expert_kernel, dim3(neb), dim3(1024), 0, st, psum, pcnt, pz, nb, T, N,
                     k, fpb, stats);
  if (neb > 1)
    hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(64), 0, st, fpb, neb, pz, nb, T, N, stats);
  return hipGetLastError();
}

}  // namespace moe
