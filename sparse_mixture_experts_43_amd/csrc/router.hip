// Router: logits, softmax statistics, top-k, renormalised gates and the fp64
// capacity-rank key, fused in one kernel per block of RT tokens.
//
// Page "Mixture-of-Experts" (beta.fermi.ai wiki), step-by-step mechanism,
// steps 1-3: logits x W_g, softmax over the N experts, top-k by score,
// renormalise the k scores to sum to one. Softmax is strictly increasing, so
// the top-k set is taken on the fp32 logits (equal logits: lower expert id).
// Page "Mixture of Experts: How Sparse Routing Scales Transformers", "Inside
// the Router": router numbers are kept at higher precision, here fp32 logits
// and fp64 normalisation.
//
// Phase 1 (bf16): each wave owns 16 tokens x (a range of <= 256 experts) and
// accumulates with v_mfma_f32_16x16x32_bf16; W_g [d, N] is N-contiguous, so
// each K-chunk of it is transposed into LDS as [n][k] (one k per lane, so the
// 2-byte LDS stores of a wave are contiguous) and shared by the 4 waves.
// Phase 1 (fp32): plain FMA over LDS tiles (small workloads only).
// Phase 2: the block's logits sit in LDS (reusing the W_g staging space); one
// wave per token row does k rounds of (value desc, index asc) argmax with
// cross-lane butterflies, then the fp64 log-sum-exp and the gates.
#include "moe_common.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- phase 2
// Row r of the block's logits tile (LDS, row stride ls_stride floats).
__device__ void topk_row(const float* __restrict__ Lrow, int N, int k, int t, float* __restrict__ logits,
                         int32_t* __restrict__ idx, float* __restrict__ w, double* __restrict__ key) {
  const int l = lane_id();
  float v[kMaxN / kWave];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxN / kWave; ++i) {
    const int n = l + kWave * i;
    v[i] = (n < N) ? Lrow[n] : -INFINITY;
    if (n < N) {
      m = fmaxf(m, v[i]);
      logits[(size_t)t * N + n] = v[i];
    }
  }
  m = wave_max_f32(m);

  // fp64 softmax denominator over all N experts.
  double s = 0.0;
  const double md = (double)m;
#pragma unroll
  for (int i = 0; i < kMaxN / kWave; ++i) {
    const int n = l + kWave * i;
    if (n < N) s += exp((double)v[i] - md);
  }
  s = wave_sum_f64(s);
  const double lse = md + log(s);

  // k rounds of argmax: larger value wins, equal values -> lower index.
  unsigned taken = 0u;
  float sel_v[kMaxK];
  int sel_n[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      float bv = -INFINITY;
      int bn = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kMaxN / kWave; ++i) {
        const int n = l + kWave * i;
        if (n < N && !((taken >> i) & 1u) && (v[i] > bv || bn == 0x7fffffff)) {
          bv = v[i];
          bn = n;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = wave_shfl_xor(bv, o);
        const int on = wave_shfl_xor(bn, o);
        if (ov > bv || (ov == bv && on < bn)) {
          bv = ov;
          bn = on;
        }
      }
      if ((bn & (kWave - 1)) == l) taken |= 1u << (bn / kWave);
      sel_v[j] = bv;
      sel_n[j] = bn;
    }
  }
  double psum = 0.0;
  double p[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      p[j] = exp((double)sel_v[j] - md);
      psum += p[j];
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k && l == j) {
      idx[(size_t)t * k + j] = sel_n[j];
      w[(size_t)t * k + j] = (float)(p[j] / psum);
      key[(size_t)t * k + j] = (double)sel_v[j] - lse;
    }
  }
}

// ---------------------------------------------------------------- bf16
// RT tokens per block; KC = K-chunk staged per barrier (64 or 32).
template <int RT, int KC>
__global__ __launch_bounds__(kThreads) void router_bf16_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ Wg, const float* __restrict__ bias, int T,
    int d, int N, int k, float* __restrict__ logits, int32_t* __restrict__ idx,
    float* __restrict__ w, double* __restrict__ key) {
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* Wt = (bf16*)smem;  // [NP][KC + 8]
  float* Ls = (float*)smem;  // [RT][NP + 4] after phase 1

  constexpr int TG = RT / 16;  // token groups of 16
  constexpr int CG = 4 / TG;   // column groups
  constexpr int WROW = KC + 8;
  const int NP = cdiv(N, 16) * 16;
  const int NT = NP / 16;
  const int ntpg = cdiv(NT, CG);
  const int wv = threadIdx.x / kWave;
  const int l = lane_id();
  const int tg = wv % TG, cg = wv / TG;
  const int j0 = cg * ntpg;
  const int nj = max(0, min(NT, j0 + ntpg) - j0);
  const int t0 = blockIdx.x * RT;
  const int row = t0 + tg * 16 + (l & 15);
  const int g = l >> 4;

  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const bool vecW = (N & 7) == 0;
  for (int kc = 0; kc < d; kc += KC) {
    __syncthreads();
    // Stage W_g[kc:kc+KC, :] transposed into Wt[n][kk].
    {
      constexpr int LPK = KC;            // lanes per n8 block
      constexpr int BPW = kWave / LPK;   // n8 blocks per wave pass
      const int kl = l % LPK;
      const int kg = kc + kl;
      for (int nb = wv * BPW + l / LPK; nb < NP / 8; nb += 4 * BPW) {
        const int n8 = nb * 8;
        bf16 vals[8];
        if (kg < d && vecW && n8 + 8 <= N) {
          bf16x8 v8 = *(const bf16x8*)(Wg + (size_t)kg * N + n8);
#pragma unroll
          for (int i = 0; i < 8; ++i) vals[i] = v8[i];
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            vals[i] = (kg < d && n8 + i < N) ? Wg[(size_t)kg * N + n8 + i] : (bf16)0.0f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) Wt[(n8 + i) * WROW + kl] = vals[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KC; kk += 32) {
      const int kx = kc + kk + 8 * g;
      bf16x8 a;
      if (row < T && kx < d) {
        a = *(const bf16x8*)(x + (size_t)row * d + kx);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = (bf16)0.0f;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j < nj) {
          const int n = (j0 + j) * 16 + (l & 15);
          const bf16x8 b = *(const bf16x8*)(Wt + n * WROW + kk + 8 * g);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();
  // D layout: lane holds column n = l%16, rows 4g + i.
  const int LS = NP + 4;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < nj) {
      const int n = (j0 + j) * 16 + (l & 15);
      const float b = (bias != nullptr && n < N) ? bias[n] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) Ls[(tg * 16 + 4 * g + i) * LS + n] = acc[j][i] + b;
    }
  }
  __syncthreads();
  for (int r = wv; r < RT; r += 4) {
    const int t = t0 + r;
    if (t < T) topk_row(Ls + r * LS, N, k, t, logits, idx, w, key);
  }
}

// ---------------------------------------------------------------- fp32
__global__ __launch_bounds__(kThreads) void router_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ Wg, const float* __restrict__ bias, int T,
    int d, int N, int k, float* __restrict__ logits, int32_t* __restrict__ idx,
    float* __restrict__ w, double* __restrict__ key) {
  constexpr int RT = 16, KC = 32, NC = 256;
  extern __shared__ __align__(16) unsigned char smem[];
  float* xs = (float*)smem;   // [RT][KC]
  float* ws = xs + RT * KC;   // [KC][NC]
  float* Ls = ws + KC * NC;   // [RT][NP + 4]
  const int NP = cdiv(N, 16) * 16;
  const int LS = NP + 4;
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * RT;
  const int rq = (tid / 64) * 4;  // rows rq..rq+3
  const int cq = tid % 64;        // columns cq + 64*q
  for (int c0 = 0; c0 < N; c0 += NC) {
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][q] = 0.f;
    for (int kc = 0; kc < d; kc += KC) {
      __syncthreads();
      for (int e = tid; e < RT * KC; e += kThreads) {
        const int r = e / KC, kk = e % KC;
        xs[e] = (t0 + r < T && kc + kk < d) ? x[(size_t)(t0 + r) * d + kc + kk] : 0.f;
      }
      for (int e = tid; e < KC * NC; e += kThreads) {
        const int kk = e / NC, n = c0 + e % NC;
        ws[e] = (kc + kk < d && n < N) ? Wg[(size_t)(kc + kk) * N + n] : 0.f;
      }
      __syncthreads();
#pragma unroll 8
      for (int kk = 0; kk < KC; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xv = xs[(rq + i) * KC + kk];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(xv, ws[kk * NC + cq + 64 * q], acc[i][q]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = c0 + cq + 64 * q;
      if (n < N) {
        const float b = bias != nullptr ? bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) Ls[(rq + i) * LS + n] = acc[i][q] + b;
      }
    }
  }
  __syncthreads();
  const int wv = tid / kWave;
  for (int r = wv; r < RT; r += 4) {
    const int t = t0 + r;
    if (t < T) topk_row(Ls + r * LS, N, k, t, logits, idx, w, key);
  }
}

template <int RT, int KC>
hipError_t launch_bf16(const void* x, const void* W_g, const float* bias, int T, int d, int N, int k,
                       float* logits, int32_t* idx, float* w, double* key, hipStream_t st) {
  const int NP = cdiv(N, 16) * 16;
  const size_t lds_w = (size_t)NP * (KC + 8) * sizeof(bf16);
  const size_t lds_l = (size_t)RT * (NP + 4) * sizeof(float);
  const size_t lds = lds_w > lds_l ? lds_w : lds_l;
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)router_bf16_kernel<RT, KC>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr = true;
  }
  hipLaunchKernelGGL((router_bf16_kernel<RT, KC>), dim3(cdiv(T, RT)), dim3(kThreads), lds, st,
                     (const bf16*)x, (const bf16*)W_g, bias, T, d, N, k, logits, idx, w, key);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const void* x, const void* W_g, const float* bias, int T, int d, int N,
                        int k, int dtype, float* logits, int32_t* idx, float* w, double* key,
                        hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (dtype == kF32) {
    const int NP = cdiv(N, 16) * 16;
    const size_t lds = (16 * 32 + 32 * 256 + 16 * (NP + 4)) * sizeof(float);
    static bool attr = false;
    if (!attr) {
      hipFuncSetAttribute((const void*)router_f32_kernel,
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      attr = true;
    }
    hipLaunchKernelGGL(router_f32_kernel, dim3(cdiv(T, 16)), dim3(kThreads), lds, st,
                       (const float*)x, (const float*)W_g, bias, T, d, N, k, logits, idx, w, key);
    return hipGetLastError();
  }
  // Token rows per block: as many as the expert count allows (each wave holds
  // at most 256 expert columns), fewer when that would leave CUs idle.
  if (N <= 256 && T >= 64 * 256) return launch_bf16<64, 64>(x, W_g, bias, T, d, N, k, logits, idx, w, key, st);
  if (N <= 512 && T >= 32 * 256) return launch_bf16<32, 64>(x, W_g, bias, T, d, N, k, logits, idx, w, key, st);
  if (N <= 512) return launch_bf16<16, 64>(x, W_g, bias, T, d, N, k, logits, idx, w, key, st);
  return launch_bf16<16, 32>(x, W_g, bias, T, d, N, k, logits, idx, w, key, st);
}

}  // namespace moe
