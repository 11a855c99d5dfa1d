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
#include "gemm_ring.h"
#include "moe_common.h"
#include "topk.h"

#include <utility>

namespace moe {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- expert choice
// Every (token, expert) pair is a candidate (page "Mixture of Experts: Scaling
// Language Models with Sparse Activation", "Expert Choice Routing"): pair
// t*N + e gets expert e, weight p[t,e] (the softmax probability itself) and the
// fp64 rank key L[t,e] - lse_t, computed as in topk_row (wave max, per-lane
// sums of exp over the lane's experts, DPP wave sum). One wave per token.
template <int S>
__device__ __forceinline__ void ec_route_row(const float* __restrict__ row, int t, int N,
                                             int32_t* __restrict__ idx, float* __restrict__ w,
                                             double* __restrict__ key) {
  const int l = lane_id();
  float v[S];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int n = l + kWave * i;
    v[i] = (n < N) ? row[n] : -INFINITY;
    if (n < N) m = fmaxf(m, v[i]);
  }
  m = wave_max_dpp(m);
  const double md = (double)m;
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int n = l + kWave * i;
    if (n < N) s += exp((double)v[i] - md);
  }
  s = wave_sum_dpp(s);
  const double lse = md + log(s);
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int n = l + kWave * i;
    if (n < N) {
      const size_t p = (size_t)t * N + n;
      const double kk = (double)v[i] - lse;
      idx[p] = n;
      key[p] = kk;
      w[p] = (float)exp(kk);
    }
  }
}

__global__ __launch_bounds__(256) void ec_route_kernel(const float* __restrict__ logits, int T,
                                                       int N, int32_t* __restrict__ idx,
                                                       float* __restrict__ w,
                                                       double* __restrict__ key) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  const float* row = logits + (size_t)t * N;
  // 64-expert slots per lane: the smallest count that covers N
  if (N <= 64) ec_route_row<1>(row, t, N, idx, w, key);
  else if (N <= 128) ec_route_row<2>(row, t, N, idx, w, key);
  else if (N <= 256) ec_route_row<4>(row, t, N, idx, w, key);
  else if (N <= 512) ec_route_row<8>(row, t, N, idx, w, key);
  else ec_route_row<kMaxN / kWave>(row, t, N, idx, w, key);
}

// ---------------------------------------------------------------- W_g transpose
// W_g [d, N] (N-contiguous) -> WgT [NP, d] (K-contiguous, rows n >= N zero), the
// layout the MFMA B operand wants: 8 consecutive k of one expert per lane.
__global__ __launch_bounds__(256) void transpose_wg_kernel(const bf16* __restrict__ Wg, int d, int N,
                                                           int NP, bf16* __restrict__ WgT) {
  // 64 x 64 tile through LDS; 16-byte loads (8 experts of one k) when N % 8 ==
  // 0, 16-byte stores (8 k of one expert; d % 8 == 0)
  __shared__ bf16 tile[64][72];  // [k][n]
  const int k0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int kk = tid / 8 + 32 * q, nc = (tid % 8) * 8;
    const int kg = k0 + kk, ng = n0 + nc;
    bf16x8 v;
    if (kg < d && ng + 8 <= N && (N % 8) == 0) {
      v = *(const bf16x8*)(Wg + (size_t)kg * N + ng);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = (kg < d && ng + u < N) ? Wg[(size_t)kg * N + ng + u] : (bf16)0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) tile[kk][nc + u] = v[u];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int nn = tid / 8 + 32 * q, kc = (tid % 8) * 8;
    const int ng = n0 + nn, kg = k0 + kc;
    if (ng >= NP || kg >= d) continue;
    bf16x8 v;
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = tile[kc + u][nn];
    *(bf16x8*)(WgT + (size_t)ng * d + kg) = v;
  }
}

// ---------------------------------------------------------------- skinny router
// N <= 64 (at most 4 MFMA column tiles): one block = 16 tokens, its WAVES
// waves split K; x rows stream straight from global memory, several 32-wide K
// steps of loads in flight per wave. Partial logits are summed across waves in
// a fixed order in LDS, then each wave runs the top-k of some of the 16 rows.
// Weight fragments (8 consecutive k of one expert per lane, the layout of the
// MFMA B operand):
//   LDSW:  the block first copies W_g [d, N] into LDS transposed (row n holds
//          expert n's d weights, rows padded by 16 bytes so the fragment reads
//          of 16 rows hit distinct banks); used where N*d is small, so no
//          separate transpose launch is needed;
//   else:  from WgT [NP, d] (the transposed copy made by transpose_wg_kernel,
//          L1/L2-resident).
inline int wt_ld(int d) { return d + 8; }
inline size_t wt_lds_bytes(int d, int N) { return (size_t)N * wt_ld(d) * sizeof(bf16); }
// LDS left for the staged W_g^T next to the 16-wave kernel's static arrays
// (part[16][16][NP], Ls[16][NP+4] floats)
constexpr size_t wt_lds_budget(int NP) {
  return (size_t)160 * 1024 - (size_t)16 * 16 * NP * 4 - (size_t)16 * (NP + 4) * 4 - 1024;
}

template <int WAVES, int NT, bool LDSW>
__global__ __launch_bounds__(WAVES * 64) void router_skinny_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ Wsrc, const float* __restrict__ bias,
    int T, int d, int N, int k, float* __restrict__ logits, int32_t* __restrict__ idx,
    float* __restrict__ w, double* __restrict__ key) {
  constexpr int U = NT == 1 ? 8 : (WAVES >= 16 ? 2 : 4);  // 32-wide K steps of loads in flight
  constexpr int NP = NT * 16;
  __shared__ float part[WAVES][16][NP];
  __shared__ float Ls[16][NP + 4];
  extern __shared__ __align__(16) unsigned char wt_smem[];
  bf16* wt = (bf16*)wt_smem;  // LDSW: [N][d + 8]
  const int ldw = d + 8;
  const int l = lane_id();
  const int wv = threadIdx.x / kWave;
  const int g = l >> 4, c16 = l & 15;
  const int t0 = blockIdx.x * 16;
  const int row = t0 + c16;
  const bool rok = row < T;
  const bf16* xr = x + (size_t)(rok ? row : 0) * d;
  const int nsteps = cdiv(d, 32);
  const int spw = cdiv(nsteps, WAVES);
  const int s_begin = wv * spw, s_end = min(nsteps, s_begin + spw);
  bf16x8 z;
#pragma unroll
  for (int q = 0; q < 8; ++q) z[q] = (bf16)0.f;
  bf16x8 a[U];
  auto load_x = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = (s0 + u) * 32 + 8 * g;
      const bool ok = (s0 + u) < s_end && kk < d;
      a[u] = (ok && rok) ? *(const bf16x8*)(xr + kk) : z;
    }
  };
  load_x(s_begin);  // the first x fragments fly while W_g is staged
  if constexpr (LDSW) {
    // W_g [d, N] -> wt[n][k]: coalesced reads of the row-major matrix (16-byte
    // groups of 8 experts when N % 8 == 0), scattered 2-byte LDS writes
    if (N % 8 == 0) {
      // batches of 8 groups per thread, the batch's loads issued first
      const int groups = d * N / 8;
      for (int q0 = 0; q0 < groups; q0 += 8 * WAVES * 64) {
        bf16x8 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int q = q0 + u * WAVES * 64 + (int)threadIdx.x;
          if (q < groups) v[u] = *(const bf16x8*)(Wsrc + (size_t)q * 8);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int q = q0 + u * WAVES * 64 + (int)threadIdx.x;
          if (q < groups) {
            const int e0 = q * 8, kk = e0 / N, n0 = e0 - kk * N;
#pragma unroll
            for (int i = 0; i < 8; ++i) wt[(n0 + i) * ldw + kk] = v[u][i];
          }
        }
      }
    } else {
      for (int q = threadIdx.x; q < d * N; q += WAVES * 64) {
        const int kk = q / N, n = q - kk * N;
        wt[n * ldw + kk] = Wsrc[q];
      }
    }
    __syncthreads();
  }
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int s0 = s_begin; s0 < s_end; s0 += U) {
    if (s0 != s_begin) load_x(s0);
    bf16x8 b[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = (s0 + u) * 32 + 8 * g;
      const bool ok = (s0 + u) < s_end && kk < d;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if constexpr (LDSW) {
          // d % 8 == 0: a fragment never straddles the end of a row
          const int n = 16 * j + c16;
          b[u][j] = (ok && n < N) ? *(const bf16x8*)(wt + n * ldw + kk) : z;
        } else {
          b[u][j] = ok ? *(const bf16x8*)(Wsrc + (size_t)(16 * j + c16) * d + kk) : z;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u][j], acc[j], 0, 0, 0);
  }
  // D layout: lane holds column 16j + l%16, rows 4g + i
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wv][4 * g + i][16 * j + c16] = acc[j][i];
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * NP; i += WAVES * 64) {
    const int r = i / NP, n = i - r * NP;
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < WAVES; ++q) sum += part[q][r][n];
    Ls[r][n] = sum + ((bias != nullptr && n < N) ? bias[n] : 0.f);
  }
  __syncthreads();
  if constexpr (NT == 1) {
    // 4 rows per wave in 16-lane groups (waves 0..3)
    if (wv < 4) {
      const int r = wv * 4 + (l >> 4);
      const int t = t0 + r;
      topk_row16(&Ls[r][0], t < T, N, k, t, logits, idx, w, key);
    }
  } else {
    for (int r = wv; r < 16; r += WAVES) {
      const int t = t0 + r;
      if (t < T) topk_row(&Ls[r][0], N, k, t, logits, idx, w, key);
    }
  }
}

// ---------------------------------------------------------------- split-K router
// Few tokens (T <= 64), N <= 64, d % 128 == 0. The kernels above give each
// block 16 tokens and all of K, so a batch this small runs on one to four
// CUs, each reading all of W_g. Here K is split over S blocks per 16 tokens,
// so the reads of x and W_g spread over the chip, and a second small kernel
// adds the S partial logits in a fixed order (s = 0, 1, ...), adds the bias
// and runs the top-k.
//
// Block (s, g), 4 waves: tokens 16g..16g+15; wave v takes the 32-wide K steps
// (4s + v)*spw ... (4s + v + 1)*spw - 1, the loads of up to kSkU steps in
// flight together. The B fragment (8 consecutive k of one expert per lane) is
// gathered with 2-byte loads straight from the N-contiguous W_g; a block's K
// range of W_g is contiguous, so the gathers of a wave fall in a few cache
// lines. The 4 waves' tiles are added in LDS in wave order and written as
// part[s][16g + r][n] (fp32, n < NP). At most 8 partial tiles (spw grows with
// d) keep the single block that adds them short.
constexpr int kSkU = 4;  // K steps of loads in flight per wave
template <int NT>
__global__ __launch_bounds__(256) void router_splitk_kernel(const bf16* __restrict__ x,
                                                            const bf16* __restrict__ Wg, int T,
                                                            int d, int N, int spw,
                                                            float* __restrict__ part) {
  constexpr int NP = NT * 16;
  __shared__ float red[4][16][NP];
  const int l = lane_id();
  const int wv = threadIdx.x / kWave;
  const int g4 = l >> 4, c16 = l & 15;
  const int tg = blockIdx.y;
  const int row = tg * 16 + c16;
  const bool rok = row < T;
  const bf16* xr = x + (size_t)(rok ? row : 0) * d;
  const int nsteps = d / 32;
  const int st0 = (blockIdx.x * 4 + wv) * spw, st1 = min(nsteps, st0 + spw);
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int sb = st0; sb < st1; sb += kSkU) {
    bf16x8 a[kSkU], b[kSkU][NT];
#pragma unroll
    for (int u = 0; u < kSkU; ++u) {
      const bool ok = sb + u < st1;
      const int kk = (sb + u) * 32 + 8 * g4;
#pragma unroll
      for (int q = 0; q < 8; ++q) a[u][q] = (bf16)0.f;
      if (ok && rok) a[u] = *(const bf16x8*)(xr + kk);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int n = 16 * j + c16;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          b[u][j][q] = (ok && n < N) ? Wg[(size_t)(kk + q) * N + n] : (bf16)0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kSkU; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u][j], acc[j], 0, 0, 0);
  }
  // D layout: lane holds column 16j + l%16, rows 4g + i
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wv][4 * g4 + i][16 * j + c16] = acc[j][i];
  __syncthreads();
  const size_t Tp = (size_t)gridDim.y * 16;
  for (int i = threadIdx.x; i < 16 * NP; i += 256) {
    const int r = i / NP, n = i - r * NP;
    const float v = ((red[0][r][n] + red[1][r][n]) + red[2][r][n]) + red[3][r][n];
    part[((size_t)blockIdx.x * Tp + tg * 16 + r) * NP + n] = v;
  }
}

// Sum of the S partial tiles, bias, top-k: 16 tokens per block.
template <int NT>
__global__ __launch_bounds__(256) void router_splitk_topk_kernel(
    const float* __restrict__ part, int S, const float* __restrict__ bias, int T, int N, int k,
    float* __restrict__ logits, int32_t* __restrict__ idx, float* __restrict__ w,
    double* __restrict__ key) {
  constexpr int NP = NT * 16;
  __shared__ float Ls[16][NP + 4];
  const int t0 = blockIdx.x * 16;
  const size_t stride = (size_t)gridDim.x * 16 * NP;
  for (int i = threadIdx.x; i < 16 * NP; i += 256) {
    const int r = i / NP, n = i - r * NP;
    const float sum = splitk_logit<32>(part + (size_t)(t0 + r) * NP + n, S, stride);
    Ls[r][n] = sum + ((bias != nullptr && n < N) ? bias[n] : 0.f);
  }
  __syncthreads();
  const int wv = threadIdx.x / kWave;
  if constexpr (NT == 1) {
    const int r = wv * 4 + (lane_id() >> 4);
    const int t = t0 + r;
    topk_row16(&Ls[r][0], t < T, N, k, t, logits, idx, w, key);
  } else {
    for (int r = wv; r < 16; r += 4) {
      const int t = t0 + r;
      if (t < T) topk_row(&Ls[r][0], N, k, t, logits, idx, w, key);
    }
  }
}

// Top-k of one logits row per 16-lane group (4 rows per wave), 64 < N <= 16*SL:
// lane c of the group holds experts c, c+16, ..., the reductions are the DPP
// row all-reduces above. Picks, their order and the gates are those of
// topk_row (largest logit first, equal logits to the lower expert; gates from
// the picks' probabilities summed in pick order); only the fp64 softmax sum is
// added in another order. `active` gates loads and stores; every lane of the
// wave takes part in the reductions.
//
// The code has no data-dependent branch: every selection is a compare and a
// conditional move. A pick is struck out by setting its value to NaN, which
// no `>=` admits; slots past N are NaN for the scans too, after the softmax
// (which needs them at -inf, whose exponential is exactly 0). A real -inf
// logit is still pickable, as in topk_row.
template <int SL>
__device__ __forceinline__ void topk_row16x(const float* __restrict__ Lrow, bool active, int N,
                                            int k, int t, int32_t* __restrict__ idx,
                                            float* __restrict__ w, double* __restrict__ key) {
  const int c = lane_id() & 15;
  float v[SL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const int n = c + 16 * i;
    v[i] = (active && n < N) ? Lrow[n] : -INFINITY;
    m = fmaxf(m, v[i]);
  }
  m = fmaxf(m, dpp_f32<kDppXor1>(m));
  m = fmaxf(m, dpp_f32<kDppXor2>(m));
  m = fmaxf(m, dpp_f32<kDppHalfMirror>(m));
  m = fmaxf(m, dpp_f32<kDppMirror>(m));
  const double md = (double)m;
  // fp64 softmax denominator. (Rows past T, all -inf, get NaN; nothing of
  // theirs is stored.)
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < SL; ++i) s += exp((double)v[i] - md);
  s += dpp_f64<kDppXor1>(s);
  s += dpp_f64<kDppXor2>(s);
  s += dpp_f64<kDppHalfMirror>(s);
  s += dpp_f64<kDppMirror>(s);
  const double lse = md + log(s);
#pragma unroll
  for (int i = 0; i < SL; ++i)
    if (c + 16 * i >= N) v[i] = __builtin_nanf("");
  // Lane c of the group keeps pick c.
  float my_v = 0.f;
  int my_n = 0;
  constexpr int kNone = 1 << 24;  // slot of a lane with nothing left: expert >= 2^28
  for (int j = 0; j < k; ++j) {
    // this lane's best: scanning down with >= leaves equal values to the
    // lowest slot, i.e. the lowest expert
    float bv = -INFINITY;
    int bi = kNone;
#pragma unroll
    for (int i = SL - 1; i >= 0; --i) {
      const bool p = v[i] >= bv;
      bv = p ? v[i] : bv;
      bi = p ? i : bi;
    }
    int bn = c + 16 * bi;
    argmax_step<kDppXor1>(bv, bn);
    argmax_step<kDppXor2>(bv, bn);
    argmax_step<kDppHalfMirror>(bv, bn);
    argmax_step<kDppMirror>(bv, bn);
    // strike the pick out in its lane
    const int q = (bn & 15) == c ? (bn >> 4) : -1;
#pragma unroll
    for (int i = 0; i < SL; ++i) v[i] = q == i ? __builtin_nanf("") : v[i];
    my_v = c == j ? bv : my_v;
    my_n = c == j ? bn : my_n;
  }
  // The picks' unnormalised probabilities, then their sum in pick order: after
  // k steps of "shift right one lane, add own", lane k-1 of the group holds
  // (((p_0 + p_1) + p_2) + ...) + p_{k-1}.
  const double my_p = exp((double)my_v - md);
  double acc = 0.0;
  for (int j = 0; j < k; ++j) acc = dpp_f64<kDppRowShr1>(acc) + my_p;
  const double psum = __shfl(acc, (lane_id() & ~15) | (k - 1), kWave);
  if (active && c < k) {
    idx[(size_t)t * k + c] = my_n;
    w[(size_t)t * k + c] = (float)(my_p / psum);
    key[(size_t)t * k + c] = (double)my_v - lse;
  }
}

// ---------------------------------------------------------------- top-k over logits rows
// One wave per token; the logits are already in global memory.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int N, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ w,
                                                   double* __restrict__ key) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  topk_row(logits + (size_t)t * N, N, k, t, nullptr, idx, w, key);
}

// 64 < N <= 16*SL: a 16-lane group per row, 16 rows per block.
template <int SL>
__global__ __launch_bounds__(256) void topk16_kernel(const float* __restrict__ logits, int T, int N,
                                                     int k, int32_t* __restrict__ idx,
                                                     float* __restrict__ w, double* __restrict__ key) {
  const int t = blockIdx.x * 16 + threadIdx.x / 16;
  const bool active = t < T;
  topk_row16x<SL>(logits + (size_t)(active ? t : 0) * N, active, N, k, t, idx, w, key);
}

// ---------------------------------------------------------------- wide router (64 < N <= 256)
// Logits, softmax statistics, top-k, gates and keys of 64 tokens per block
// for up to 256 experts (NP = 128 * NB, padded), in one launch. The block's
// 8 waves share the 64 token rows, which stream through an LDS ring (64-wide K
// stages, global_load_lds, rows of 128 bytes with the 16-byte chunk c of row r
// at position c ^ ((r >> 1) & 7), so the fragment reads of 16 rows hit
// distinct banks); wave w multiplies them against its own 16 * NB experts,
// whose fragments come straight from W_g^T [NP, d] (K-contiguous,
// L2-resident) into registers. Both are requested kWrLook stages ahead: every
// block reads all of W_g^T from L2, and with only a stage or two in flight the
// loop waits out the L2 latency at every stage. v_mfma_f32_16x16x32_bf16 with
// the weight fragment as the A operand: each lane accumulates 4 consecutive
// experts of one token. The finished logits tile goes to LDS (plus the bias),
// then each 16-lane group runs topk_row16x on one token row: the same picks,
// order and gates as the other router kernels, the fp64 softmax sum in the
// 16-lane order.
// ---------------------------------------------------------------- wide router (64 < N <= 256)
// Logits, softmax statistics, top-k, gates and keys of 64 tokens per block
// for up to 256 experts (NP = 128 * NB, padded), in one launch. Wave w of the
// block's 8 owns experts 16*NB*w .. +16*NB for all 64 tokens. Everything
// streams through LDS with global_load_lds in 64-wide K stages (rows of 128
// bytes, the 16-byte chunk c of row r at position c ^ ((r >> 1) & 7), so the
// fragment reads of 16 rows hit distinct banks):
//   token rows : shared by the 8 waves (each copies 8 of the 64 rows), a
//                kWrRingA-slot ring requested kWrLookA stages ahead (they
//                come from HBM);
//   weight rows: W_g^T [NP, d] (K-contiguous, L2-resident); each wave copies
//                and reads only its own experts' rows, so these need no
//                barrier, a kWrRingB-slot ring requested kWrLookB ahead.
// v_mfma_f32_16x16x32_bf16 with the weight fragment as the A operand: each
// lane accumulates 4 consecutive experts of one token. The finished logits
// tile goes to LDS (plus the bias), then each 16-lane group runs the top-k of
// one token row (topk_row16x): the same picks, order and gates as the other
// router kernels, the fp64 softmax sum in the 16-lane order.
constexpr int kWrTok = 64;   // tokens per block
constexpr int kWrKS = 64;    // K per stage
constexpr int kWrRowB = kWrKS * 2;
constexpr int kWrLookA = 4, kWrRingA = 6;
constexpr int kWrLookB = 2, kWrRingB = 3;
template <int NB>
__host__ __device__ constexpr size_t wide_router_lds() {
  return (size_t)kWrRingA * kWrTok * kWrRowB + (size_t)kWrRingB * 128 * NB * kWrRowB;
}

template <int NB>
__global__ __launch_bounds__(512) void router_wide_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ WgT, const float* __restrict__ bias,
    int T, int d, int N, int k, float* __restrict__ logits, int32_t* __restrict__ idx,
    float* __restrict__ w, double* __restrict__ key) {
  constexpr int NP = 128 * NB;
  constexpr int LDL = NP + 4;                    // logits tile row stride (floats)
  constexpr int SLOT_A = kWrTok * kWrRowB;       // 8 KB
  constexpr int WROWS = 16 * NB;                 // weight rows of one wave
  constexpr int SLOT_B = 8 * WROWS * kWrRowB;    // all waves' rows of one stage
  static_assert(kWrRingA >= kWrLookA + 1 && kWrRingB >= kWrLookB + 1, "slot reuse");
  static_assert(kWrLookA >= kWrLookB, "token rows go out first");
  static_assert((size_t)kWrTok * LDL * sizeof(float) <= wide_router_lds<NB>(),
                "the logits tile reuses the rings");
  extern __shared__ __align__(16) unsigned char wr_smem[];
  MOE_LDS unsigned char* ldsp = (MOE_LDS unsigned char*)wr_smem;
  const int l = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t0 = blockIdx.x * kWrTok;
  const int nst = d / kWrKS;  // d % 64 == 0

  // DMA lanes: lane l lands at row 8q + l/8 (q: the instruction), position
  // l%8, which holds chunk (l%8) ^ ((row>>1)&7) of the row
  const int drow = l >> 3;
  // token rows 8*wv .. 8*wv+7
  const int arow = 8 * wv + drow;
  const unsigned char* asrc = (const unsigned char*)(x + (size_t)min(t0 + arow, T - 1) * d) +
                              16 * ((l & 7) ^ ((arow >> 1) & 7));
  // this wave's weight rows (experts e0 + r, r < WROWS), 8 per instruction;
  // the transposed weight holds N rows rounded up to 16, so columns past N
  // repeat row N-1 (their logits are never read)
  const int e0 = wv * WROWS;
  const unsigned char* bsrc[2 * NB];
#pragma unroll
  for (int q = 0; q < 2 * NB; ++q) {
    const int r = 8 * q + drow;
    const int er = e0 + r < N ? e0 + r : N - 1;
    bsrc[q] = (const unsigned char*)(WgT + (size_t)er * d) + 16 * ((l & 7) ^ ((r >> 1) & 7));
  }
  // past the last stage the copies repeat it (dead data into a free slot)
  auto issue_a = [&](int s) {
    const int sc = s < nst ? s : nst - 1;
    dma16(asrc + (size_t)sc * kWrRowB, ldsp + (s % kWrRingA) * SLOT_A + wv * 1024);
  };
  auto issue_b = [&](int s) {
    const int sc = s < nst ? s : nst - 1;
    MOE_LDS unsigned char* dst =
        ldsp + kWrRingA * SLOT_A + (s % kWrRingB) * SLOT_B + wv * (WROWS * kWrRowB);
#pragma unroll
    for (int q = 0; q < 2 * NB; ++q) dma16(bsrc[q] + (size_t)sc * kWrRowB, dst + q * 1024);
  };
  // fragment reads: row 16b + (l&15), chunk 4h + (l>>4)
  int aoff[4][2], boff[NB][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = 4 * h + (l >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * i + (l & 15);
      aoff[i][h] = r * kWrRowB + 16 * (c ^ ((r >> 1) & 7));
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int r = 16 * j + (l & 15);
      boff[j][h] = kWrRingA * SLOT_A + wv * (WROWS * kWrRowB) + r * kWrRowB +
                   16 * (c ^ ((r >> 1) & 7));
    }
  }

  f32x4 acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // Step j issues the token rows of stage j + kWrLookA, then the weight rows
  // of stage j + kWrLookB; the prologue is steps -kWrLookA .. -1 of that
  // pattern. At step s only what was issued after stage s's weight rows may
  // still fly: the token rows of stage s + kWrLookA - 1 and the weight rows of
  // stage s + 1 ... s + kWrLookB - 1, i.e. (kWrLookB - 1) steps of 1 + 2*NB
  // operations (kWrLookB = 2: 1 + 2*NB).
  for (int j = -kWrLookA; j < 0; ++j) {
    issue_a(j + kWrLookA);
    if (j + kWrLookB >= 0) issue_b(j + kWrLookB);
  }
  constexpr int kWait = (kWrLookB - 1) * (1 + 2 * NB);
  static_assert(kWait < 64, "vmcnt range");
  for (int s = 0; s < nst; ++s) {
    // this wave's copies of stage s have landed; after the barrier every
    // wave's token rows of stage s have, and every wave is done with stage
    // s-1, whose token-row slot the copies below may reuse
    vm_wait_n<kWait>();
    wg_barrier();
    issue_a(s + kWrLookA);
    issue_b(s + kWrLookB);
    const unsigned char* sa = wr_smem + (s % kWrRingA) * SLOT_A;
    const unsigned char* sb = wr_smem + (s % kWrRingB) * SLOT_B;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 af[4], bf[NB];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)(sa + aoff[i][h]);
#pragma unroll
      for (int j = 0; j < NB; ++j) bf[j] = *(const bf16x8*)(sb + boff[j][h]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
  }
  vm_wait_n<0>();  // the dead copies too
  wg_barrier();    // no wave still reads the rings, which the tile now reuses

  // logits tile (+ bias) into LDS: lane holds token 16i + (l&15), experts
  // e0 + 16j + 4(l>>4) .. +3
  float* Lt = (float*)wr_smem;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int r = 16 * i + (l & 15);
      const int c = e0 + 16 * j + 4 * (l >> 4);
      f32x4 v = acc[i][j];
      if (bias != nullptr) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += c + q < N ? bias[c + q] : 0.f;
      }
      *(f32x4*)(Lt + r * LDL + c) = v;
    }
  __syncthreads();
  // logits out: a wave per row, coalesced
  for (int r = wv; r < kWrTok && t0 + r < T; r += 8)
    for (int c = l; c < N; c += kWave) logits[(size_t)(t0 + r) * N + c] = Lt[r * LDL + c];
  // top-k: a 16-lane group per row, 32 rows per pass of the block
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int r = pass * 32 + threadIdx.x / 16;
    const int t = t0 + r;
    topk_row16x<8 * NB>(Lt + r * LDL, t < T, N, k, t, idx, w, key);
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
// 16 tokens per block; K in chunks of 32; NQ*64 expert columns per pass (NQ =
// ceil(N/64), at most 4), so few experts cost few columns. The next chunk's x
// and W_g values are loaded into registers before the current one is
// multiplied. Top-k per token: 16-lane groups (4 tokens per wave) for N <= 16,
// a wave per token else.
template <int NQ>
__global__ __launch_bounds__(kThreads) void router_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ Wg, const float* __restrict__ bias, int T,
    int d, int N, int k, float* __restrict__ logits, int32_t* __restrict__ idx,
    float* __restrict__ w, double* __restrict__ key) {
  constexpr int RT = 16, KC = 32, NC = 64 * NQ;
  constexpr int XE = RT * KC / kThreads;  // x values per thread per chunk
  constexpr int WE = KC * NC / kThreads;  // W_g values per thread per chunk
  __shared__ float xs[RT * KC];
  __shared__ float ws[KC * NC];
  extern __shared__ __align__(16) unsigned char smem[];
  float* Ls = (float*)smem;  // [RT][NP + 4]
  const int NP = cdiv(N, 16) * 16;
  const int LS = NP + 4;
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * RT;
  const int rq = (tid / 64) * 4;  // rows rq..rq+3
  const int cq = tid % 64;        // columns cq + 64*q
  for (int c0 = 0; c0 < N; c0 += NC) {
    float acc[4][NQ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < NQ; ++q) acc[i][q] = 0.f;
    float xr[XE], wr[WE];
    auto load = [&](int kc) {
#pragma unroll
      for (int q = 0; q < XE; ++q) {
        const int e = tid + q * kThreads, r = e / KC, kk = e % KC;
        xr[q] = (t0 + r < T && kc + kk < d) ? x[(size_t)(t0 + r) * d + kc + kk] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < WE; ++q) {
        const int e = tid + q * kThreads, kk = e / NC, n = c0 + e % NC;
        wr[q] = (kc + kk < d && n < N) ? Wg[(size_t)(kc + kk) * N + n] : 0.f;
      }
    };
    load(0);
    for (int kc = 0; kc < d; kc += KC) {
      __syncthreads();
#pragma unroll
      for (int q = 0; q < XE; ++q) xs[tid + q * kThreads] = xr[q];
#pragma unroll
      for (int q = 0; q < WE; ++q) ws[tid + q * kThreads] = wr[q];
      __syncthreads();
      if (kc + KC < d) load(kc + KC);
#pragma unroll 8
      for (int kk = 0; kk < KC; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xv = xs[(rq + i) * KC + kk];
#pragma unroll
          for (int q = 0; q < NQ; ++q) acc[i][q] = fmaf(xv, ws[kk * NC + cq + 64 * q], acc[i][q]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
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
  if (N <= 16) {
    const int r = wv * 4 + (lane_id() >> 4);
    const int t = t0 + r;
    topk_row16(Ls + r * LS, t < T, N, k, t, logits, idx, w, key);
  } else {
    for (int r = wv; r < RT; r += 4) {
      const int t = t0 + r;
      if (t < T) topk_row(Ls + r * LS, N, k, t, logits, idx, w, key);
    }
  }
}

template <int RT, int KC>
hipError_t launch_bf16(const void* x, const void* W_g, const float* bias, int T, int d, int N, int k,
                       float* logits, int32_t* idx, float* w, double* key, hipStream_t st) {
  const int NP = cdiv(N, 16) * 16;
  const size_t lds_w = (size_t)NP * (KC + 8) * sizeof(bf16);
  const size_t lds_l = (size_t)RT * (NP + 4) * sizeof(float);
  const size_t lds = lds_w > lds_l ? lds_w : lds_l;
  MOE_SET_LDS_ONCE((router_bf16_kernel<RT, KC>), 160 * 1024);
  hipLaunchKernelGGL((router_bf16_kernel<RT, KC>), dim3(cdiv(T, RT)), dim3(kThreads), lds, st,
                     (const bf16*)x, (const bf16*)W_g, bias, T, d, N, k, logits, idx, w, key);
  return hipGetLastError();
}

template <int NT, bool LDSW>
void launch_skinny(bool wide, const void* x, const bf16* Wsrc, const float* bias, int T, int d,
                   int N, int k, float* logits, int32_t* idx, float* w, double* key,
                   hipStream_t st) {
  const size_t lds = LDSW ? wt_lds_bytes(d, N) : 0;
  if constexpr (LDSW) {
    MOE_SET_LDS_ONCE((router_skinny_kernel<16, NT, true>), (int)wt_lds_budget(NT * 16));
  }
  if (wide || LDSW)
    hipLaunchKernelGGL((router_skinny_kernel<16, NT, LDSW>), dim3(cdiv(T, 16)), dim3(1024), lds,
                       st, (const bf16*)x, Wsrc, bias, T, d, N, k, logits, idx, w, key);
  else
    hipLaunchKernelGGL((router_skinny_kernel<4, NT, false>), dim3(cdiv(T, 16)), dim3(256), 0, st,
                       (const bf16*)x, Wsrc, bias, T, d, N, k, logits, idx, w, key);
}

bool splitk_route_ok(int T, int d, int N, int dtype) {
  return dtype == kBF16 && T >= 1 && T <= 64 && N <= 64 && d % 128 == 0;
}

// S = cdiv(d/128, spw) <= d/128 partial tiles of 16*cdiv(T,16) <= 64 rows x NP
// fp32: at most 2*d*NP bytes, the size of the router scratch.
template <int NT>
void launch_splitk_partials(const void* x, const bf16* W_g, int T, int d, int N, float* part,
                            int* S_out, hipStream_t st) {
  const int kb = d / 128;
  const int spw = cdiv(kb, 8);  // at most 8 partial tiles to add
  const int S = cdiv(kb, spw);
  hipLaunchKernelGGL(router_splitk_kernel<NT>, dim3(S, cdiv(T, 16)), dim3(256), 0, st,
                     (const bf16*)x, W_g, T, d, N, spw, part);
  *S_out = S;
}

}  // namespace

hipError_t launch_route_partials(const void* x, const void* W_g, const float* bias, int T, int d,
                                 int N, int dtype, float* logits, int32_t* idx, float* w,
                                 double* key, void* scratch, hipStream_t st, RoutePartials* rp) {
  *rp = RoutePartials{};
  if (!splitk_route_ok(T, d, N, dtype)) return hipSuccess;
  const int NP = cdiv(N, 16) * 16;
  float* part = (float*)scratch;
  int S = 0;
  switch (NP / 16) {
    case 1: launch_splitk_partials<1>(x, (const bf16*)W_g, T, d, N, part, &S, st); break;
    case 2: launch_splitk_partials<2>(x, (const bf16*)W_g, T, d, N, part, &S, st); break;
    case 3: launch_splitk_partials<3>(x, (const bf16*)W_g, T, d, N, part, &S, st); break;
    default: launch_splitk_partials<4>(x, (const bf16*)W_g, T, d, N, part, &S, st); break;
  }
  rp->part = part;
  rp->S = S;
  rp->Tp = cdiv(T, 16) * 16;
  rp->NP = NP;
  rp->bias = bias;
  rp->logits = logits;
  rp->idx = idx;
  rp->w = w;
  rp->key = key;
  return hipGetLastError();
}

size_t route_scratch_bytes(int d, int N, int dtype) {
  if (dtype != kBF16) return 0;
  const int NP = cdiv(N, 16) * 16;
  return align_up((size_t)NP * d * sizeof(bf16), 256);
}

template <int NQ>
void launch_route_f32(const void* x, const void* W_g, const float* bias, int T, int d, int N,
                      int k, size_t lds, float* logits, int32_t* idx, float* w, double* key,
                      hipStream_t st) {
  MOE_SET_LDS_ONCE(router_f32_kernel<NQ>, 160 * 1024);
  hipLaunchKernelGGL(router_f32_kernel<NQ>, dim3(cdiv(T, 16)), dim3(kThreads), lds, st,
                     (const float*)x, (const float*)W_g, bias, T, d, N, k, logits, idx, w, key);
}

hipError_t launch_route(const void* x, const void* W_g, const float* bias, int T, int d, int N,
                        int k, int dtype, float* logits, int32_t* idx, float* w, double* key,
                        void* scratch, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (dtype == kF32) {
    const int NP = cdiv(N, 16) * 16;
    const size_t lds = (size_t)16 * (NP + 4) * sizeof(float);
    const int nq = cdiv(N, 64) < 4 ? cdiv(N, 64) : 4;
    switch (nq) {
      case 1: launch_route_f32<1>(x, W_g, bias, T, d, N, k, lds, logits, idx, w, key, st); break;
      case 2: launch_route_f32<2>(x, W_g, bias, T, d, N, k, lds, logits, idx, w, key, st); break;
      case 3: launch_route_f32<3>(x, W_g, bias, T, d, N, k, lds, logits, idx, w, key, st); break;
      default: launch_route_f32<4>(x, W_g, bias, T, d, N, k, lds, logits, idx, w, key, st); break;
    }
    return hipGetLastError();
  }
  const int NP = cdiv(N, 16) * 16;
  if (splitk_route_ok(T, d, N, dtype)) {
    // few tokens: K split over many blocks (partials in the router scratch),
    // then the sum of the partials and the top-k, 16 tokens per block
    RoutePartials rp;
    const hipError_t e = launch_route_partials(x, W_g, bias, T, d, N, dtype, logits, idx, w, key,
                                               scratch, st, &rp);
    if (e != hipSuccess) return e;
    const dim3 g(cdiv(T, 16)), b(256);
    switch (NP / 16) {
      case 1: hipLaunchKernelGGL(router_splitk_topk_kernel<1>, g, b, 0, st, rp.part, rp.S, bias, T, N, k, logits, idx, w, key); break;
      case 2: hipLaunchKernelGGL(router_splitk_topk_kernel<2>, g, b, 0, st, rp.part, rp.S, bias, T, N, k, logits, idx, w, key); break;
      case 3: hipLaunchKernelGGL(router_splitk_topk_kernel<3>, g, b, 0, st, rp.part, rp.S, bias, T, N, k, logits, idx, w, key); break;
      default: hipLaunchKernelGGL(router_splitk_topk_kernel<4>, g, b, 0, st, rp.part, rp.S, bias, T, N, k, logits, idx, w, key); break;
    }
    return hipGetLastError();
  }
  if (NP <= 64 && d % 8 == 0 && wt_lds_bytes(d, N) <= wt_lds_budget(NP)) {
    // few experts, small W_g: each block stages W_g^T in LDS (no transpose launch)
    switch (NP / 16) {
      case 1: launch_skinny<1, true>(true, x, (const bf16*)W_g, bias, T, d, N, k, logits, idx, w, key, st); break;
      case 2: launch_skinny<2, true>(true, x, (const bf16*)W_g, bias, T, d, N, k, logits, idx, w, key, st); break;
      case 3: launch_skinny<3, true>(true, x, (const bf16*)W_g, bias, T, d, N, k, logits, idx, w, key, st); break;
      default: launch_skinny<4, true>(true, x, (const bf16*)W_g, bias, T, d, N, k, logits, idx, w, key, st); break;
    }
    return hipGetLastError();
  }
  bf16* WgT = (bf16*)scratch;
  hipLaunchKernelGGL(transpose_wg_kernel, dim3(cdiv(d, 64), cdiv(NP, 64)), dim3(256), 0, st,
                     (const bf16*)W_g, d, N, NP, WgT);
  if (NP <= 64 && T >= 4096 && d % kWrKS == 0) {
    // few experts and many tokens: the one-kernel wide router with its expert
    // columns padded to 128 (measured on the Switch-style layer, 64 experts,
    // 8192 tokens: 21.5 us against 26 for the transpose + skinny kernels)
    MOE_SET_LDS_ONCE(router_wide_kernel<1>, (int)wide_router_lds<1>());
    hipLaunchKernelGGL(router_wide_kernel<1>, dim3(cdiv(T, kWrTok)), dim3(512),
                       wide_router_lds<1>(), st, (const bf16*)x, WgT, bias, T, d, N, k, logits,
                       idx, w, key);
    return hipGetLastError();
  }
  if (NP <= 64) {
    // few experts: K split over the waves of a block; more waves when T is small
    const bool wide = T < 16 * 256;
    switch (NP / 16) {
      case 1: launch_skinny<1, false>(wide, x, WgT, bias, T, d, N, k, logits, idx, w, key, st); break;
      case 2: launch_skinny<2, false>(wide, x, WgT, bias, T, d, N, k, logits, idx, w, key, st); break;
      case 3: launch_skinny<3, false>(wide, x, WgT, bias, T, d, N, k, logits, idx, w, key, st); break;
      default: launch_skinny<4, false>(wide, x, WgT, bias, T, d, N, k, logits, idx, w, key, st); break;
    }
    return hipGetLastError();
  }
  if (NP <= 256 && d % kWrKS == 0) {
    // up to 256 experts: logits and top-k of 64 tokens per block in one launch
    if (NP <= 128) {
      MOE_SET_LDS_ONCE(router_wide_kernel<1>, (int)wide_router_lds<1>());
      hipLaunchKernelGGL(router_wide_kernel<1>, dim3(cdiv(T, kWrTok)), dim3(512),
                         wide_router_lds<1>(), st, (const bf16*)x, WgT, bias, T, d, N, k, logits,
                         idx, w, key);
    } else {
      MOE_SET_LDS_ONCE(router_wide_kernel<2>, (int)wide_router_lds<2>());
      hipLaunchKernelGGL(router_wide_kernel<2>, dim3(cdiv(T, kWrTok)), dim3(512),
                         wide_router_lds<2>(), st, (const bf16*)x, WgT, bias, T, d, N, k, logits,
                         idx, w, key);
    }
    return hipGetLastError();
  }
  if (d % kRK == 0) {
    // many experts: logits as a plain GEMM on the LDS-DMA ring (each step issues
    // a whole stage: one 4-wave block per CU has little else to overlap), then
    // top-k rows
    constexpr int BM = 128, BN = 128;
    const size_t lds = (size_t)kRing * (BM + BN) * kRowB;
    MOE_SET_LDS_ONCE((gemm_ring_kernel<BM, BN, 64, 64, kEpiLogit, false, kRing, true>), lds);
    const int grid = ring_grid((const void*)gemm_ring_kernel<BM, BN, 64, 64, kEpiLogit, false, kRing, true>,
                               256, lds, cdiv(T, BM) * cdiv(NP, BN));
    hipLaunchKernelGGL((gemm_ring_kernel<BM, BN, 64, 64, kEpiLogit, false, kRing, true>), dim3(grid),
                       dim3(256), lds, st, (const bf16*)x, nullptr, nullptr, 1, WgT,
                       (const void*)bias, nullptr, nullptr, nullptr, d, NP, (void*)logits, nullptr,
                       T, N, nullptr, nullptr, 0, nullptr, nullptr, 0);
    if (N <= 128)
      hipLaunchKernelGGL(topk16_kernel<8>, dim3(cdiv(T, 16)), dim3(256), 0, st, logits, T, N, k,
                         idx, w, key);
    else if (N <= 256)
      hipLaunchKernelGGL(topk16_kernel<16>, dim3(cdiv(T, 16)), dim3(256), 0, st, logits, T, N, k,
                         idx, w, key);
    else
      hipLaunchKernelGGL(topk_kernel, dim3(cdiv(T, 4)), dim3(256), 0, st, logits, T, N, k, idx, w,
                         key);
    return hipGetLastError();
  }
  // d not a multiple of 32: LDS-transposing kernel with fused top-k
  if (N <= 256 && T >= 64 * 256) return launch_bf16<64, 64>(x, W_g, bias, T, d, N, k, logits, idx, w, key, st);
  if (N <= 512 && T >= 32 * 256) return launch_bf16<32, 64>(x, W_g, bias, T, d, N, k, logits, idx, w, key, st);
  if (N <= 512) return launch_bf16<16, 64>(x, W_g, bias, T, d, N, k, logits, idx, w, key, st);
  return launch_bf16<16, 32>(x, W_g, bias, T, d, N, k, logits, idx, w, key, st);
}

hipError_t launch_route_expert_choice(const float* logits, int T, int N, int32_t* idx, float* w,
                                     double* key, hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(ec_route_kernel, dim3(cdiv(T, 4)), dim3(256), 0, st, logits, T, N, idx, w,
                     key);
  return hipGetLastError();
}

}  // namespace moe
