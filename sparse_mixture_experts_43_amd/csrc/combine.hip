// Combine: y[t] = sum over token t's kept picks of the (already gate-scaled)
// expert outputs, in fixed pick order, fp32 sums, no atomics.
//
// Page "Mixture-of-Experts" (wiki), step 7 and the combine of its pseudocode
// (Y[t] += w * o over the token's experts); a dropped pick adds nothing and a
// token with every pick dropped gets zeros (its residual path lives outside
// the layer), or its input row when the caller asks for the pseudocode's
// identity fallback (x not null). A shared expert's fp32 output, when given,
// is added to every token last (after the fallback, which replaces only the
// routed part), so y is still rounded once. The gate-scaled expert outputs
// arrive in fp32. Each thread owns 16 bytes of one output row: coalesced fp32
// loads per kept pick, one 16-byte store. When the second expert GEMM wrote
// the rows of tokens that kept a single pick straight into y (no fallback, no
// shared expert), those tokens are skipped here. With more than 8 pairs per
// token (expert choice) and a whole wave on one token row, the wave finds the
// kept pairs with one ballot per 64 and loads their rows 8 at a time.
#include "moe_common.h"

namespace moe {

namespace {

// y[t][c .. c+V) = x[t][c .. c+V) widened to fp32 (identity fallback)
template <int V, typename XT>
__device__ __forceinline__ void load_x_row(const XT* __restrict__ x, int t, int d, int c,
                                           float (&acc)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = to_f32(x[(size_t)t * d + c + i]);
}

// acc += sh[t][c .. c+V) (shared expert output, fp32)
template <int V>
__device__ __forceinline__ void add_shared(const float* __restrict__ sh, int t, int d, int c,
                                           float (&acc)[V]) {
  const f32x4* src = (const f32x4*)(sh + (size_t)t * d + c);
#pragma unroll
  for (int h = 0; h < V / 4; ++h) {
    const f32x4 v = src[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[4 * h + i] += v[i];
  }
}

template <typename T, typename XT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ slot_out,
                                                      const int32_t* __restrict__ inv, int T_,
                                                      int d, int k, const XT* __restrict__ x,
                                                      const float* __restrict__ sh,
                                                      T* __restrict__ y, int skip_single) {
  constexpr int V = 16 / sizeof(T);  // output elements per 16-byte store
  const int vpr = d / V;             // vectors per row (d % 8 == 0)
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)T_ * vpr) return;
  const int t = (int)(gid / vpr);
  const int c = (int)(gid - (long long)t * vpr) * V;
  const int32_t* it = inv + (size_t)t * k;
  // skip_single: a token with exactly one kept pick has its row written by
  // the second expert GEMM already (counted from the first group's slot
  // indices when k <= 8, else in a pass of its own)
  constexpr int G = 8;
  if (skip_single && k > G) {
    int kept = 0;
    for (int j = 0; j < k; ++j) kept += it[j] >= 0 ? 1 : 0;
    if (kept == 1) return;
  }
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  bool any = false;
  if (k > G && vpr % kWave == 0) {
    // Many picks per token (expert choice: every expert is a candidate) and a
    // whole wave on one token row: the wave reads 64 of the token's slot
    // indices at once (one per lane), a ballot marks the kept ones, and their
    // rows are loaded 8 at a time (all in flight together) and added in pick
    // order, the order of the loop below: the same sums, bit for bit.
    const int lane = threadIdx.x & (kWave - 1);
    for (int j0 = 0; j0 < k; j0 += kWave) {
      const int sv = j0 + lane < k ? it[j0 + lane] : -1;
      unsigned long long m = __ballot(sv >= 0);
      while (m != 0ull) {
        int s[G];
#pragma unroll
        for (int q = 0; q < G; ++q) {
          s[q] = -1;
          if (m != 0ull) {
            s[q] = __shfl(sv, __ffsll((long long)m) - 1, kWave);
            m &= m - 1;
          }
        }
        f32x4 v[G][V / 4];
#pragma unroll
        for (int q = 0; q < G; ++q) {
          const f32x4* src = (const f32x4*)(slot_out + (size_t)(s[q] < 0 ? 0 : s[q]) * d + c);
#pragma unroll
          for (int h = 0; h < V / 4; ++h)
            v[q][h] = s[q] >= 0 ? src[h] : (f32x4){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < G; ++q) {
          if (s[q] < 0) continue;
          any = true;
#pragma unroll
          for (int h = 0; h < V / 4; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[4 * h + i] += v[q][h][i];
        }
      }
    }
    k = 0;  // the loop below has nothing left to do
  }
  // picks in groups of 8 (all of them for k <= 8): the slot indices first,
  // then every kept pick's row load issued before the first add (one round
  // trip per group), then the sums in fixed pick order
  for (int j0 = 0; j0 < k; j0 += G) {
    int s[G];
    int kept = 0;
#pragma unroll
    for (int q = 0; q < G; ++q) {
      s[q] = j0 + q < k ? it[j0 + q] : -1;
      any |= s[q] >= 0;
      kept += s[q] >= 0 ? 1 : 0;
    }
    if (skip_single && k <= G && kept == 1) return;
    f32x4 v[G][V / 4];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const f32x4* src = (const f32x4*)(slot_out + (size_t)(s[q] < 0 ? 0 : s[q]) * d + c);
#pragma unroll
      for (int h = 0; h < V / 4; ++h) v[q][h] = s[q] >= 0 ? src[h] : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (s[q] < 0) continue;
#pragma unroll
      for (int h = 0; h < V / 4; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * h + i] += v[q][h][i];
    }
  }
  if (!any && x != nullptr) load_x_row<V>(x, t, d, c, acc);
  if (sh != nullptr) add_shared<V>(sh, t, d, c, acc);
  i32x4 outv;
  T* o = (T*)&outv;
#pragma unroll
  for (int i = 0; i < V; ++i) o[i] = from_f32<T>(acc[i]);
  *(i32x4*)(y + (size_t)t * d + c) = outv;
}

// The same combine when the second expert GEMM left K-split partials: each
// kept pick's slot value is finished here as gate * (((0 + p_0) + p_1) + ... +
// b2), the operations and order of the split-K reduction, then summed over the
// picks in fixed order, so y is bit-identical to the two-kernel path. Picks go
// in groups of 4: their slot indices first, then every partial vector and gate
// of the group (splits 2 at a time) in flight together, then the sums.
template <typename T, typename B, typename XT>
__global__ __launch_bounds__(256) void combine_splitk_kernel(
    const float* __restrict__ part, int nsplit, int S_cap, const B* __restrict__ bias,
    const float* __restrict__ gate, const int32_t* __restrict__ off, int N,
    const int32_t* __restrict__ inv, int T_, int d, int k, const XT* __restrict__ x,
    const float* __restrict__ sh, T* __restrict__ y) {
#pragma clang fp contract(off)
  constexpr int V = 16 / sizeof(T);
  constexpr int G = 4;  // picks per group
  constexpr int Q = 2;  // splits per batch of loads
  const int vpr = d / V;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)T_ * vpr) return;
  const int t = (int)(gid / vpr);
  const int c = (int)(gid - (long long)t * vpr) * V;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  bool any = false;
  for (int j0 = 0; j0 < k; j0 += G) {
    int s[G];
    float g[G];
#pragma unroll
    for (int q = 0; q < G; ++q) s[q] = j0 + q < k ? inv[(size_t)t * k + j0 + q] : -1;
#pragma unroll
    for (int q = 0; q < G; ++q) {
      any |= s[q] >= 0;
      g[q] = s[q] >= 0 ? gate[s[q]] : 0.f;
    }
    float v[G][V];
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
      for (int i = 0; i < V; ++i) v[q][i] = 0.f;
    for (int h0 = 0; h0 < nsplit; h0 += Q) {
      f32x4 pv[Q][G][V / 4];
#pragma unroll
      for (int h = 0; h < Q; ++h)
#pragma unroll
        for (int q = 0; q < G; ++q) {
          const bool ld = h0 + h < nsplit && s[q] >= 0;
          const f32x4* src =
              (const f32x4*)(part + ((size_t)(ld ? h0 + h : 0) * S_cap + (ld ? s[q] : 0)) * d + c);
#pragma unroll
          for (int u = 0; u < V / 4; ++u) pv[h][q][u] = ld ? src[u] : (f32x4){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int h = 0; h < Q; ++h)
#pragma unroll
        for (int q = 0; q < G; ++q) {
          if (h0 + h >= nsplit || s[q] < 0) continue;
#pragma unroll
          for (int u = 0; u < V / 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[q][4 * u + i] += pv[h][q][u][i];
        }
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (s[q] < 0) continue;
      int e = 0;
      if (bias != nullptr) {
        // expert of slot s: the last e with off[e] <= s
        int lo = 0, hi = N - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (off[mid] <= s[q]) lo = mid; else hi = mid - 1;
        }
        e = lo;
      }
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const float vb = v[q][i] + (bias != nullptr ? to_f32(bias[(size_t)e * d + c + i]) : 0.f);
        acc[i] += vb * g[q];  // rounded product, as the stored slot value (no fma)
      }
    }
  }
  if (!any && x != nullptr) load_x_row<V>(x, t, d, c, acc);
  if (sh != nullptr) add_shared<V>(sh, t, d, c, acc);
  i32x4 outv;
  T* o = (T*)&outv;
#pragma unroll
  for (int i = 0; i < V; ++i) o[i] = from_f32<T>(acc[i]);
  *(i32x4*)(y + (size_t)t * d + c) = outv;
}

}  // namespace

hipError_t launch_combine_splitk(const SplitK& sk, const int32_t* inv, int T, int d, int k,
                                 int y_dtype, const void* x, int x_dtype, const float* sh,
                                 void* y, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int V = y_dtype == kF32 ? 4 : 8;
  const long long n = (long long)T * (d / V);
  const int blocks = (int)((n + 255) / 256);
  if (sk.f32) {
    // fp32 layer (fp32 y, bias and x)
    hipLaunchKernelGGL((combine_splitk_kernel<float, float, float>), dim3(blocks), dim3(256), 0,
                       st, sk.part, sk.nsplit, sk.S_cap, (const float*)sk.bias, sk.gate, sk.off,
                       sk.N, inv, T, d, k, x_dtype == kF32 ? (const float*)x : nullptr, sh,
                       (float*)y);
    return hipGetLastError();
  }
  // otherwise bf16 weights and activations; y may be fp32 or bf16
  if (x_dtype != kBF16) x = nullptr;
  const bf16* b = (const bf16*)sk.bias;
  const bf16* xb = (const bf16*)x;
  if (y_dtype == kF32)
    hipLaunchKernelGGL((combine_splitk_kernel<float, bf16, bf16>), dim3(blocks), dim3(256), 0, st,
                       sk.part, sk.nsplit, sk.S_cap, b, sk.gate, sk.off, sk.N, inv, T, d, k, xb,
                       sh, (float*)y);
  else
    hipLaunchKernelGGL((combine_splitk_kernel<bf16, bf16, bf16>), dim3(blocks), dim3(256), 0, st,
                       sk.part, sk.nsplit, sk.S_cap, b, sk.gate, sk.off, sk.N, inv, T, d, k, xb,
                       sh, (bf16*)y);
  return hipGetLastError();
}

hipError_t launch_combine(const void* slot_out, const int32_t* inv, int T, int d, int k,
                          int y_dtype, const void* x, int x_dtype, const float* sh, void* y,
                          hipStream_t st, bool skip_single) {
  const int ss = skip_single ? 1 : 0;
  if (T == 0) return hipSuccess;
  const int V = y_dtype == kF32 ? 4 : 8;
  const long long n = (long long)T * (d / V);
  const int blocks = (int)((n + 255) / 256);
  const float* so = (const float*)slot_out;
  if (y_dtype == kF32) {
    if (x_dtype == kBF16)
      hipLaunchKernelGGL((combine_kernel<float, bf16>), dim3(blocks), dim3(256), 0, st, so, inv,
                         T, d, k, (const bf16*)x, sh, (float*)y, ss);
    else
      hipLaunchKernelGGL((combine_kernel<float, float>), dim3(blocks), dim3(256), 0, st, so, inv,
                         T, d, k, (const float*)x, sh, (float*)y, ss);
  } else {
    if (x_dtype == kBF16)
      hipLaunchKernelGGL((combine_kernel<bf16, bf16>), dim3(blocks), dim3(256), 0, st, so, inv,
                         T, d, k, (const bf16*)x, sh, (bf16*)y, ss);
    else
      hipLaunchKernelGGL((combine_kernel<bf16, float>), dim3(blocks), dim3(256), 0, st, so, inv,
                         T, d, k, (const float*)x, sh, (bf16*)y, ss);
  }
  return hipGetLastError();
}

}  // namespace moe
