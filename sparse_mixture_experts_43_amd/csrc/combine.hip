// Combine: y[t] = sum over token t's kept picks of the (already gate-scaled)
// expert outputs, in fixed pick order, fp32 sums, no atomics.
//
// Page "Mixture-of-Experts" (wiki), step 7 and the combine of its pseudocode
// (Y[t] += w * o over the token's experts); a dropped pick adds nothing and a
// token with every pick dropped gets zeros (its residual path lives outside
// the layer). The gate-scaled expert outputs arrive in fp32. Each thread owns
// 16 bytes of one output row: coalesced fp32 loads per kept pick, one 16-byte
// store.
#include "moe_common.h"

namespace moe {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ slot_out,
                                                      const int32_t* __restrict__ inv, int T_,
                                                      int d, int k, T* __restrict__ y) {
  constexpr int V = 16 / sizeof(T);  // output elements per 16-byte store
  const int vpr = d / V;             // vectors per row (d % 8 == 0)
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)T_ * vpr) return;
  const int t = (int)(gid / vpr);
  const int c = (int)(gid - (long long)t * vpr) * V;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int s = inv[(size_t)t * k + j];
    if (s < 0) continue;
    const f32x4* src = (const f32x4*)(slot_out + (size_t)s * d + c);
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      const f32x4 v = src[q];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[4 * q + i] += v[i];
    }
  }
  i32x4 outv;
  T* o = (T*)&outv;
#pragma unroll
  for (int i = 0; i < V; ++i) o[i] = from_f32<T>(acc[i]);
  *(i32x4*)(y + (size_t)t * d + c) = outv;
}

}  // namespace

hipError_t launch_combine(const void* slot_out, const int32_t* inv, int T, int d, int k,
                          int dtype, void* y, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int V = dtype == kF32 ? 4 : 8;
  const long long n = (long long)T * (d / V);
  const int blocks = (int)((n + 255) / 256);
  if (dtype == kF32)
    hipLaunchKernelGGL(combine_kernel<float>, dim3(blocks), dim3(256), 0, st,
                       (const float*)slot_out, inv, T, d, k, (float*)y);
  else
    hipLaunchKernelGGL(combine_kernel<bf16>, dim3(blocks), dim3(256), 0, st,
                       (const float*)slot_out, inv, T, d, k, (bf16*)y);
  return hipGetLastError();
}

}  // namespace moe
