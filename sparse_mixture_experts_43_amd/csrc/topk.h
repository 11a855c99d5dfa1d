// Per-row routing shared by the router kernels and the small-batch fused
// route + dispatch kernel: DPP reductions inside 16-lane rows and whole
// waves, and the softmax / top-k / gate / capacity-key computation of one
// logits row (one wave per row, or one 16-lane group per row for N <= 16).
//
// Page "Mixture-of-Experts" (beta.fermi.ai wiki), step-by-step mechanism,
// steps 1-3: softmax over the N experts, top-k by score, the k scores
// renormalised to sum to one. Softmax is strictly increasing, so the top-k
// set is taken on the fp32 logits (equal logits: lower expert id); the
// softmax sums are fp64.
#pragma once

#include "moe_common.h"

namespace moe {

namespace {

// ---------------------------------------------------------------- 16-lane groups, DPP
// All-reduce within each 16-lane row of a wave with DPP register moves (no
// LDS crossbar): xor 1 and xor 2 inside quads, then the half-row mirror pairs
// the two quads of each 8-lane half, the row mirror the two halves. Every
// lane of the row ends with the reduction of all 16 (any pairing pattern is
// valid for an associative, commutative combine).
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_i32<CTRL>(__builtin_bit_cast(int, v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = (unsigned)dpp_i32<CTRL>((int)(unsigned)b);
  const unsigned hi = (unsigned)dpp_i32<CTRL>((int)(unsigned)(b >> 32));
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
// Shift right by one lane within each 16-lane row; lane 0 of a row reads 0.
constexpr int kDppRowShr1 = 0x111;

template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& bn) {
  const float ov = dpp_f32<CTRL>(bv);
  const int on = dpp_i32<CTRL>(bn);
  if (ov > bv || (ov == bv && on < bn)) {
    bv = ov;
    bn = on;
  }
}

// Wave-wide versions: the row all-reduce, then the four rows' results (lanes
// 0, 16, 32, 48) read as scalars and combined in a fixed order; every lane
// gets the same value.
__device__ __forceinline__ float wave_max_dpp(float m) {
  m = fmaxf(m, dpp_f32<kDppXor1>(m));
  m = fmaxf(m, dpp_f32<kDppXor2>(m));
  m = fmaxf(m, dpp_f32<kDppHalfMirror>(m));
  m = fmaxf(m, dpp_f32<kDppMirror>(m));
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), lane);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_dpp(double s) {
  s += dpp_f64<kDppXor1>(s);
  s += dpp_f64<kDppXor2>(s);
  s += dpp_f64<kDppHalfMirror>(s);
  s += dpp_f64<kDppMirror>(s);
  return (readlane_f64(s, 0) + readlane_f64(s, 16)) + (readlane_f64(s, 32) + readlane_f64(s, 48));
}
__device__ __forceinline__ void wave_argmax_dpp(float& bv, int& bn) {
  argmax_step<kDppXor1>(bv, bn);
  argmax_step<kDppXor2>(bv, bn);
  argmax_step<kDppHalfMirror>(bv, bn);
  argmax_step<kDppMirror>(bv, bn);
  float v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 0));
  int n = __builtin_amdgcn_readlane(bn, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const float ov = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), r));
    const int on = __builtin_amdgcn_readlane(bn, r);
    if (ov > v || (ov == v && on < n)) {
      v = ov;
      n = on;
    }
  }
  bv = v;
  bn = n;
}

// ---------------------------------------------------------------- phase 2
// Row r of the block's logits tile (LDS, row stride ls_stride floats).
// `logits` may be null (the row is already in global memory). S: 64-expert
// slots per lane, S * 64 >= N (slots past N add nothing, so every S gives the
// same bits; topk_row picks the smallest).
template <int S>
__device__ __forceinline__ void topk_row_s(const float* __restrict__ Lrow, int N, int k, int t,
                                           float* __restrict__ logits, int32_t* __restrict__ idx,
                                           float* __restrict__ w, double* __restrict__ key) {
  static_assert(S >= 1 && S <= kMaxN / kWave, "slots");
  const int l = lane_id();
  float v[S];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int n = l + kWave * i;
    v[i] = (n < N) ? Lrow[n] : -INFINITY;
    if (n < N) {
      m = fmaxf(m, v[i]);
      if (logits != nullptr) logits[(size_t)t * N + n] = v[i];
    }
  }
  m = wave_max_dpp(m);

  // fp64 softmax denominator over all N experts (no branch: v = -inf past N
  // and exp(-inf) is exactly 0).
  double s = 0.0;
  const double md = (double)m;
#pragma unroll
  for (int i = 0; i < S; ++i) s += exp((double)v[i] - md);
  s = wave_sum_dpp(s);
  const double lse = md + log(s);

  // k rounds of argmax: larger value wins, equal values -> lower index. Lane j
  // keeps pick j (value, expert, unnormalised probability); no local arrays,
  // so nothing lands in scratch memory.
  unsigned taken = 0u;
  float my_v = 0.f;
  int my_n = 0;
  double my_p = 0.0, psum = 0.0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bn = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int n = l + kWave * i;
      if (n < N && !((taken >> i) & 1u) && (v[i] > bv || bn == 0x7fffffff)) {
        bv = v[i];
        bn = n;
      }
    }
    wave_argmax_dpp(bv, bn);
    if ((bn & (kWave - 1)) == l) taken |= 1u << (bn / kWave);
    const double pj = exp((double)bv - md);
    psum += pj;
    if (l == j) {
      my_v = bv;
      my_n = bn;
      my_p = pj;
    }
  }
  if (l < k) {
    idx[(size_t)t * k + l] = my_n;
    w[(size_t)t * k + l] = (float)(my_p / psum);
    key[(size_t)t * k + l] = (double)my_v - lse;
  }
}

__device__ __forceinline__ void topk_row(const float* __restrict__ Lrow, int N, int k, int t,
                                         float* __restrict__ logits, int32_t* __restrict__ idx,
                                         float* __restrict__ w, double* __restrict__ key) {
  if (N <= 64) topk_row_s<1>(Lrow, N, k, t, logits, idx, w, key);
  else if (N <= 128) topk_row_s<2>(Lrow, N, k, t, logits, idx, w, key);
  else if (N <= 256) topk_row_s<4>(Lrow, N, k, t, logits, idx, w, key);
  else if (N <= 512) topk_row_s<8>(Lrow, N, k, t, logits, idx, w, key);
  else topk_row_s<kMaxN / kWave>(Lrow, N, k, t, logits, idx, w, key);
}

// N <= 16: topk_row with one 16-lane group per token row (lane c of the group
// holds expert c), so a wave serves 4 rows; the reductions are the DPP row
// all-reduces above. Same picks and gates as topk_row; the fp64 softmax sum
// is added in another order. Every lane of the wave takes part in the
// reductions; `active` only gates the stores.
__device__ __forceinline__ void topk_row16(const float* __restrict__ Lrow, bool active, int N,
                                           int k, int t, float* __restrict__ logits,
                                           int32_t* __restrict__ idx, float* __restrict__ w,
                                           double* __restrict__ key) {
  const int c = lane_id() & 15;
  const bool has = c < N;
  const float v = has ? Lrow[c] : -INFINITY;
  if (active && has && logits != nullptr) logits[(size_t)t * N + c] = v;
  float m = v;
  m = fmaxf(m, dpp_f32<kDppXor1>(m));
  m = fmaxf(m, dpp_f32<kDppXor2>(m));
  m = fmaxf(m, dpp_f32<kDppHalfMirror>(m));
  m = fmaxf(m, dpp_f32<kDppMirror>(m));
  const double md = (double)m;
  double s = has ? exp((double)v - md) : 0.0;
  s += dpp_f64<kDppXor1>(s);
  s += dpp_f64<kDppXor2>(s);
  s += dpp_f64<kDppHalfMirror>(s);
  s += dpp_f64<kDppMirror>(s);
  const double lse = md + log(s);
  bool taken = false;
  float my_v = 0.f;
  int my_n = 0;
  double my_p = 0.0, psum = 0.0;
  for (int j = 0; j < k; ++j) {
    const bool cand = has && !taken;
    float bv = cand ? v : -INFINITY;
    int bn = cand ? c : 0x7fffffff;
    argmax_step<kDppXor1>(bv, bn);
    argmax_step<kDppXor2>(bv, bn);
    argmax_step<kDppHalfMirror>(bv, bn);
    argmax_step<kDppMirror>(bv, bn);
    if (bn == c) taken = true;
    const double pj = exp((double)bv - md);
    psum += pj;
    if (c == j) {
      my_v = bv;
      my_n = bn;
      my_p = pj;
    }
  }
  if (active && c < k) {
    idx[(size_t)t * k + c] = my_n;
    w[(size_t)t * k + c] = (float)(my_p / psum);
    key[(size_t)t * k + c] = (double)my_v - lse;
  }
}

// Split-K logits (few tokens): the S partial values of one (token, expert)
// entry, part[s * stride], added in the order s = 0, 1, ..., S - 1, with B
// loads in flight per thread (B = 32: one round trip for S <= 32; B only sets
// how the loads are batched, never the order of the adds). Every kernel that
// consumes split-K partials sums them with this function, so all of them see
// the same logits bits.
template <int B>
__device__ __forceinline__ float splitk_logit(const float* __restrict__ p, int S, size_t stride) {
  float sum = 0.f;
  for (int s0 = 0; s0 < S; s0 += B) {
    float v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) v[u] = s0 + u < S ? p[(size_t)(s0 + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (s0 + u < S) sum += v[u];
  }
  return sum;
}

}  // namespace

}  // namespace moe
