// Expert FFN over dispatched slots: grouped GEMM1 + GELU, grouped GEMM2 +
// gate scale.
//
// Page "Mixture of Experts (MoE): Architecture, Routing, and Scaling", "Core
// Architecture": each expert is FFN(x) = W2 GELU(W1 x + b1) + b2 with
// nn.Linear weights stored [out, in] (the SparseMoE snippet's
// Linear-GELU-Linear). Page "Mixture-of-Experts" (wiki), steps 5-7: every
// expert runs on the batch of tokens gathered for it, and its output is scaled
// by the combine weight. "Expert-aware batching" on the "Scaling Language
// Models with Sparse Activation" page is what grouping slots by expert buys:
// one dense GEMM per expert instead of per-token work.
//
// Code paths, chosen on the host from sizes only (no device sync, make_plan):
//   tiled bf16  : the grouped GEMM of gemm_ring.h (K % 32 == 0):
//                 v_mfma_f32_16x16x32_bf16 on an LDS ring filled by
//                 global_load_lds, persistent workgroups walking an XCD-aware
//                 tile list written by schedule_kernel (static shares with a
//                 split K tail, or per-XCD work queues), token gather fused
//                 into the copies of the first GEMM, GELU fused into its
//                 epilogue, bias and gate into the second's (fp32 output);
//                 256x256 tiles (eight waves of 128x64) for large experts
//                 without capacity limit, 128x128 (four waves of 64x64)
//                 otherwise. gemm_bf16_kernel below (32x32x16, register-staged
//                 tiles) serves K % 32 != 0.
//   decode bf16 : when an expert can hold at most 64 slots, weights are
//                 streamed once by decode_dma_kernel (gemm_decode.h: weight
//                 rows as the 16-row operand, slots as the 16-column operand,
//                 LDS-DMA ring, split K with a fixed-order reduction), or by
//                 decode_bf16_kernel below when K % 128 != 0.
//   fp32        : FMA tiles (64 x 64), same schedule mechanism; a second GEMM
//                 with few tiles splits its K over up to 8 blocks per tile,
//                 the fp32 partials summed in split order by the combine
//                 (moe_forward) or reduce_f32_kernel (moe_expert_ffn).
// Direct rows (tiled bf16, when the caller passes y): the schedule kernel
// marks each slot whose token kept no other pick, and GEMM2's epilogue writes
// that row straight into y (0 + gate * (acc + b2), as the combine would),
// leaving the combine only the tokens with zero or several kept picks.
// With the hidden-split flag, GEMM1 also stores the bf16 residual h - bf16(h)
// of each hidden activation and GEMM2 runs a second MFMA on it, so GEMM2 sees
// the hidden layer to about 16 significant bits instead of 8 (twice GEMM2's
// MFMA work; used where the weight stream, not MFMA, bounds the time).
#include "gemm_decode.h"
#include "gemm_ring.h"
#include "moe_common.h"

namespace moe {

namespace {

// ---------------------------------------------------------------- schedule
// Tile entry: {expert, first slot of the m-tile, rows in the m-tile, n-tile}.
// The grouped GEMMs hand XCD x the x-th contiguous eighth of the list, so the
// list is written band-residue-major: group r (r = 0..7) holds the weight
// bands (expert e, n-tile nt) with nt % 8 == r, expert by expert, each band
// with all its m-tiles (so one XCD's L2 serves the band's weight rows). With
// NT % 8 == 0 every group holds exactly the same m-tiles, so every XCD sees the
// same mix of full and partly filled tiles, instead of contiguous runs whose
// cost depends on where the experts' ragged last m-tiles fall. Group r has
// c_r = #{nt < NT : nt % 8 == r} bands per expert, i.e. total_mt * c_r tiles,
// so entry p decodes in closed form.
// expert_major (bit 0: first GEMM, bit 1: second): the list is instead expert
// by expert, each expert's m-tiles in order with all their n-tiles, so an XCD's
// eighth holds whole experts and the token rows of an m-tile are fetched into
// one L2 for all its n-tiles. Used for the 128x128 tiles of capacity-limited
// layers: the first GEMM when experts span several m-tiles, the second when
// each expert fits one m-tile (measured; with skewed routing and several
// m-tiles per expert, contiguous experts load the second GEMM's XCDs unevenly).
// expert_band (bit 2: first GEMM, bit 3: second): expert by expert as well,
// but each expert's bands in order with all their m-tiles, so an XCD's eighth
// holds about N/8 whole experts and its co-scheduled tiles share both the
// expert's token rows and each band's weight rows.
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* __restrict__ off, int N,
                                                        int S_max, int Ccap, int BM, int NT1,
                                                        int NT2, int max1, int max2,
                                                        int expert_major,
                                                        int4* __restrict__ tiles1,
                                                        int4* __restrict__ tiles2,
                                                        int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ inv, int T,
                                                        int kp, int32_t* __restrict__ dmap) {
  // counts[4 .. 19]: the two GEMMs' per-XCD work-queue counters, zeroed here
  if (blockIdx.x == 0 && threadIdx.x < 16) counts[4 + threadIdx.x] = 0;
  __shared__ int mtoff[kMaxN + 1];
  __shared__ int rbeg[kMaxN], rcnt[kMaxN];  // each expert's rows, clamped to the plan
  __shared__ int tmp[17];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  const int l = lane_id(), wv = threadIdx.x / kWave;
  for (int e0 = 0; e0 < N; e0 += 1024) {
    const int e = e0 + threadIdx.x;
    int mt = 0;
    if (e < N) {
      int m0, mc;
      expert_rows(off, e, S_max, Ccap, m0, mc);
      rbeg[e] = m0;
      rcnt[e] = mc;
      mt = cdiv(mc, BM);
    }
    // block exclusive scan
    int x = mt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(x, o, kWave);
      if (l >= o) x += y;
    }
    __syncthreads();
    if (l == kWave - 1) tmp[wv] = x;
    __syncthreads();
    if (wv == 0) {
      int s = (l < 16) ? tmp[l] : 0;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const int y = __shfl_up(s, o, kWave);
        if (l >= o) s += y;
      }
      if (l < 16) tmp[l] = s;
    }
    __syncthreads();
    const int excl = (wv > 0 ? tmp[wv - 1] : 0) + x - mt;
    if (e < N) mtoff[e] = carry + excl;
    __syncthreads();
    if (threadIdx.x == 0) carry += tmp[15];
    __syncthreads();
  }
  if (threadIdx.x == 0) mtoff[N] = carry;
  __syncthreads();
  const int total_mt = mtoff[N];
  for (int pass = 0; pass < 2; ++pass) {
    const int NTn = pass == 0 ? NT1 : NT2;
    const int mx = pass == 0 ? max1 : max2;
    int4* tl = pass == 0 ? tiles1 : tiles2;
    const int total = min(total_mt * NTn, mx);
    for (int p = blockIdx.x * 1024 + threadIdx.x; p < total; p += gridDim.x * 1024) {
      if ((expert_major >> pass) & 5) {
        int lo = 0, hi = N - 1;  // expert: largest e with mtoff[e] * NTn <= p
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (mtoff[mid] * NTn <= p) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int local = p - mtoff[e] * NTn;
        int mt, nt;
        if ((expert_major >> pass) & 4) {
          const int me = mtoff[e + 1] - mtoff[e];  // > 0 where p lands
          nt = local / me;
          mt = local - nt * me;
        } else {
          mt = local / NTn;
          nt = local - mt * NTn;
        }
        tl[p] = make_int4(e, rbeg[e] + mt * BM, min(BM, rcnt[e] - mt * BM), nt);
        continue;
      }
      // residue group r of entry p (groups are never empty where p lands)
      int r = 0, base = 0, c = 0;
      for (; r < 8; ++r) {
        c = NTn / 8 + (r < NTn % 8 ? 1 : 0);
        if (p < base + total_mt * c) break;
        base += total_mt * c;
      }
      const int q = p - base;
      int lo = 0, hi = N - 1;  // expert: largest e with mtoff[e] * c <= q
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mtoff[mid] * c <= q) lo = mid; else hi = mid - 1;
      }
      const int e = lo;
      const int me = mtoff[e + 1] - mtoff[e];
      const int local = q - mtoff[e] * c;
      const int band = local / me;  // the expert's band-th n-tile of residue r
      const int mt = local - band * me;
      const int nt = band * 8 + r;
      tl[p] = make_int4(e, rbeg[e] + mt * BM, min(BM, rcnt[e] - mt * BM), nt);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) counts[pass] = total;
  }
  // direct-row map (dmap not null), one thread per token: each kept slot of
  // token t gets t when it is the token's only kept pick, else -1
  if (dmap != nullptr) {
    for (int t = blockIdx.x * 1024 + threadIdx.x; t < T; t += gridDim.x * 1024) {
      const int32_t* it = inv + (size_t)t * kp;
      if (kp <= 16) {
        // all of the token's slot indices requested at once
        int sl[16];
        int kept = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          sl[j] = j < kp ? it[j] : -1;
          kept += sl[j] >= 0 ? 1 : 0;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (sl[j] >= 0 && sl[j] < S_max) dmap[sl[j]] = kept == 1 ? t : -1;
      } else {
        int kept = 0;
        for (int j = 0; j < kp; ++j) kept += it[j] >= 0 ? 1 : 0;
        for (int j = 0; j < kp; ++j) {
          const int sl = it[j];
          if (sl >= 0 && sl < S_max) dmap[sl] = kept == 1 ? t : -1;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- tiled bf16
constexpr int kBK = 64;
constexpr int kLdsRow = kBK + 8;  // bf16 elements per LDS row (144 B, conflict-free b128 reads)

// G1: A = x gathered through perm, epilogue GELU(acc + b1) -> hidden (bf16,
//     plus the bf16 residual h - bf16(h) into out_lo when SPLIT).
// G2: A = hidden (+ A_lo residual when SPLIT, a second MFMA per step),
//     epilogue gate * (acc + b2) -> fp32 slot output.
template <int BM, int BN, int WM, int WN, bool G1, bool SPLIT>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * kWave) void gemm_bf16_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ A_lo, const int32_t* __restrict__ perm,
    int kpairs, const bf16* __restrict__ W, const bf16* __restrict__ bias,
    const float* __restrict__ gate, const int4* __restrict__ tiles,
    const int32_t* __restrict__ ntiles_p, int K, int Nout, void* __restrict__ out,
    bf16* __restrict__ out_lo) {
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int NTH = NW * kWave;
  constexpr int ACH = BM * (kBK / 8) / NTH;  // 16-byte A chunks per thread per stage
  constexpr int BCH = BN * (kBK / 8) / NTH;
  constexpr int MT = WM / 32, NTW = WN / 32;
  constexpr bool ALO = SPLIT && !G1;  // second A operand (hidden residual)
  static_assert(ACH >= 1 && BCH >= 1, "tile too small for the thread count");

  extern __shared__ __align__(16) unsigned char smem[];
  bf16* As = (bf16*)smem;                    // [2][BM][kLdsRow]
  bf16* Bs = As + 2 * BM * kLdsRow;          // [2][BN][kLdsRow]
  bf16* Al = Bs + 2 * BN * kLdsRow;          // [2][BM][kLdsRow] when ALO

  const int ntiles = *ntiles_p;
  const int b = blockIdx.x;
  const int chunk = (ntiles + 7) >> 3;
  const int jx = b >> 3;
  const int tile = (b & 7) * chunk + jx;
  if (jx >= chunk || tile >= ntiles) return;
  const int4 te = tiles[tile];
  const int e = te.x, m0 = te.y, mcount = te.z, n0 = te.w * BN;

  const int tid = threadIdx.x;
  const int l = lane_id();
  const int wv = tid / kWave;
  const int wm0 = (wv / (BN / WN)) * WM;
  const int wn0 = (wv % (BN / WN)) * WN;

  // Per-thread source rows (fixed over the K loop).
  size_t aoff[ACH];
  const bf16* brow[BCH];
  const int kc8 = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int r = (tid >> 3) + i * (NTH / 8);
    const int rr = r < mcount ? r : mcount - 1;
    const int slot = m0 + rr;
    aoff[i] = G1 ? (size_t)(perm[slot] / kpairs) * K : (size_t)slot * K;
  }
  const bf16* We = W + (size_t)e * Nout * K;
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int r = (tid >> 3) + i * (NTH / 8);
    const int n = n0 + r < Nout ? n0 + r : Nout - 1;
    brow[i] = We + (size_t)n * K;
  }

  f32x16 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  bf16x8 ra[ACH], rl[ALO ? ACH : 1], rb[BCH];
  auto gload = [&](int kt) {
    const int kk = kt * kBK + kc8;
    const bool ok = kk < K;
    bf16x8 z;
#pragma unroll
    for (int q = 0; q < 8; ++q) z[q] = (bf16)0.f;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      ra[i] = ok ? *(const bf16x8*)(A + aoff[i] + kk) : z;
      if constexpr (ALO) rl[i] = ok ? *(const bf16x8*)(A_lo + aoff[i] + kk) : z;
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) rb[i] = ok ? *(const bf16x8*)(brow[i] + kk) : z;
  };
  auto lstore = [&](int buf) {
    bf16* as = As + buf * BM * kLdsRow;
    bf16* bs = Bs + buf * BN * kLdsRow;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int r = (tid >> 3) + i * (NTH / 8);
      *(bf16x8*)(as + r * kLdsRow + kc8) = ra[i];
      if constexpr (ALO) *(bf16x8*)(Al + buf * BM * kLdsRow + r * kLdsRow + kc8) = rl[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int r = (tid >> 3) + i * (NTH / 8);
      *(bf16x8*)(bs + r * kLdsRow + kc8) = rb[i];
    }
  };

  const int nk = cdiv(K, kBK);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const bf16* as = As + buf * BM * kLdsRow;
    const bf16* al = Al + buf * BM * kLdsRow;
    const bf16* bs = Bs + buf * BN * kLdsRow;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kof = ks * 16 + 8 * (l >> 5);
      bf16x8 af[MT], bfr[NTW];
#pragma unroll
      for (int i = 0; i < MT; ++i) af[i] = *(const bf16x8*)(as + (wm0 + i * 32 + (l & 31)) * kLdsRow + kof);
#pragma unroll
      for (int j = 0; j < NTW; ++j) bfr[j] = *(const bf16x8*)(bs + (wn0 + j * 32 + (l & 31)) * kLdsRow + kof);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      if constexpr (ALO) {
#pragma unroll
        for (int i = 0; i < MT; ++i) af[i] = *(const bf16x8*)(al + (wm0 + i * 32 + (l & 31)) * kLdsRow + kof);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NTW; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue. Lane holds column l%32 and rows 8*jj + 4*(l/32) + r of each 32x32 tile.
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int col = n0 + wn0 + j * 32 + (l & 31);
    if (col >= Nout) continue;
    const float bv = bias != nullptr ? (float)bias[(size_t)e * Nout + col] : 0.f;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = wm0 + i * 32 + 8 * (q >> 2) + 4 * (l >> 5) + (q & 3);
        if (r < mcount) {
          const int slot = m0 + r;
          const float v = acc[i][j][q] + bv;
          const size_t o = (size_t)slot * Nout + col;
          if constexpr (G1) {
            const float h = gelu_erf(v);
            const bf16 hi = (bf16)h;
            ((bf16*)out)[o] = hi;
            if constexpr (SPLIT) out_lo[o] = (bf16)(h - (float)hi);
          } else {
            ((float*)out)[o] = v * gate[slot];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- decode bf16
// Block = 4 waves = 64 weight rows of one expert; each wave 16 rows x all K.
constexpr int kDecRows = 64;
constexpr int kDecUnroll = 4;  // 64-wide K steps in flight per wave

template <bool G1, bool SPLIT>
__global__ __launch_bounds__(256) void decode_bf16_kernel(
    const bf16* __restrict__ X, const bf16* __restrict__ X_lo, const int32_t* __restrict__ perm,
    int kpairs, const int32_t* __restrict__ off, const bf16* __restrict__ W,
    const bf16* __restrict__ bias, const float* __restrict__ gate, int K, int Nout, int nblk_n,
    void* __restrict__ out, bf16* __restrict__ out_lo, int S_cap, int cap) {
  constexpr bool XLO = SPLIT && !G1;
  const int e = blockIdx.x / nblk_n;
  const int nb = blockIdx.x - e * nblk_n;
  int m0, mcount;
  expert_rows(off, e, S_cap, cap < 64 ? cap : 64, m0, mcount);
  if (mcount <= 0) return;
  const int l = lane_id();
  const int wv = threadIdx.x / kWave;
  const int r16 = l & 15, g = l >> 4;
  const int n0 = nb * kDecRows + wv * 16;
  if (n0 >= Nout) return;
  const int nrow = min(n0 + r16, Nout - 1);
  const bf16* wrow = W + ((size_t)e * Nout + nrow) * K;
  const int ng = cdiv(mcount, 16);  // <= 4
  size_t xoff[4];
#pragma unroll
  for (int sg = 0; sg < 4; ++sg) {
    const int s = min(sg * 16 + r16, mcount - 1);
    const int slot = m0 + s;
    xoff[sg] = G1 ? (size_t)(perm[slot] / kpairs) * K : (size_t)slot * K;
  }
  f32x4 acc[4];
#pragma unroll
  for (int sg = 0; sg < 4; ++sg) acc[sg] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // One 64-wide K step: lane group g owns k = 16g..16g+15 (two bf16x8 halves
  // feeding two MFMAs), so the 4 lanes of a weight row read one contiguous
  // 128-byte segment. kk_a / kk_b < 0 marks a half that lies past K (tail).
  auto step = [&](const bf16x8& w0, const bf16x8& w1, int ka, int kb) {
    bf16x8 z;
#pragma unroll
    for (int q = 0; q < 8; ++q) z[q] = (bf16)0.f;
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
      if (sg < ng) {
        const bf16x8 x0 = ka >= 0 ? *(const bf16x8*)(X + xoff[sg] + ka) : z;
        const bf16x8 x1 = kb >= 0 ? *(const bf16x8*)(X + xoff[sg] + kb) : z;
        acc[sg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, x0, acc[sg], 0, 0, 0);
        acc[sg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, x1, acc[sg], 0, 0, 0);
        if constexpr (XLO) {
          const bf16x8 y0 = ka >= 0 ? *(const bf16x8*)(X_lo + xoff[sg] + ka) : z;
          const bf16x8 y1 = kb >= 0 ? *(const bf16x8*)(X_lo + xoff[sg] + kb) : z;
          acc[sg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, y0, acc[sg], 0, 0, 0);
          acc[sg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, y1, acc[sg], 0, 0, 0);
        }
      }
    }
  };

  const int nsteps = K / 64;
  int s0 = 0;
  for (; s0 + kDecUnroll <= nsteps; s0 += kDecUnroll) {
    bf16x8 wa[kDecUnroll][2];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int kk = (s0 + u) * 64 + 16 * g;
      wa[u][0] = *(const bf16x8*)(wrow + kk);
      wa[u][1] = *(const bf16x8*)(wrow + kk + 8);
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int kk = (s0 + u) * 64 + 16 * g;
      step(wa[u][0], wa[u][1], kk, kk + 8);
    }
  }
  for (; s0 < nsteps; ++s0) {
    const int kk = s0 * 64 + 16 * g;
    step(*(const bf16x8*)(wrow + kk), *(const bf16x8*)(wrow + kk + 8), kk, kk + 8);
  }
  // K tail (K % 64 != 0, K % 8 == 0): 8-wide pieces, zero-filled.
  const int kt0 = nsteps * 64;
  if (kt0 < K) {
    const int ka = kt0 + 16 * g, kb = ka + 8;
    bf16x8 w0, w1;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      w0[q] = (bf16)0.f;
      w1[q] = (bf16)0.f;
    }
    if (ka < K) w0 = *(const bf16x8*)(wrow + ka);
    if (kb < K) w1 = *(const bf16x8*)(wrow + kb);
    step(w0, w1, ka < K ? ka : -1, kb < K ? kb : -1);
  }
  // D[n][s]: lane holds slot column s = l%16, weight rows n0 + 4g + i.
#pragma unroll
  for (int sg = 0; sg < 4; ++sg) {
    if (sg >= ng) continue;
    const int s = sg * 16 + r16;
    if (s >= mcount) continue;
    const int slot = m0 + s;
    const float gs = G1 ? 1.f : gate[slot];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 4 * g + i;
      if (n < Nout) {
        const float v = acc[sg][i] + (bias != nullptr ? (float)bias[(size_t)e * Nout + n] : 0.f);
        const size_t o = (size_t)slot * Nout + n;
        if constexpr (G1) {
          const float h = gelu_erf(v);
          const bf16 hi = (bf16)h;
          ((bf16*)out)[o] = hi;
          if constexpr (SPLIT) out_lo[o] = (bf16)(h - (float)hi);
        } else {
          ((float*)out)[o] = v * gs;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- fp32
// K split (second GEMM, gridDim.y = nsplit > 1): block (tile, q) takes the
// q-th range of kchunk K values (a multiple of 16) and writes its raw fp32
// tile to part[q][slot][n] (S_cap rows per split); the reduction adds the
// splits in order q = 0, 1, ... and applies bias and gate.
template <bool G1>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ perm, int kpairs,
    const float* __restrict__ W, const float* __restrict__ bias, const float* __restrict__ gate,
    const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles_p, int K, int Nout,
    float* __restrict__ out, int kchunk, float* __restrict__ part, int S_cap) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tile = blockIdx.x;
  if (tile >= *ntiles_p) return;
  const int kbeg = blockIdx.y * kchunk;
  const int kend = kbeg + kchunk < K ? kbeg + kchunk : K;
  const int4 te = tiles[tile];
  const int e = te.x, m0 = te.y, mcount = te.z, n0 = te.w * BN;
  const int tid = threadIdx.x;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int ar = lr < mcount ? lr : mcount - 1;
  const float* arow = G1 ? A + (size_t)(perm[m0 + ar] / kpairs) * K : A + (size_t)(m0 + ar) * K;
  const int bn = n0 + lr < Nout ? n0 + lr : Nout - 1;
  const float* brow = W + ((size_t)e * Nout + bn) * K;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    const int kk = k0 + lk;
    float4 av = make_float4(0.f, 0.f, 0.f, 0.f), bv = av;
    if (kk < kend) {
      av = *(const float4*)(arow + kk);
      bv = *(const float4*)(brow + kk);
    }
    __syncthreads();
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < BK; ++q) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[q][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = Bs[q][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= mcount) continue;
    const int slot = m0 + r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= Nout) continue;
      if (part != nullptr) {
        part[((size_t)blockIdx.y * S_cap + slot) * Nout + col] = acc[i][j];
        continue;
      }
      float v = acc[i][j] + (bias != nullptr ? bias[(size_t)e * Nout + col] : 0.f);
      v = G1 ? gelu_erf(v) : v * gate[slot];
      out[(size_t)slot * Nout + col] = v;
    }
  }
}

// The reduction of a K-split fp32 second GEMM: slot value gate * (((0 + p_0)
// + p_1) + ... + b2), the operations and order of combine_splitk_kernel, so
// moe_expert_ffn + moe_combine give the bits of the forward, which folds the
// reduction into its combine. A block per (expert, 64 output columns),
// threads over (slot, column).
__global__ __launch_bounds__(256) void reduce_f32_kernel(
    const float* __restrict__ part, int nsplit, int S_cap, int cap, const int32_t* __restrict__ off,
    const float* __restrict__ bias, const float* __restrict__ gate, int Nout, int nblk_n,
    float* __restrict__ out) {
#pragma clang fp contract(off)
  const int e = blockIdx.x / nblk_n;
  const int nb = blockIdx.x - e * nblk_n;
  int m0, mcount;
  expert_rows(off, e, S_cap, cap, m0, mcount);
  const int n0 = nb * 64;
  for (int i = threadIdx.x; i < mcount * 64; i += 256) {
    const int sl = i / 64, n = n0 + i % 64;
    if (n >= Nout) continue;
    const int slot = m0 + sl;
    float v = 0.f;
    for (int q = 0; q < nsplit; ++q) v += part[((size_t)q * S_cap + slot) * Nout + n];
    v += bias != nullptr ? bias[(size_t)e * Nout + n] : 0.f;
    out[(size_t)slot * Nout + n] = v * gate[slot];
  }
}

// ---------------------------------------------------------------- planning
enum PathKind { kPathF32 = 0, kPathDecode = 1, kPathTiledL = 2, kPathTiledM = 3 };

struct Plan {
  int path;
  int BM, BN1, BN2;
  int max1, max2;  // tile-table capacities
  bool split;
  int ks1, ks2;    // decode split-K factors (1 = none)
  bool dma1, dma2; // decode GEMMs on the LDS-DMA stream kernel
  int xg;          // decode: 16-slot groups an expert can hold (capacity / 16, rounded up to 1, 2, 4)
  int cap;         // slots an expert can hold: min(C, T)
  bool packed;     // W1 and W2 in the packed piece layout (moe_pack_weights)
};

// Split-K factor for a decode GEMM: double it (keeping at least 8 chunks of
// K per share) while there are fewer than 1024 items; measured on the
// Mixtral-shaped decode layer, more items per workgroup stream better than
// splits chosen to fill whole rounds.
int decode_splits(int N, int Nout, int K, int xg, bool xlo) {
  (void)xg;
  (void)xlo;
  const int items = N * cdiv(Nout, kDWRows);
  const int nch = K / kDKC;
  int s = 1;
  while (items * s < 1024 && s < 8 && nch / (2 * s) >= 8) s *= 2;
  return s;
}

Plan make_plan(int T, int d, int d_ff, int N, int k, int C, int S_max, int dtype, int flags) {
  Plan p{};
  p.ks1 = p.ks2 = 1;
  const int Ccap = C < T ? C : T;
  p.cap = Ccap;
  p.split = dtype == kBF16 && (flags & kFlagHiddenSplit);
  p.packed = dtype == kBF16 && (flags & kFlagPacked);
  if (dtype == kF32) {
    p.path = kPathF32;
    p.BM = 64; p.BN1 = 64; p.BN2 = 64;
  } else if (Ccap <= 64) {
    p.path = kPathDecode;
    p.BM = 64; p.BN1 = p.BN2 = kDecRows;
    p.xg = Ccap <= 16 ? 1 : (Ccap <= 32 ? 2 : 4);
    p.dma1 = d % kDKC == 0;
    p.dma2 = d_ff % kDKC == 0;
    p.ks1 = p.dma1 ? decode_splits(N, d_ff, d, p.xg, false) : 1;
    p.ks2 = p.dma2 ? decode_splits(N, d, d_ff, p.xg, p.split) : 1;
  } else if (!p.split && Ccap >= 1024 && S_max / N >= 512) {
    p.path = kPathTiledL;
    p.BM = 256; p.BN1 = p.BN2 = 256;
  } else {
    p.path = kPathTiledM;
    p.BM = 128; p.BN1 = p.BN2 = 128;
  }
  // sum_e ceil(c_e / BM) with sum c_e <= S_max and c_e <= Ccap
  const long long a = ((long long)S_max + (long long)N * (p.BM - 1)) / p.BM;
  const long long b = (long long)N * cdiv(Ccap, p.BM);
  const long long mt = a < b ? a : b;
  p.max1 = (int)(mt * cdiv(d_ff, p.BN1));
  p.max2 = (int)(mt * cdiv(d, p.BN2));
  if (p.path == kPathF32) {
    // second GEMM: split K (d_ff) while fewer than 256 blocks could run, each
    // split keeping at least 64 K values (the tiny fp32 layer: 16 tiles of
    // K = 512 on 256 CUs otherwise)
    int s = 1;
    while (p.max2 * s < 256 && d_ff / (2 * s) >= 64 && s < 8) s *= 2;
    p.ks2 = s;
  }
  return p;
}

// K values per split of an fp32 GEMM (a multiple of the kernel's 16-wide steps)
int f32_kchunk(int K, int nsplit) { return cdiv(cdiv(K, nsplit), 16) * 16; }



// Ring slots of a grouped GEMM: 4, or 3 where the split hidden layer's extra
// token rows would otherwise leave one workgroup per CU (128x128 tiles: 96 KB
// at 4 slots, 72 KB at 3); the 128x128 tiles issue each stage's copies at the
// start of a step (EARLY), which a 3-slot ring needs.
constexpr int ring_slots(bool alo) { return alo ? 3 : kRing; }

// Largest persistent grid a ring GEMM of this shape is launched with (and the
// split-tail partial buffer is sized for): the workgroups that fit in LDS on
// 256 CUs, at most one per tile, a multiple of 8. (With ring_slots, the split
// second GEMM fits no more workgroups than the first, so the partial buffer
// sized for alo = false covers both.)
constexpr int kRingCUs = 256;
int ring_grid_bound(int BM, int BN, bool alo, int max_tiles) {
  const int lds = ring_slots(alo) * (BM + BN + (alo ? BM : 0)) * kRowB;
  int occ = (160 * 1024) / lds;
  occ = occ < 1 ? 1 : occ;
  const int g = cdiv(max_tiles > 0 ? max_tiles : 1, 8) * 8;
  return g < kRingCUs * occ ? g : kRingCUs * occ;
}

// fp32 partial tiles of a ring GEMM's split tail (2 per workgroup)
size_t ring_part_floats(int BM, int BN, bool alo, int max_tiles) {
  return (size_t)ring_grid_bound(BM, BN, alo, max_tiles) * 2 * BM * BN;
}

// One grouped GEMM launch: the LDS-DMA ring kernel (+ the reduction of its
// split tail) when K % 32 == 0, else the register-staged kernel (any K % 8 == 0).
// dr (second GEMM, ring kernel only): direct rows of single-pick tokens, or
// null.
template <int BM, int BN, int WM, int WN, bool G1, bool SPLIT>
void launch_gemm(const bf16* A, const bf16* A_lo, const int32_t* perm, int k, const bf16* W,
                 const bf16* bias, const float* gate, const int4* tl, const int32_t* cnt, int K,
                 int Nout, int grid, void* out, bf16* out_lo, float* part, hipStream_t st,
                 int* wq, bool packed, const DirectRows* dr = nullptr) {
  const int32_t* dmap = dr != nullptr ? dr->map : nullptr;
  void* ydir = dr != nullptr ? dr->y : nullptr;
  const int ybf16 = dr != nullptr && dr->y_dtype == kBF16 ? 1 : 0;
  constexpr int NTH = (BM / WM) * (BN / WN) * kWave;
  constexpr bool ALO = SPLIT && !G1;
  if (K % kRK == 0) {
    constexpr int MODE = G1 ? kEpiGelu : kEpiGate;
    constexpr int R = ring_slots(ALO);
    constexpr bool EARLY = BM < 256;
    const size_t lds = (size_t)R * (BM + BN + (ALO ? BM : 0)) * kRowB;
    MOE_SET_LDS_ONCE((gemm_ring_kernel<BM, BN, WM, WN, MODE, SPLIT, R, EARLY>), lds);
    int pgrid = ring_grid((const void*)gemm_ring_kernel<BM, BN, WM, WN, MODE, SPLIT, R, EARLY>,
                          NTH, lds, grid);
    const int bound = ring_grid_bound(BM, BN, ALO, grid);
    pgrid = pgrid < bound ? pgrid : bound;
    hipLaunchKernelGGL((gemm_ring_kernel<BM, BN, WM, WN, MODE, SPLIT, R, EARLY>), dim3(pgrid),
                       dim3(NTH), lds, st, A, A_lo, perm, k, W, (const void*)bias, gate, tl, cnt, K,
                       Nout, out, out_lo, 0, 0, wq != nullptr ? nullptr : part, wq,
                       packed ? 1 : 0, dmap, ydir, ybf16);
    if (part != nullptr && wq == nullptr) {
      // at most per-1 tail tiles per XCD, BM*BN/4/256 group blocks each
      const int work = 8 * (pgrid / 8) * (BM * BN / 4 / kReduceThreads);
      hipLaunchKernelGGL((ring_reduce_kernel<BM, BN, WM, WN, MODE, SPLIT>),
                         dim3(work < 4096 ? work : 4096), dim3(kReduceThreads), 0, st, part, pgrid,
                         (const void*)bias, gate, tl, cnt, K, Nout, out, out_lo, dmap, ydir,
                         ybf16);
    }
  } else {
    const size_t lds = (size_t)2 * (BM + BN + (ALO ? BM : 0)) * kLdsRow * sizeof(bf16);
    MOE_SET_LDS_ONCE((gemm_bf16_kernel<BM, BN, WM, WN, G1, SPLIT>), lds);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, G1, SPLIT>), dim3(grid), dim3(NTH), lds,
                       st, A, A_lo, perm, k, W, bias, gate, tl, cnt, K, Nout, out, out_lo);
  }
}

template <int BM, int BN, int WM, int WN, bool SPLIT>
hipError_t launch_tiled(const void* x, const int32_t* perm, const float* gate, const void* W1,
                        const void* b1, const void* W2, const void* b2, int d, int d_ff, int k,
                        const Plan& pl, void* hid, bf16* hid_lo, const int4* t1, const int4* t2,
                        const int32_t* cnts, void* slot_out, float* part, hipStream_t st,
                        const DirectRows* dr) {
  const int g1 = cdiv(pl.max1 > 0 ? pl.max1 : 1, 8) * 8;
  const int g2 = cdiv(pl.max2 > 0 ? pl.max2 : 1, 8) * 8;
  // A GEMM with many tiles (at least four per CU: the Mixtral-shaped first
  // GEMM's 8 rounds, the capacity-limited layers' 128x128 tiles) takes them from
  // per-XCD work queues (counters zeroed by the schedule kernel): Mixtral-shaped
  // first GEMM -4%, fine-grained first -7% and second -9%. With few rounds of
  // long tiles (the Mixtral-shaped second GEMM: about 2 rounds of 448 stages)
  // the static shares and their split tail are better (+9% with the queue).
  int* wq1 = pl.max1 >= 4 * 256 ? (int*)cnts + 4 : nullptr;
  int* wq2 = pl.max2 >= 4 * 256 ? (int*)cnts + 12 : nullptr;
  profile_mark(3, st);
  launch_gemm<BM, BN, WM, WN, true, SPLIT>((const bf16*)x, nullptr, perm, k, (const bf16*)W1,
                                           (const bf16*)b1, nullptr, t1, cnts + 0, d, d_ff, g1,
                                           hid, hid_lo, part, st, wq1, pl.packed);
  profile_mark(4, st);
  launch_gemm<BM, BN, WM, WN, false, SPLIT>((const bf16*)hid, hid_lo, nullptr, k,
                                            (const bf16*)W2, (const bf16*)b2, gate, t2, cnts + 1,
                                            d_ff, d, g2, slot_out, nullptr, part, st, wq2,
                                            pl.packed, dr);
  profile_mark(5, st);
  return hipGetLastError();
}

template <bool G1, bool SPLIT, int XG, int KC>
void launch_decode_dma(int nsplit, const bf16* X, const bf16* X_lo, const int32_t* perm, int k,
                       const int32_t* off, const bf16* W, const bf16* bias, const float* gate,
                       int K, int Nout, int N, void* out, bf16* out_lo, float* part, int S_cap,
                       int cap, hipStream_t st, bool reduce, bool packed) {
  constexpr int RING = decode_ring(XG, SPLIT && !G1, KC);
  using Geo = DecodeGeom<G1, SPLIT, XG, RING, KC>;
  const int nb = cdiv(Nout, kDWRows);
  MOE_SET_LDS_ONCE((decode_dma_kernel<G1, SPLIT, XG, RING, KC>), Geo::LDS);
  const int grid = ring_grid((const void*)decode_dma_kernel<G1, SPLIT, XG, RING, KC>, 256,
                             Geo::LDS, N * nb * nsplit);
  hipLaunchKernelGGL((decode_dma_kernel<G1, SPLIT, XG, RING, KC>), dim3(grid), dim3(256), Geo::LDS,
                     st, X, X_lo, perm, k, off, W, bias, gate, K, Nout, nb, nsplit, out, out_lo,
                     part, S_cap, cap, N, packed ? 1 : 0);
  if (nsplit > 1 && reduce)
    hipLaunchKernelGGL((decode_reduce_kernel<G1, SPLIT>), dim3(N * nb), dim3(256), 0, st, part,
                       nsplit, S_cap, cap < 16 * XG ? cap : 16 * XG, off, bias, gate, Nout, nb,
                       out, out_lo);
}

// One decode GEMM: LDS-DMA stream kernel (+ split-K reduce) when K % 128 == 0,
// else the direct-load kernel. xg: 16-slot groups per expert (<= 4).
template <bool G1, bool SPLIT>
void launch_decode_gemm(bool dma, int nsplit, int xg, const bf16* X, const bf16* X_lo,
                        const int32_t* perm, int k, const int32_t* off, const bf16* W,
                        const bf16* bias, const float* gate, int K, int Nout, int N, void* out,
                        bf16* out_lo, float* part, int S_cap, int cap, hipStream_t st,
                        bool reduce, bool packed) {
  if (dma) {
    // the first GEMM (shorter K) streams better in 512-byte row chunks, one
    // workgroup per CU; the second in 256-byte chunks, two per CU (measured)
    if (G1 && K % 256 == 0 && xg <= 2) {
      if (xg <= 1)
        launch_decode_dma<G1, SPLIT, 1, 256>(nsplit, X, X_lo, perm, k, off, W, bias, gate, K,
                                             Nout, N, out, out_lo, part, S_cap, cap, st, reduce,
                                             packed);
      else
        launch_decode_dma<G1, SPLIT, 2, 256>(nsplit, X, X_lo, perm, k, off, W, bias, gate, K,
                                             Nout, N, out, out_lo, part, S_cap, cap, st, reduce,
                                             packed);
    } else if (xg <= 1) {
      launch_decode_dma<G1, SPLIT, 1, 128>(nsplit, X, X_lo, perm, k, off, W, bias, gate, K, Nout,
                                           N, out, out_lo, part, S_cap, cap, st, reduce, packed);
    } else if (xg == 2) {
      launch_decode_dma<G1, SPLIT, 2, 128>(nsplit, X, X_lo, perm, k, off, W, bias, gate, K, Nout,
                                           N, out, out_lo, part, S_cap, cap, st, reduce, packed);
    } else {
      launch_decode_dma<G1, SPLIT, 4, 128>(nsplit, X, X_lo, perm, k, off, W, bias, gate, K, Nout,
                                           N, out, out_lo, part, S_cap, cap, st, reduce, packed);
    }
    return;
  }
  const int nb = cdiv(Nout, kDecRows);
  hipLaunchKernelGGL((decode_bf16_kernel<G1, SPLIT>), dim3(N * nb), dim3(256), 0, st, X, X_lo,
                     perm, k, off, W, bias, gate, K, Nout, nb, out, out_lo, S_cap, cap);
}

template <bool SPLIT>
hipError_t launch_decode(const void* x, const int32_t* perm, const int32_t* off, const float* gate,
                         const void* W1, const void* b1, const void* W2, const void* b2, int d,
                         int d_ff, int N, int k, const Plan& pl, int S_cap, void* hid,
                         bf16* hid_lo, float* part, void* slot_out, hipStream_t st,
                         SplitK* defer) {
  const bool defer2 = defer != nullptr && pl.dma2 && pl.ks2 > 1;
  profile_mark(3, st);
  launch_decode_gemm<true, SPLIT>(pl.dma1, pl.ks1, pl.xg, (const bf16*)x, nullptr, perm, k, off,
                                  (const bf16*)W1, (const bf16*)b1, nullptr, d, d_ff, N, hid,
                                  hid_lo, part, S_cap, pl.cap, st, true, pl.packed);
  profile_mark(4, st);
  launch_decode_gemm<false, SPLIT>(pl.dma2, pl.ks2, pl.xg, (const bf16*)hid, hid_lo, perm, k, off,
                                   (const bf16*)W2, (const bf16*)b2, gate, d_ff, d, N, slot_out,
                                   nullptr, part, S_cap, pl.cap, st, !defer2, pl.packed);
  if (defer2) {
    defer->part = part;
    defer->nsplit = pl.ks2;
    defer->S_cap = S_cap;
    defer->bias = b2;
    defer->gate = gate;
    defer->off = off;
    defer->N = N;
  }
  profile_mark(5, st);
  return hipGetLastError();
}

}  // namespace

void carve_ffn(Carver& c, int T, int d, int d_ff, int N, int k, int C, int S_max, int dtype,
               int flags, FfnScratch* s) {
  const Plan pl = make_plan(T, d, d_ff, N, k, C, S_max, dtype, flags);
  const size_t rows = (size_t)(S_max > 0 ? S_max : 1);
  const size_t es = dtype == kF32 ? 4 : 2;
  s->hidden = c.take<unsigned char>(rows * d_ff * es);
  s->hidden_lo = pl.split ? (void*)c.take<bf16>(rows * d_ff) : nullptr;
  s->tiles = (int32_t*)c.take<int4>((size_t)(pl.max1 > 0 ? pl.max1 : 1) + (pl.max2 > 0 ? pl.max2 : 1));
  s->counts = c.take<int32_t>(20);
  // decode: split-K partials; tiled bf16 on the ring: split-tail partial tiles
  size_t pn = 0;
  if (pl.path == kPathDecode) {
    const size_t p1 = pl.ks1 > 1 ? (size_t)pl.ks1 * rows * d_ff : 0;
    const size_t p2 = pl.ks2 > 1 ? (size_t)pl.ks2 * rows * d : 0;
    pn = p1 > p2 ? p1 : p2;
  } else if (pl.path == kPathTiledL || pl.path == kPathTiledM) {
    const int mx = pl.max1 > pl.max2 ? pl.max1 : pl.max2;
    pn = ring_part_floats(pl.BM, pl.BN1, false, mx);
  } else if (pl.path == kPathF32 && pl.ks2 > 1) {
    pn = (size_t)pl.ks2 * rows * d;
  }
  s->part = pn ? c.take<float>(pn) : nullptr;
  s->direct = (pl.path == kPathTiledL || pl.path == kPathTiledM) ? c.take<int32_t>(rows) : nullptr;
}

hipError_t launch_expert_ffn(const void* x, const int32_t* perm, const int32_t* off,
                             const float* gate, const void* W1, const void* b1, const void* W2,
                             const void* b2, int T, int d, int d_ff, int N, int k, int C,
                             int S_max, int dtype, int flags, void* slot_out,
                             const FfnScratch& s, hipStream_t st, SplitK* defer,
                             DirectRows* dr) {
  if (defer != nullptr) defer->nsplit = 1;
  if (dr != nullptr) dr->used = false;
  if (T == 0 || S_max == 0) return hipSuccess;
  const Plan pl = make_plan(T, d, d_ff, N, k, C, S_max, dtype, flags);
  int4* t1 = (int4*)s.tiles;
  int4* t2 = t1 + (pl.max1 > 0 ? pl.max1 : 1);
  bf16* lo = (bf16*)s.hidden_lo;
  if (pl.path == kPathDecode) {
    if (pl.split)
      return launch_decode<true>(x, perm, off, gate, W1, b1, W2, b2, d, d_ff, N, k, pl, S_max,
                                 s.hidden, lo, s.part, slot_out, st, defer);
    return launch_decode<false>(x, perm, off, gate, W1, b1, W2, b2, d, d_ff, N, k, pl, S_max,
                                s.hidden, nullptr, s.part, slot_out, st, defer);
  }
  // tile order of the 128x128 GEMMs (measured with the work queues): experts of
  // one m-tile (capacity <= 128) take band-residue order for the first GEMM and
  // expert-major for the second, experts of several m-tiles the reverse. The
  // 256x256 GEMMs: band-residue for the first, expert-band-major for the
  // second (Mixtral-shaped prefill: 28% fewer bytes fetched past L2 per call,
  // 3.47 against 4.85 GB, at the same time; the first GEMM in that order
  // fetches 5% less and runs 5% longer)
  const bool single_mt = (C < T ? C : T) <= pl.BM;
  const int em = pl.path == kPathTiledM ? (single_mt ? 2 : 1) : 8;
  // every block repeats the per-expert scan (N <= 1024) and writes its share
  // of the tile entries
  const int mx = pl.max1 > pl.max2 ? pl.max1 : pl.max2;
  int sgrid = mx <= 1024 ? 1 : (cdiv(mx, 1024) < 32 ? cdiv(mx, 1024) : 32);
  // direct rows: the second GEMM on the LDS ring (bf16, d_ff % 32 == 0) writes
  // the rows of single-pick tokens into y
  const bool direct = dr != nullptr && dr->y != nullptr && dr->inv != nullptr &&
                      s.direct != nullptr && d_ff % kRK == 0 &&
                      (pl.path == kPathTiledL || pl.path == kPathTiledM);
  if (direct) {
    dr->map = s.direct;
    dr->used = true;
    // a block per 1024 tokens for the map (up to 64)
    const int tg = cdiv(T, 1024) < 64 ? cdiv(T, 1024) : 64;
    sgrid = sgrid > tg ? sgrid : tg;
  }
  hipLaunchKernelGGL(schedule_kernel, dim3(sgrid), dim3(1024), 0, st, off, N, S_max, C < T ? C : T,
                     pl.BM, cdiv(d_ff, pl.BN1), cdiv(d, pl.BN2), pl.max1, pl.max2, em, t1, t2,
                     s.counts, direct ? dr->inv : nullptr, T, k, direct ? s.direct : nullptr);
  if (pl.path == kPathF32) {
    profile_mark(3, st);
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(pl.max1 > 0 ? pl.max1 : 1), dim3(256), 0, st,
                       (const float*)x, perm, k, (const float*)W1, (const float*)b1, nullptr, t1,
                       s.counts + 0, d, d_ff, (float*)s.hidden, f32_kchunk(d, 1), nullptr, 0);
    profile_mark(4, st);
    const int ks = pl.ks2;
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(pl.max2 > 0 ? pl.max2 : 1, ks), dim3(256), 0,
                       st, (const float*)s.hidden, nullptr, k, (const float*)W2, (const float*)b2,
                       gate, t2, s.counts + 1, d_ff, d, (float*)slot_out, f32_kchunk(d_ff, ks),
                       ks > 1 ? s.part : nullptr, S_max);
    if (ks > 1) {
      if (defer != nullptr) {
        // the combine finishes the slot values (combine_splitk_kernel)
        defer->part = s.part;
        defer->nsplit = ks;
        defer->S_cap = S_max;
        defer->bias = b2;
        defer->f32 = true;
        defer->gate = gate;
        defer->off = off;
        defer->N = N;
      } else {
        const int nbn = cdiv(d, 64);
        hipLaunchKernelGGL(reduce_f32_kernel, dim3(N * nbn), dim3(256), 0, st, s.part, ks, S_max,
                           pl.cap, off, (const float*)b2, gate, d, nbn, (float*)slot_out);
      }
    }
    profile_mark(5, st);
    return hipGetLastError();
  }
  if (pl.path == kPathTiledL)
    return launch_tiled<256, 256, 128, 64, false>(x, perm, gate, W1, b1, W2, b2, d, d_ff, k, pl,
                                                   s.hidden, nullptr, t1, t2, s.counts, slot_out,
                                                   s.part, st, direct ? dr : nullptr);
  if (pl.split)
    return launch_tiled<128, 128, 64, 64, true>(x, perm, gate, W1, b1, W2, b2, d, d_ff, k, pl,
                                                 s.hidden, lo, t1, t2, s.counts, slot_out, s.part,
                                                 st, direct ? dr : nullptr);
  return launch_tiled<128, 128, 64, 64, false>(x, perm, gate, W1, b1, W2, b2, d, d_ff, k, pl,
                                                s.hidden, nullptr, t1, t2, s.counts, slot_out,
                                                s.part, st, direct ? dr : nullptr);
}

namespace {
// Packed weight layout (see gemm_ring.h): output word g (16 bytes) of piece
// (e, row block rb, K chunk kc) = g / 64 is word w = g % 64 of the piece: row
// rb*16 + piece_row(w), 8 bf16 from K offset kc*32 + 8*piece_chunk(w). A grid
// stride over the words; consecutive threads write consecutive words.
__global__ __launch_bounds__(256) void pack_weights_kernel(const bf16* __restrict__ W, int rows,
                                                           int K, size_t words,
                                                           uint4* __restrict__ out) {
  const int kcs = K / 32, rbs = rows / 16;
  for (size_t g = (size_t)blockIdx.x * 256 + threadIdx.x; g < words;
       g += (size_t)gridDim.x * 256) {
    const int w = (int)(g & 63);
    const size_t piece = g >> 6;
    const int kc = (int)(piece % kcs);
    const size_t rest = piece / kcs;
    const int rb = (int)(rest % rbs);
    const size_t e = rest / rbs;
    const int row = rb * 16 + piece_row(w);
    const int chunk = piece_chunk(w);
    out[g] = *(const uint4*)(W + ((e * rows + row) * K + (size_t)kc * 32 + chunk * 8));
  }
}
}  // namespace

hipError_t launch_pack_weights(const void* W, int N, int rows, int K, void* out,
                               hipStream_t st) {
  const size_t words = (size_t)N * rows * K / 8;
  if (words == 0) return hipSuccess;
  const size_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(pack_weights_kernel, dim3(blocks < 65536 ? (unsigned)blocks : 65536u),
                     dim3(256), 0, st, (const bf16*)W, rows, K, words, (uint4*)out);
  return hipGetLastError();
}

namespace {
// Identity dispatch of a shared expert: one expert holding every token in
// order (slot t = token t), combine weight 1.
__global__ __launch_bounds__(256) void identity_dispatch_kernel(int T, int32_t* __restrict__ perm,
                                                                int32_t* __restrict__ off,
                                                                float* __restrict__ gate) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < T) {
    perm[t] = t;
    gate[t] = 1.0f;
  }
  if (t == 0) {
    off[0] = 0;
    off[1] = T;
  }
}
}  // namespace

void carve_shared(Carver& c, int T, int d, int d_fs, int dtype, int flags, SharedScratch* s) {
  const size_t n = (size_t)(T > 0 ? T : 1);
  s->perm = c.take<int32_t>(n);
  s->off = c.take<int32_t>(2);
  s->gate = c.take<float>(n);
  carve_ffn(c, T, d, d_fs, 1, 1, T, T, dtype, flags, &s->fs);
}

hipError_t launch_shared_expert(const void* x, const void* W1s, const void* b1s, const void* W2s,
                                const void* b2s, int T, int d, int d_fs, int dtype, int flags,
                                float* out, const SharedScratch& s, hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(identity_dispatch_kernel, dim3(cdiv(T, 256)), dim3(256), 0, st, T, s.perm,
                     s.off, s.gate);
  return launch_expert_ffn(x, s.perm, s.off, s.gate, W1s, b1s, W2s, b2s, T, d, d_fs, 1, 1, T, T,
                           dtype, flags, out, s.fs, st, nullptr);
}

}  // namespace moe
