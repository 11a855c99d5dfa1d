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
// Three code paths, chosen on the host from sizes only (no device sync):
//   tiled bf16  : grouped GEMM on v_mfma_f32_32x32x16_bf16, LDS double-buffered
//                 tiles (BM x BN x 64), token gather fused into the A-tile load
//                 of GEMM1, GELU fused into GEMM1's epilogue, bias and gate
//                 fused into GEMM2's (fp32 output). Tiles come from a device-built schedule
//                 (expert, n-tile, m-tile fastest) walked in an XCD-aware
//                 order: each of the 8 XCDs takes one contiguous run of tiles
//                 so m-tiles sharing a weight tile share that XCD's L2.
//   decode bf16 : when an expert can hold at most 64 slots, weights are
//                 streamed once with v_mfma_f32_16x16x32_bf16 (weight rows as
//                 the 16-row operand, slots as the 16-column operand), 128-byte
//                 row segments per 4 lanes.
//   fp32        : FMA tiles (64 x 64), same schedule mechanism.
// With the hidden-split flag, GEMM1 also stores the bf16 residual h - bf16(h)
// of each hidden activation and GEMM2 runs a second MFMA on it, so GEMM2 sees
// the hidden layer to about 16 significant bits instead of 8 (twice GEMM2's
// MFMA work; used where the weight stream, not MFMA, bounds the time).
#include "moe_common.h"

namespace moe {

namespace {

// ---------------------------------------------------------------- schedule
// Tile entry: {expert, first slot of the m-tile, rows in the m-tile, n-tile}.
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* __restrict__ off, int N,
                                                        int BM, int NT1, int NT2, int max1,
                                                        int max2, int4* __restrict__ tiles1,
                                                        int4* __restrict__ tiles2,
                                                        int32_t* __restrict__ counts) {
  __shared__ int mtoff[kMaxN + 1];
  __shared__ int tmp[17];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  for (int e0 = 0; e0 < N; e0 += 1024) {
    const int e = e0 + threadIdx.x;
    const int mt = (e < N) ? cdiv(off[e + 1] - off[e], BM) : 0;
    // block exclusive scan
    const int l = lane_id(), wv = threadIdx.x / kWave;
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
    for (int i = threadIdx.x; i < total; i += 1024) {
      // expert e: largest e with mtoff[e] * NTn <= i
      int lo = 0, hi = N - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mtoff[mid] * NTn <= i) lo = mid; else hi = mid - 1;
      }
      const int e = lo;
      const int me = mtoff[e + 1] - mtoff[e];
      const int local = i - mtoff[e] * NTn;
      const int nt = local / me, mt = local - nt * me;
      const int cnt_e = off[e + 1] - off[e];
      tl[i] = make_int4(e, off[e] + mt * BM, min(BM, cnt_e - mt * BM), nt);
    }
    if (threadIdx.x == 0) counts[pass] = total;
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

// ---------------------------------------------------------------- tiled bf16, LDS-DMA ring
// Fast path for K % 32 == 0. Tiles stream into a 4-slot LDS ring with
// global_load_lds_dwordx4 (each lane's 16 bytes land at base + 16 * lane, so a
// wave instruction fills 16 rows x 64 bytes); no VGPR staging and no ds_write.
// Rows are 64 bytes (32 bf16 of K); the 16-byte chunk c of row r sits at
// position c ^ ((r >> 2) & 3), which keeps the b128 fragment reads of 16
// consecutive rows on distinct banks. Stage kt+3 is requested while stage kt
// is multiplied; one wave barrier per stage, taken mid-stage so that the next
// stage's first fragments are read while the current stage's last MFMAs run.
constexpr int kRK = 32;       // K per ring stage
constexpr int kRing = 4;      // ring slots
constexpr int kRowB = kRK * 2;  // bytes per tile row per stage

#define MOE_LDS __attribute__((address_space(3)))

// s_waitcnt vmcnt(N) with expcnt/lgkmcnt unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void vm_wait_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// 16 bytes per lane, global -> LDS (lane i lands at dst + 16 * i).
__device__ __forceinline__ void dma16(const unsigned char* src, MOE_LDS unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BM, int BN, int WM, int WN, bool G1, bool SPLIT>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * kWave) void gemm_ring_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ A_lo, const int32_t* __restrict__ perm,
    int kpairs, const bf16* __restrict__ W, const bf16* __restrict__ bias,
    const float* __restrict__ gate, const int4* __restrict__ tiles,
    const int32_t* __restrict__ ntiles_p, int K, int Nout, void* __restrict__ out,
    bf16* __restrict__ out_lo) {
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int MT = WM / 32, NTW = WN / 32;
  constexpr bool ALO = SPLIT && !G1;
  constexpr int AI = BM / (NW * 16);  // A wave-loads per stage
  constexpr int BI = BN / (NW * 16);
  constexpr int LPS = AI + BI + (ALO ? AI : 0);  // loads per wave per stage
  constexpr int A_OFF = 0;
  constexpr int B_OFF = BM * kRowB;
  constexpr int L_OFF = B_OFF + BN * kRowB;
  constexpr int STAGE = L_OFF + (ALO ? BM * kRowB : 0);
  static_assert(AI >= 1 && BI >= 1, "tile too small for the wave count");
  static_assert(2 * LPS < 64, "vmcnt range");

  extern __shared__ __align__(16) unsigned char smem[];

  const int ntiles = *ntiles_p;
  const int b = blockIdx.x;
  const int chunk = (ntiles + 7) >> 3;
  const int jx = b >> 3;
  const int tile = (b & 7) * chunk + jx;
  if (jx >= chunk || tile >= ntiles) return;
  const int4 te = tiles[tile];
  const int e = te.x, m0 = te.y, mcount = te.z, n0 = te.w * BN;

  const int l = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm0 = (wv / (BN / WN)) * WM;
  const int wn0 = (wv % (BN / WN)) * WN;

  // DMA source pointers: wave-load i covers tile rows (i*NW + wv)*16 .. +16;
  // lane l fills row +l/4, position l%4, which holds chunk (l%4) ^ ((l>>4)&3).
  const int csw = ((l & 3) ^ ((l >> 4) & 3)) * 16;  // byte offset of the chunk
  const unsigned char* pa[AI];
  const unsigned char* pl[ALO ? AI : 1];
  const unsigned char* pb[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = (i * NW + wv) * 16 + (l >> 2);
    const int rr = r < mcount ? r : mcount - 1;
    const int slot = m0 + rr;
    const size_t row = G1 ? (size_t)(perm[slot] / kpairs) : (size_t)slot;
    pa[i] = (const unsigned char*)(A + row * K) + csw;
    if constexpr (ALO) pl[i] = (const unsigned char*)(A_lo + row * K) + csw;
  }
  const bf16* We = W + (size_t)e * Nout * K;
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int r = (i * NW + wv) * 16 + (l >> 2);
    const int n = n0 + r < Nout ? n0 + r : Nout - 1;
    pb[i] = (const unsigned char*)(We + (size_t)n * K) + csw;
  }
  MOE_LDS unsigned char* lds = (MOE_LDS unsigned char*)smem;
  auto issue_stage = [&](int slot, int kt) {
    MOE_LDS unsigned char* st = lds + (slot & (kRing - 1)) * STAGE;
    const int kb = kt * kRowB;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      dma16(pa[i] + kb, st + A_OFF + (i * NW + wv) * 1024);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      dma16(pb[i] + kb, st + B_OFF + (i * NW + wv) * 1024);
    if constexpr (ALO) {
#pragma unroll
      for (int i = 0; i < AI; ++i)
        dma16(pl[i] + kb, st + L_OFF + (i * NW + wv) * 1024);
    }
  };

  // Fragment reads: row R, 16-byte chunk c (= 2*ks + l/32) at position c ^ ((R>>2)&3).
  const int lr = l & 31;
  const int half = l >> 5;
  int aoffs[MT], boffs[NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i) aoffs[i] = (wm0 + i * 32 + lr) * kRowB;
#pragma unroll
  for (int j = 0; j < NTW; ++j) boffs[j] = (wn0 + j * 32 + lr) * kRowB;
  const int sw = (lr >> 2) & 3;  // (R >> 2) & 3 with R = 32*x + lr
  const int pos0 = ((0 + half) ^ sw) * 16;  // ks = 0
  const int pos1 = ((2 + half) ^ sw) * 16;  // ks = 1

  bf16x8 af[2][MT], bfr[2][NTW], alf[ALO ? 2 : 1][ALO ? MT : 1];
  auto read_frags = [&](int kt, int ks, int set) {
    const unsigned char* st = smem + (kt & (kRing - 1)) * STAGE;
    const int pos = ks ? pos1 : pos0;
#pragma unroll
    for (int i = 0; i < MT; ++i) af[set][i] = *(const bf16x8*)(st + A_OFF + aoffs[i] + pos);
#pragma unroll
    for (int j = 0; j < NTW; ++j) bfr[set][j] = *(const bf16x8*)(st + B_OFF + boffs[j] + pos);
    if constexpr (ALO) {
#pragma unroll
      for (int i = 0; i < MT; ++i) alf[set][i] = *(const bf16x8*)(st + L_OFF + aoffs[i] + pos);
    }
  };

  f32x16 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  auto mma = [&](int set) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[set][i], bfr[set][j], acc[i][j], 0, 0, 0);
    if constexpr (ALO) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alf[set][i], bfr[set][j], acc[i][j], 0, 0, 0);
    }
  };

  const int nk = K / kRK;
  // Every ring step issues exactly LPS loads per wave: stage min(s, nk-1) into
  // slot s % 4 (past the last stage the copies land in slots nobody reads), so
  // "stage s+1 has landed" is always vmcnt <= LPS at the wait below.
  issue_stage(0, 0);
  issue_stage(1, nk > 1 ? 1 : nk - 1);
  issue_stage(2, nk > 2 ? 2 : nk - 1);
  vm_wait_n<2 * LPS>();
  wg_barrier();
  read_frags(0, 0, 0);

  for (int kt = 0; kt < nk; ++kt) {
    // fragments (kt, ks=0) are in set 0
    read_frags(kt, 1, 1);
    mma(0);
    // issue the (kt, ks=1) fragment reads between the first MFMAs
#pragma unroll
    for (int q = 0; q < MT + NTW + (ALO ? MT : 0); ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // stage kt+1 has landed (only stage kt+2's loads may still fly) and no
    // wave still reads the slot of stage kt-1
    lgkm_wait0();
    vm_wait_n<LPS>();
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_stage(kt + 3, kt + 3 < nk ? kt + 3 : nk - 1);
    read_frags(kt + 1, 0, 0);  // past the last stage: reads a dead slot, never used
    mma(1);
    // interleave: one MFMA, one DMA issue (x LPS), then one MFMA, one fragment read
#pragma unroll
    for (int q = 0; q < LPS; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
#pragma unroll
    for (int q = 0; q < MT + NTW + (ALO ? MT : 0); ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  vm_wait_n<0>();  // no LDS DMA may outlive the workgroup

  // Epilogue. Lane holds column l%32 and rows 8*jj + 4*(l/32) + r of each 32x32 tile.
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int col = n0 + wn0 + j * 32 + lr;
    if (col >= Nout) continue;
    const float bv = bias != nullptr ? (float)bias[(size_t)e * Nout + col] : 0.f;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = wm0 + i * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
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
    void* __restrict__ out, bf16* __restrict__ out_lo) {
  constexpr bool XLO = SPLIT && !G1;
  const int e = blockIdx.x / nblk_n;
  const int nb = blockIdx.x - e * nblk_n;
  const int m0 = off[e];
  const int mcount = off[e + 1] - m0;
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
template <bool G1>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ perm, int kpairs,
    const float* __restrict__ W, const float* __restrict__ bias, const float* __restrict__ gate,
    const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles_p, int K, int Nout,
    float* __restrict__ out) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tile = blockIdx.x;
  if (tile >= *ntiles_p) return;
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
  for (int k0 = 0; k0 < K; k0 += BK) {
    const int kk = k0 + lk;
    float4 av = make_float4(0.f, 0.f, 0.f, 0.f), bv = av;
    if (kk < K) {
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
      float v = acc[i][j] + (bias != nullptr ? bias[(size_t)e * Nout + col] : 0.f);
      v = G1 ? gelu_erf(v) : v * gate[slot];
      out[(size_t)slot * Nout + col] = v;
    }
  }
}

// ---------------------------------------------------------------- planning
enum PathKind { kPathF32 = 0, kPathDecode = 1, kPathTiledL = 2, kPathTiledM = 3 };

struct Plan {
  int path;
  int BM, BN1, BN2;
  int max1, max2;  // tile-table capacities
  bool split;
};

Plan make_plan(int T, int d, int d_ff, int N, int k, int C, int S_max, int dtype, int flags) {
  Plan p{};
  const int Ccap = C < T ? C : T;
  p.split = dtype == kBF16 && (flags & kFlagHiddenSplit);
  if (dtype == kF32) {
    p.path = kPathF32;
    p.BM = 64; p.BN1 = 64; p.BN2 = 64;
  } else if (Ccap <= 64) {
    p.path = kPathDecode;
    p.BM = 64; p.BN1 = p.BN2 = kDecRows;
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
  return p;
}

// once per call site (idempotent; a race between threads only repeats the call)
#define MOE_SET_LDS_ONCE(kern, lds)                                                        \
  do {                                                                                     \
    static bool done_ = false;                                                             \
    if (!done_) {                                                                          \
      hipFuncSetAttribute((const void*)(kern), hipFuncAttributeMaxDynamicSharedMemorySize, \
                          (int)(lds));                                                     \
      done_ = true;                                                                        \
    }                                                                                      \
  } while (0)

// One grouped GEMM launch: the LDS-DMA ring kernel when K % 32 == 0, else the
// register-staged kernel (any K % 8 == 0).
template <int BM, int BN, int WM, int WN, bool G1, bool SPLIT>
void launch_gemm(const bf16* A, const bf16* A_lo, const int32_t* perm, int k, const bf16* W,
                 const bf16* bias, const float* gate, const int4* tl, const int32_t* cnt, int K,
                 int Nout, int grid, void* out, bf16* out_lo, hipStream_t st) {
  constexpr int NTH = (BM / WM) * (BN / WN) * kWave;
  constexpr bool ALO = SPLIT && !G1;
  if (K % kRK == 0) {
    const size_t lds = (size_t)kRing * (BM + BN + (ALO ? BM : 0)) * kRowB;
    MOE_SET_LDS_ONCE((gemm_ring_kernel<BM, BN, WM, WN, G1, SPLIT>), lds);
    hipLaunchKernelGGL((gemm_ring_kernel<BM, BN, WM, WN, G1, SPLIT>), dim3(grid), dim3(NTH), lds,
                       st, A, A_lo, perm, k, W, bias, gate, tl, cnt, K, Nout, out, out_lo);
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
                        const int32_t* cnts, void* slot_out, hipStream_t st) {
  const int g1 = cdiv(pl.max1 > 0 ? pl.max1 : 1, 8) * 8;
  const int g2 = cdiv(pl.max2 > 0 ? pl.max2 : 1, 8) * 8;
  profile_mark(3, st);
  launch_gemm<BM, BN, WM, WN, true, SPLIT>((const bf16*)x, nullptr, perm, k, (const bf16*)W1,
                                           (const bf16*)b1, nullptr, t1, cnts + 0, d, d_ff, g1,
                                           hid, hid_lo, st);
  profile_mark(4, st);
  launch_gemm<BM, BN, WM, WN, false, SPLIT>((const bf16*)hid, hid_lo, nullptr, k,
                                            (const bf16*)W2, (const bf16*)b2, gate, t2, cnts + 1,
                                            d_ff, d, g2, slot_out, nullptr, st);
  profile_mark(5, st);
  return hipGetLastError();
}

template <bool SPLIT>
hipError_t launch_decode(const void* x, const int32_t* perm, const int32_t* off, const float* gate,
                         const void* W1, const void* b1, const void* W2, const void* b2, int d,
                         int d_ff, int N, int k, void* hid, bf16* hid_lo, void* slot_out,
                         hipStream_t st) {
  const int nb1 = cdiv(d_ff, kDecRows), nb2 = cdiv(d, kDecRows);
  profile_mark(3, st);
  hipLaunchKernelGGL((decode_bf16_kernel<true, SPLIT>), dim3(N * nb1), dim3(256), 0, st,
                     (const bf16*)x, nullptr, perm, k, off, (const bf16*)W1, (const bf16*)b1,
                     nullptr, d, d_ff, nb1, hid, hid_lo);
  profile_mark(4, st);
  hipLaunchKernelGGL((decode_bf16_kernel<false, SPLIT>), dim3(N * nb2), dim3(256), 0, st,
                     (const bf16*)hid, (const bf16*)hid_lo, perm, k, off, (const bf16*)W2,
                     (const bf16*)b2, gate, d_ff, d, nb2, slot_out, nullptr);
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
  s->counts = c.take<int32_t>(4);
}

hipError_t launch_expert_ffn(const void* x, const int32_t* perm, const int32_t* off,
                             const float* gate, const void* W1, const void* b1, const void* W2,
                             const void* b2, int T, int d, int d_ff, int N, int k, int C,
                             int S_max, int dtype, int flags, void* slot_out,
                             const FfnScratch& s, hipStream_t st) {
  if (T == 0 || S_max == 0) return hipSuccess;
  const Plan pl = make_plan(T, d, d_ff, N, k, C, S_max, dtype, flags);
  int4* t1 = (int4*)s.tiles;
  int4* t2 = t1 + (pl.max1 > 0 ? pl.max1 : 1);
  bf16* lo = (bf16*)s.hidden_lo;
  if (pl.path == kPathDecode) {
    if (pl.split)
      return launch_decode<true>(x, perm, off, gate, W1, b1, W2, b2, d, d_ff, N, k, s.hidden, lo,
                                 slot_out, st);
    return launch_decode<false>(x, perm, off, gate, W1, b1, W2, b2, d, d_ff, N, k, s.hidden,
                                nullptr, slot_out, st);
  }
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, st, off, N, pl.BM,
                     cdiv(d_ff, pl.BN1), cdiv(d, pl.BN2), pl.max1, pl.max2, t1, t2, s.counts);
  if (pl.path == kPathF32) {
    profile_mark(3, st);
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(pl.max1 > 0 ? pl.max1 : 1), dim3(256), 0, st,
                       (const float*)x, perm, k, (const float*)W1, (const float*)b1, nullptr, t1,
                       s.counts + 0, d, d_ff, (float*)s.hidden);
    profile_mark(4, st);
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(pl.max2 > 0 ? pl.max2 : 1), dim3(256), 0, st,
                       (const float*)s.hidden, nullptr, k, (const float*)W2, (const float*)b2, gate,
                       t2, s.counts + 1, d_ff, d, (float*)slot_out);
    profile_mark(5, st);
    return hipGetLastError();
  }
  if (pl.path == kPathTiledL)
    return launch_tiled<256, 256, 128, 128, false>(x, perm, gate, W1, b1, W2, b2, d, d_ff, k, pl,
                                                    s.hidden, nullptr, t1, t2, s.counts, slot_out,
                                                    st);
  if (pl.split)
    return launch_tiled<128, 128, 64, 64, true>(x, perm, gate, W1, b1, W2, b2, d, d_ff, k, pl,
                                                 s.hidden, lo, t1, t2, s.counts, slot_out, st);
  return launch_tiled<128, 128, 64, 64, false>(x, perm, gate, W1, b1, W2, b2, d, d_ff, k, pl,
                                                s.hidden, nullptr, t1, t2, s.counts, slot_out, st);
}

}  // namespace moe
