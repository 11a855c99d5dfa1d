// Grouped / plain bf16 GEMM on an LDS-DMA ring, shared by the expert FFN and
// the wide router. gfx950: global_load_lds_dwordx4, v_mfma_f32_32x32x16_bf16.
#pragma once

#include "moe_common.h"

namespace moe {

// Epilogue / tiling modes of gemm_ring_kernel.
constexpr int kEpiGelu = 0;   // expert GEMM1: gather x through perm, GELU, bf16 hidden
constexpr int kEpiGate = 1;   // expert GEMM2: gate * (acc + b2), fp32 slot output
constexpr int kEpiLogit = 2;  // router: static tiles, fp32 acc + fp32 bias, row stride ldo

namespace {

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

template <int BM, int BN, int WM, int WN, int MODE, bool SPLIT>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * kWave) void gemm_ring_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ A_lo, const int32_t* __restrict__ perm,
    int kpairs, const bf16* __restrict__ W, const bf16* __restrict__ bias,
    const float* __restrict__ gate, const int4* __restrict__ tiles,
    const int32_t* __restrict__ ntiles_p, int K, int Nout, void* __restrict__ out,
    bf16* __restrict__ out_lo, int M_total, int ldo) {
  constexpr bool G1 = MODE == kEpiGelu;
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

  int e, m0, mcount, n0;
  if constexpr (MODE == kEpiLogit) {
    // static tiling over [M_total rows] x [Nout rows of W]: n-tiles fastest
    const int ntn = (Nout + BN - 1) / BN;
    const int tile = blockIdx.x;
    const int mt = tile / ntn;
    e = 0;
    m0 = mt * BM;
    if (m0 >= M_total) return;
    mcount = min(BM, M_total - m0);
    n0 = (tile - mt * ntn) * BN;
  } else {
    const int ntiles = *ntiles_p;
    const int b = blockIdx.x;
    const int chunk = (ntiles + 7) >> 3;
    const int jx = b >> 3;
    const int tile = (b & 7) * chunk + jx;
    if (jx >= chunk || tile >= ntiles) return;
    const int4 te = tiles[tile];
    e = te.x; m0 = te.y; mcount = te.z; n0 = te.w * BN;
  }

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
    if constexpr (MODE == kEpiLogit) {
      if (col >= ldo) continue;
      const float bv = bias != nullptr ? ((const float*)bias)[col] : 0.f;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = wm0 + i * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
          if (r < mcount) ((float*)out)[(size_t)(m0 + r) * ldo + col] = acc[i][j][q] + bv;
        }
      continue;
    }
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


}  // namespace

}  // namespace moe
