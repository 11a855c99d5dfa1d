// Grouped / plain bf16 GEMM on an LDS-DMA ring, shared by the expert FFN and
// the wide router. gfx950: global_load_lds_dwordx4, v_mfma_f32_32x32x16_bf16.
#pragma once

#include "moe_common.h"

#include <type_traits>

namespace moe {

// Epilogue / tiling modes of gemm_ring_kernel.
constexpr int kEpiGelu = 0;   // expert GEMM1: gather x through perm, GELU, bf16 hidden
constexpr int kEpiGate = 1;   // expert GEMM2: gate * (acc + b2), fp32 slot output
constexpr int kEpiLogit = 2;  // router: static tiles, fp32 acc + fp32 bias, row stride ldo

// GELU z * Phi(z) for the expert FFN epilogue, written as
//   h = max(z, 0) - |z| * erfc(|z| / sqrt 2) / 2,
// with erfc from the rational approximation 7.1.26 of Abramowitz and Stegun
// (Handbook of Mathematical Functions): erfc(x) ~ t (a1 + a2 t + ... + a5 t^4)
// exp(-x^2), t = 1 / (1 + p x), x >= 0, absolute error at most 1.5e-7. So the
// absolute error of h is at most |z| * 0.75e-7 plus a few fp32 roundings; the
// exact erf form of GELU is what is computed (not the tanh form).
__device__ __forceinline__ float gelu_as(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f),
                       -0.284496736f),
               0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-(x * x) * 1.44269504088896341f);  // exp(-x^2)
  return fmaxf(z, 0.0f) - 0.5f * fabsf(z) * (poly * e);
}

namespace {

// ---------------------------------------------------------------- tiled bf16, LDS-DMA ring
// Fast path for K % 32 == 0. Tiles stream into a RING-slot LDS ring with
// global_load_lds_dwordx4 (each lane's 16 bytes land at base + 16 * lane, so a
// wave instruction fills 16 rows x 64 bytes); no VGPR staging and no ds_write.
// Rows are 64 bytes (32 bf16 of K); the 16-byte chunk c of row r sits at
// position c ^ ((r >> 2) & 3), which keeps the b128 fragment reads of 16
// consecutive rows on distinct banks. Stage kt+RING-1 is requested while stage
// kt is multiplied; one workgroup barrier per stage, taken mid-stage so that
// the next stage's first fragments are read while the current stage's last
// MFMAs run.
//
// Persistent: the grid holds one wave of resident workgroups; workgroup b runs
// on XCD b % 8 and walks the tiles of that XCD's contiguous share of the tile
// list, so the 8 L2s each see their own band of weights and token rows. The
// next tile's first RING-1 stages are requested before the current tile's
// epilogue, so their latency hides behind it.
//
// MFMA operands: the weight fragment is the matrix-core A operand and the
// token fragment the B operand, so each lane's accumulator holds one token row
// and 4 consecutive output columns per 32x32 block: the epilogue writes 8-byte
// (bf16) or 16-byte (fp32) vectors.
constexpr int kRK = 32;         // K per ring stage
constexpr int kRing = 4;        // default ring slots
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

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16 ha = (bf16)a, hb = (bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Resident workgroups for a persistent ring kernel: every workgroup that fits
// on the device at once, at most one per tile, rounded up to a multiple of 8
// (one share per XCD).
inline int ring_grid(const void* kernel, int threads, size_t lds, int max_tiles) {
  int dev = 0, cus = 0, occ = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, lds) != hipSuccess ||
      occ < 1)
    occ = 1;
  (void)hipGetLastError();
  long long g = (long long)cus * occ;
  const long long mt = max_tiles > 0 ? max_tiles : 1;
  if (g > mt) g = mt;
  return (int)((g + 7) / 8 * 8);
}

template <int BM, int BN, int WM, int WN, int MODE, bool SPLIT, int RING>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * kWave) void gemm_ring_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ A_lo, const int32_t* __restrict__ perm,
    int kpairs, const bf16* __restrict__ W, const void* __restrict__ bias,
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
  static_assert(RING >= 3 && (RING - 2) * LPS < 64, "ring depth / vmcnt range");

  extern __shared__ __align__(16) unsigned char smem[];

  // ---- this workgroup's share of the tile list
  int ntiles;
  if constexpr (MODE == kEpiLogit) {
    ntiles = ((M_total + BM - 1) / BM) * ((Nout + BN - 1) / BN);
  } else {
    ntiles = *ntiles_p;
  }
  const int xcd = blockIdx.x & 7;
  const int per = gridDim.x >> 3;
  const int chunk = (ntiles + 7) >> 3;
  int jt = blockIdx.x >> 3;
  if (jt >= chunk || xcd * chunk + jt >= ntiles) return;

  auto decode = [&](int tile, int& e, int& m0, int& mcount, int& n0) {
    if constexpr (MODE == kEpiLogit) {
      const int ntn = (Nout + BN - 1) / BN;  // n-tiles fastest
      const int mt = tile / ntn;
      e = 0;
      m0 = mt * BM;
      mcount = min(BM, M_total - m0);
      n0 = (tile - mt * ntn) * BN;
    } else {
      const int4 te = tiles[tile];
      e = te.x; m0 = te.y; mcount = te.z; n0 = te.w * BN;
    }
  };

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
  auto set_ptrs = [&](int e, int m0, int mcount, int n0) {
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
  };
  MOE_LDS unsigned char* lds = (MOE_LDS unsigned char*)smem;
  const int nk = K / kRK;
  // A stage's copies go out in two parts: part 0 (token rows, and their
  // residual rows) right after the mid-stage barrier, part 1 (weight rows) in
  // the first half of the next ring step, so the vector-memory issue is spread
  // over the whole step instead of bursting.
  auto issue_part = [&](int kt, int part) {
    const int src_kt = kt < nk ? kt : nk - 1;  // past the last stage: a dead copy
    MOE_LDS unsigned char* st = lds + (kt % RING) * STAGE;
    const int kb = src_kt * kRowB;
    if (part == 0) {
#pragma unroll
      for (int i = 0; i < AI; ++i)
        dma16(pa[i] + kb, st + A_OFF + (i * NW + wv) * 1024);
      if constexpr (ALO) {
#pragma unroll
        for (int i = 0; i < AI; ++i)
          dma16(pl[i] + kb, st + L_OFF + (i * NW + wv) * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < BI; ++i)
        dma16(pb[i] + kb, st + B_OFF + (i * NW + wv) * 1024);
    }
  };
  // prologue of a tile: stages 0 .. RING-3 whole, stage RING-2 part 0
  auto issue_prologue = [&]() {
#pragma unroll
    for (int q = 0; q < RING - 2; ++q) {
      issue_part(q, 0);
      issue_part(q, 1);
    }
    issue_part(RING - 2, 0);
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
  // RAG: a partly filled tile; token blocks i >= na (rows past mcount) are
  // neither read nor multiplied (na is uniform per wave).
  int na = MT;
  auto read_frags = [&](int kt, int ks, int set, auto rag) {
    constexpr bool RAG = decltype(rag)::value;
    const unsigned char* st = smem + (kt % RING) * STAGE;
    const int pos = ks ? pos1 : pos0;
#pragma unroll
    for (int i = 0; i < MT; ++i)
      if (!RAG || i < na) af[set][i] = *(const bf16x8*)(st + A_OFF + aoffs[i] + pos);
#pragma unroll
    for (int j = 0; j < NTW; ++j) bfr[set][j] = *(const bf16x8*)(st + B_OFF + boffs[j] + pos);
    if constexpr (ALO) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
        if (!RAG || i < na) alf[set][i] = *(const bf16x8*)(st + L_OFF + aoffs[i] + pos);
    }
  };

  // acc[i][j]: token block i x weight block j; lane holds token row lr and
  // output columns 8*q + 4*half + r (r = 0..3) at acc[i][j][4*q + r].
  f32x16 acc[MT][NTW];
  auto mma = [&](int set, auto rag) {
    constexpr bool RAG = decltype(rag)::value;
#pragma unroll
    for (int i = 0; i < MT; ++i)
      if (!RAG || i < na) {
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[set][j], af[set][i], acc[i][j], 0, 0, 0);
      }
    if constexpr (ALO) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
        if (!RAG || i < na) {
#pragma unroll
          for (int j = 0; j < NTW; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[set][j], alf[set][i], acc[i][j], 0, 0, 0);
        }
    }
  };

  int e, m0, mcount, n0;
  decode(xcd * chunk + jt, e, m0, mcount, n0);
  set_ptrs(e, m0, mcount, n0);
  // Every ring step issues exactly LPS loads per wave (part 1 of stage
  // kt+RING-2, then part 0 of stage kt+RING-1; past the last stage the copies
  // land in slots nobody reads), so at the mid-step wait of step kt only the
  // copies of stages kt+2 .. kt+RING-2 may still fly: vmcnt <= (RING-3)*LPS
  // means stage kt+1 has landed.
  issue_prologue();

  while (true) {
    vm_wait_n<0>();  // this tile's first stages (and the last tile's stores)
    wg_barrier();
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    auto kloop = [&](auto rag) {
      constexpr bool RAG = decltype(rag)::value;
      read_frags(0, 0, 0, rag);
      for (int kt = 0; kt < nk; ++kt) {
        // fragments (kt, ks=0) are in set 0
        read_frags(kt, 1, 1, rag);
        issue_part(kt + RING - 2, 1);
        mma(0, rag);
        if constexpr (!RAG) {
          // issue the (kt, ks=1) fragment reads between the first MFMAs, then
          // the weight-row copies of stage kt+RING-2
#pragma unroll
          for (int q = 0; q < MT + NTW + (ALO ? MT : 0); ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
#pragma unroll
          for (int q = 0; q < BI; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // stage kt+1 has landed (only the stages issued after it may still fly)
        // and no wave still reads the slot of stage kt-1
        lgkm_wait0();
        vm_wait_n<(RING - 3) * LPS>();
        wg_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(kt + 1, 0, 0, rag);  // past the last stage: reads a dead slot, never used
        issue_part(kt + RING - 1, 0);
        mma(1, rag);
        if constexpr (!RAG) {
          // interleave: one MFMA, one fragment read of the next stage (so the
          // reads land long before the next iteration needs them), then one
          // MFMA, one token-row copy of stage kt+RING-1
#pragma unroll
          for (int q = 0; q < MT + NTW + (ALO ? MT : 0); ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
#pragma unroll
          for (int q = 0; q < LPS - BI; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    kloop(std::false_type{});
    // all copies (the dead ones too) have landed: the ring is free for the next tile
    vm_wait_n<0>();

    // ---- next tile: request its first stages before this tile's epilogue
    const int ce = e, cm0 = m0, cmcount = mcount, cn0 = n0;
    jt += per;
    const bool more = jt < chunk && xcd * chunk + jt < ntiles;
    if (more) {
      decode(xcd * chunk + jt, e, m0, mcount, n0);
      set_ptrs(e, m0, mcount, n0);
      issue_prologue();
    }

    // ---- epilogue of the tile just finished
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int r = wm0 + i * 32 + lr;
      if (r >= cmcount) continue;
      const int slot = cm0 + r;
      float g = 1.f;
      if constexpr (MODE == kEpiGate) g = gate[slot];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = cn0 + wn0 + j * 32 + 8 * q + 4 * half;
          float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
          float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
          if constexpr (MODE == kEpiLogit) {
            const float* bf = (const float*)bias;
            float* o = (float*)out + (size_t)slot * ldo;
            if (col + 0 < ldo) o[col + 0] = v0 + (bf ? bf[col + 0] : 0.f);
            if (col + 1 < ldo) o[col + 1] = v1 + (bf ? bf[col + 1] : 0.f);
            if (col + 2 < ldo) o[col + 2] = v2 + (bf ? bf[col + 2] : 0.f);
            if (col + 3 < ldo) o[col + 3] = v3 + (bf ? bf[col + 3] : 0.f);
            continue;
          }
          if (col >= Nout) continue;  // Nout % 4 == 0: a group is all in or all out
          if (bias != nullptr) {
            const uint2 bb = *(const uint2*)((const bf16*)bias + (size_t)ce * Nout + col);
            v0 += __builtin_bit_cast(float, bb.x << 16);
            v1 += __builtin_bit_cast(float, bb.x & 0xFFFF0000u);
            v2 += __builtin_bit_cast(float, bb.y << 16);
            v3 += __builtin_bit_cast(float, bb.y & 0xFFFF0000u);
          }
          const size_t o = (size_t)slot * Nout + col;
          if constexpr (G1) {
            const float h0 = gelu_as(v0), h1 = gelu_as(v1), h2 = gelu_as(v2), h3 = gelu_as(v3);
            const uint2 hi = make_uint2(pack_bf16x2(h0, h1), pack_bf16x2(h2, h3));
            *(uint2*)((bf16*)out + o) = hi;
            if constexpr (SPLIT) {
              const float r0 = h0 - __builtin_bit_cast(float, hi.x << 16);
              const float r1 = h1 - __builtin_bit_cast(float, hi.x & 0xFFFF0000u);
              const float r2 = h2 - __builtin_bit_cast(float, hi.y << 16);
              const float r3 = h3 - __builtin_bit_cast(float, hi.y & 0xFFFF0000u);
              *(uint2*)(out_lo + o) = make_uint2(pack_bf16x2(r0, r1), pack_bf16x2(r2, r3));
            }
          } else {
            *(f32x4*)((float*)out + o) = f32x4{v0 * g, v1 * g, v2 * g, v3 * g};
          }
        }
      }
    }
    if (!more) break;
  }
}

}  // namespace

}  // namespace moe
