// Grouped / plain bf16 GEMM on an LDS-DMA ring, shared by the expert FFN and
// the wide router. gfx950: global_load_lds_dwordx4, v_mfma_f32_16x16x32_bf16.
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
// exact erf form of GELU is what is computed (not the tanh form). The 1/2 is
// folded into the coefficients (a_i / 2, exact) and x = |z| / sqrt 2 into p and
// the exponent (exp(-x^2) = 2^(-z^2 log2(e) / 2)): 11 fp32 operations, one
// reciprocal and one exp2 per value.
__device__ __forceinline__ float gelu_as(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752f, az, 1.0f));
  const float half_poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f),
                                 0.5f * 1.421413741f),
                       0.5f * -0.284496736f),
               0.5f * 0.254829592f);
  const float e = __builtin_amdgcn_exp2f((z * z) * (-0.5f * 1.44269504088896341f));
  // max(z, 0) as a single v_max_f32 (fmaxf adds a canonicalising max of z
  // with itself first, as z comes from a matrix-core result)
  float relu;
  asm("v_max_f32 %0, 0, %1" : "=v"(relu) : "v"(z));
  return fmaf(-az, half_poly * e, relu);
}

namespace {

// ---------------------------------------------------------------- tiled bf16, LDS-DMA ring
// Packed weights (`packed` != 0, written by moe_pack_weights): expert e's
// matrix [Nout, K] is stored as pieces of 16 rows x 32 K, piece (row block rb,
// K chunk kc) at ((e * Nout/16 + rb) * K/32 + kc) * 1024 bytes, its 16-byte
// word w holding row rb*16 + piece_row(w), chunk piece_chunk(w): exactly the
// LDS image of one weight copy below, so a copy reads 1 KB contiguous instead
// of 64 bytes from each of 16 rows (the same tile contents and results).
//
// Fast path for K % 32 == 0. Tiles stream into a RING-slot LDS ring with
// global_load_lds_dwordx4 (each lane's 16 bytes land at base + 16 * lane, so a
// wave instruction fills the 1 KB of 16 rows x 32 K); no VGPR staging and no
// ds_write. Within such a 1 KB piece, the 16-byte chunk c (K 8c .. 8c+7) of
// row r sits in slot piece_slot(r, c) (below), so that the b128 fragment
// reads (lane l: row l & 15, chunk l >> 4) of any 16 lanes that share two of
// their lane-index bits, and of any 8 lanes that share three, fall on 16
// distinct groups of 4 banks. (Row-major 64-byte rows with the chunks
// XOR-swizzled by (r >> 2) & 3 kept only the 16 consecutive lanes on distinct
// banks; rocprofv3 counted 4 bank-conflict cycles per fragment read.) Stage
// kt+RING-1 is requested while stage
// kt is multiplied; one workgroup barrier per stage, taken mid-stage. A
// stage's fragment reads are spread over both halves of the steps around that
// barrier: its first half of token blocks and its weight blocks during the
// previous step's second half of MFMAs (after the barrier that makes the stage
// visible), its second half of token blocks during its own first half of MFMAs
// (Mixtral-shaped first GEMM -3% against reading them all in one half).
//
// Persistent: the grid holds one wave of resident workgroups; workgroup b runs
// on XCD b % 8 and walks the tiles of that XCD's contiguous share of the tile
// list, so the 8 L2s each see their own band of weights and token rows. The
// next tile's first RING-1 stages are requested before the current tile's
// epilogue, so their latency hides behind it.
//
// MFMA: v_mfma_f32_16x16x32_bf16, one per 16x16 block and stage (it holds
// the matrix cores at a higher clock under the power limit than the 32x32x16
// form with live data). The weight fragment is the A operand and the token
// fragment the B operand, so each lane's accumulator holds one token row and 4
// consecutive output columns per block: the epilogue writes 8-byte (bf16) or
// 16-byte (fp32) vectors.
constexpr int kRK = 32;         // K per ring stage
constexpr int kRing = 4;        // default ring slots
constexpr int kRowB = kRK * 2;  // bytes per tile row per stage

// Slot (16-byte word, 0..63) of row r (0..15), K chunk c (0..3) in a 1 KB
// piece of 16 rows x 32 K, and its inverse: slot = 16 h + 4 g + (c ^ h) with
// h = bits 1-2 of r and g = bit 0 of r plus bit 3 of r times 2.
__host__ __device__ __forceinline__ int piece_slot(int r, int c) {
  const int h = (r >> 1) & 3;
  const int g = (r & 1) | ((r >> 3) << 1);
  return 16 * h + 4 * g + (c ^ h);
}
__host__ __device__ __forceinline__ int piece_row(int s) {
  const int h = s >> 4, g = (s >> 2) & 3;
  return (g & 1) | (h << 1) | ((g >> 1) << 3);
}
__host__ __device__ __forceinline__ int piece_chunk(int s) { return (s & 3) ^ (s >> 4); }

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
// (The device queries are cached per calling thread: they cost microseconds,
// which a small layer's launch sequence would otherwise expose.)
inline int ring_grid(const void* kernel, int threads, size_t lds, int max_tiles) {
  struct Entry {
    const void* kernel;
    int threads, dev;
    size_t lds;
    int resident;
  };
  thread_local Entry cache[32];
  thread_local int n_cache = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int resident = 0;
  for (int i = 0; i < n_cache; ++i)
    if (cache[i].kernel == kernel && cache[i].threads == threads && cache[i].lds == lds &&
        cache[i].dev == dev)
      resident = cache[i].resident;
  if (resident == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, lds) != hipSuccess ||
        occ < 1)
      occ = 1;
    (void)hipGetLastError();
    resident = cus * occ;
    if (n_cache < 32) cache[n_cache++] = Entry{kernel, threads, dev, lds, resident};
  }
  long long g = resident;
  const long long mt = max_tiles > 0 ? max_tiles : 1;
  if (g > mt) g = mt;
  return (int)((g + 7) / 8 * 8);
}

// Work split of a persistent launch. XCD x (workgroups b with b % 8 == x)
// owns the tiles [x*chunk, x*chunk + cx) of the list; its `per` workgroups
// take them in whole rounds (workgroup j: tiles j, j+per, ...), and when a
// last partial round of L < per tiles remains and split partials are enabled,
// its L*nk stage units are cut into `per` equal contiguous ranges (one per
// workgroup, each touching at most two tiles), whose fp32 partial tiles
// ring_reduce_kernel sums in a fixed order: every tile still costs at most
// one round plus one share of the tail.
struct RingSplit {
  int chunk, cx, per, rounds, tail;
  __device__ __forceinline__ RingSplit(int ntiles, int xcd, int grid, bool split_tail) {
    per = grid >> 3;
    chunk = (ntiles + 7) >> 3;
    cx = ntiles - xcd * chunk;
    cx = cx < 0 ? 0 : (cx > chunk ? chunk : cx);
    rounds = cx / per;
    tail = cx - rounds * per;
    // split only a short tail: a tail of more than half a round costs about a
    // round anyway once its partials are written and reduced
    if (tail > 0 && (!split_tail || 2 * tail > per)) {
      rounds += 1;  // whole tiles only: the last round is partly idle
      tail = 0;
    }
  }
  // first stage unit of workgroup j's share of the split tail (32-bit math:
  // j <= per <= 128, tail < per and nk <= 2048 keep the product below 2^25)
  __device__ __forceinline__ int lo(int j, int nk) const {
    return (int)((unsigned)(j * tail * nk) / (unsigned)per);
  }
};

// Direct rows (second expert GEMM): a slot whose token kept no other pick
// holds the token's whole output, so its row goes straight to y[t] (fp32, or
// bf16 when ybf16) as the combine would write it, 0 + gate * (acc + b2)
// rounded once, instead of to the slot output.
__device__ __forceinline__ void store_direct(void* __restrict__ y, int ybf16, int t, int Nout,
                                             int col, float w0, float w1, float w2, float w3) {
#pragma clang fp contract(off)
  const float a0 = 0.f + w0, a1 = 0.f + w1, a2 = 0.f + w2, a3 = 0.f + w3;
  const size_t o = (size_t)t * Nout + col;
  if (ybf16) {
    *(uint2*)((bf16*)y + o) = make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3));
  } else {
    *(f32x4*)((float*)y + o) = f32x4{a0, a1, a2, a3};
  }
}

// Epilogue of one tile from the accumulators. Lane l holds, for token block i
// and weight block j, token row (2i + wr)*16 + (l & 15) of the tile and the 4
// consecutive output columns wn0 + 16j + 4*(l >> 4) + r (r = 0..3). The
// tile's gates and direct-row tokens (second expert GEMM) and biases are read
// from LDS, where the kernel staged them (sh_gate[row], sh_dst[row], -1 for a
// slot output row; sh_bias[column - n0]); the logits mode reads its fp32 bias
// from global memory.
template <int BM, int BN, int WM, int WN, int MODE, bool SPLIT>
__device__ __forceinline__ void ring_epilogue(const f32x4 (&acc)[WM / 16][WN / 16],
                                              const float* sh_gate, const int* sh_dst,
                                              const float* sh_bias, int m0, int mcount, int n0,
                                              int wr, int wn0, int l,
                                              const void* __restrict__ bias, int Nout,
                                              void* __restrict__ out, bf16* __restrict__ out_lo,
                                              int ldo, void* __restrict__ ydir, int ybf16) {
#pragma clang fp contract(off)
  constexpr bool G1 = MODE == kEpiGelu;
  constexpr int MT = WM / 16, NTW = WN / 16;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int r = (2 * i + wr) * 16 + (l & 15);  // token blocks alternate between the wave rows
    if (r >= mcount) continue;
    const int slot = m0 + r;
    float g = 1.f;
    int dst = -1;
    if constexpr (MODE == kEpiGate) {
      g = sh_gate[r];
      dst = sh_dst[r];
    }
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int col = n0 + wn0 + j * 16 + 4 * (l >> 4);
      float v0 = acc[i][j][0], v1 = acc[i][j][1], v2 = acc[i][j][2], v3 = acc[i][j][3];
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
        const f32x4 bb = *(const f32x4*)(sh_bias + (col - n0));
        v0 += bb[0];
        v1 += bb[1];
        v2 += bb[2];
        v3 += bb[3];
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
      } else if (dst >= 0) {
        store_direct(ydir, ybf16, dst, Nout, col, v0 * g, v1 * g, v2 * g, v3 * g);
      } else {
        *(f32x4*)((float*)out + o) = f32x4{v0 * g, v1 * g, v2 * g, v3 * g};
      }
    }
  }
}

template <int MODE, int BM, int BN>
__device__ __forceinline__ void ring_decode_tile(int tile, const int4* __restrict__ tiles,
                                                 int M_total, int Nout, int& e, int& m0,
                                                 int& mcount, int& n0) {
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
}

// part: fp32 partial tiles of the split tail (2 per workgroup, BM*BN each) or
// NULL (whole tiles only).
// EARLY: every ring step issues all copies of stage kt+RING-1 at its start and
// waits for stage kt+1 with the two stages after it in flight; otherwise a
// stage's copies go out over two steps (below). The two-step form measured
// better on the 256x256 prefill tiles, the early form on the 128x128 tiles of
// capacity-limited layers, where it also lets a 3-slot ring (the split hidden
// layer's extra token rows) keep one stage in flight with two workgroups per CU.
template <int BM, int BN, int WM, int WN, int MODE, bool SPLIT, int RING, bool EARLY = false>
// Two waves per SIMD: at most 256 VGPRs (two 128x128 workgroups per CU, or
// one 256x256 workgroup of eight waves).
__global__ __launch_bounds__((BM / WM) * (BN / WN) * kWave)
__attribute__((amdgpu_waves_per_eu(2))) void gemm_ring_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ A_lo, const int32_t* __restrict__ perm,
    int kpairs, const bf16* __restrict__ W, const void* __restrict__ bias,
    const float* __restrict__ gate, const int4* __restrict__ tiles,
    const int32_t* __restrict__ ntiles_p, int K, int Nout, void* __restrict__ out,
    bf16* __restrict__ out_lo, int M_total, int ldo, float* __restrict__ part,
    int* __restrict__ wq, int packed, const int32_t* __restrict__ dmap, void* __restrict__ ydir,
    int ybf16) {
  constexpr bool G1 = MODE == kEpiGelu;
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int NTH = NW * kWave;
  constexpr int MT = WM / 16, NTW = WN / 16;  // 16-row token / weight blocks per wave
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
  static_assert(EARLY || RING >= 4, "the two-step copies need a stage of slack");
  static_assert(BM / WM == 2, "two wave rows (token blocks alternate between them)");
  static_assert(MT % 2 == 0, "token blocks are skipped in pairs");
  static_assert(NTH >= BM && NTH >= BN, "one thread per staged gate / bias");

  extern __shared__ __align__(16) unsigned char smem[];

  // ---- this workgroup's items: whole tiles, then at most two tail segments
  int ntiles;
  if constexpr (MODE == kEpiLogit) {
    ntiles = ((M_total + BM - 1) / BM) * ((Nout + BN - 1) / BN);
  } else {
    ntiles = *ntiles_p;
  }
  const int nk = K / kRK;
  const int xcd = blockIdx.x & 7;
  const int jw = blockIdx.x >> 3;
  // wq (not null): a work queue per XCD (8 counters, zero at launch); each
  // workgroup claims its next tile of the XCD's share with one integer atomic,
  // so the share's tiles finish roughly in list order and co-scheduled tiles
  // stay close in K (their shared rows meet in L2). No split tail then.
  const bool dyn = wq != nullptr;
  const RingSplit sp(ntiles, xcd, gridDim.x, part != nullptr && !dyn);
  int n_whole = sp.rounds;  // whole tiles jw + r*per that exist
  if (n_whole > 0 && jw + (n_whole - 1) * sp.per >= sp.cx) n_whole -= 1;
  int t_lo = 0, t_hi = 0;
  int seg0 = 0, n_seg = 0;
  if (sp.tail > 0) {
    t_lo = sp.lo(jw, nk);
    t_hi = sp.lo(jw + 1, nk);
    if (t_hi > t_lo) {
      seg0 = t_lo / nk;
      n_seg = (t_hi - 1) / nk - seg0 + 1;
    }
  }
  const int n_items = n_whole + n_seg;
  if (n_items == 0 && !dyn) return;
  const int base_tile = xcd * sp.chunk;
  __shared__ int sh_claim;
  __shared__ __align__(16) float sh_gate[BM];  // the finished tile's gates (second expert GEMM)
  __shared__ __align__(16) float sh_bias[BN];  // and biases by column, for its epilogue
  // and its direct-row tokens (dmap: token of a slot whose token kept no other
  // pick, else -1; null: none)
  __shared__ int sh_dst[MODE == kEpiGate ? BM : 1];
  // no copy is in flight where this is called (the barriers wait for them)
  auto claim = [&]() -> int {
    __syncthreads();
    if (threadIdx.x == 0) sh_claim = atomicAdd(wq + xcd, 1);
    __syncthreads();
    const int c = sh_claim;
    return c < sp.cx ? c : -1;
  };
  // item it -> tile, stage range [kb, ke), partial slot (-1: whole tile)
  auto item = [&](int it, int& tile, int& kb, int& ke, int& ps) {
    if (it < n_whole) {
      tile = base_tile + jw + it * sp.per;
      kb = 0; ke = nk; ps = -1;
    } else {
      const int q = it - n_whole;
      const int tau = seg0 + q;
      tile = base_tile + sp.rounds * sp.per + tau;
      const int u0 = tau * nk;
      kb = (t_lo > u0 ? t_lo : u0) - u0;
      ke = (t_hi < u0 + nk ? t_hi : u0 + nk) - u0;
      ps = (int)blockIdx.x * 2 + q;
    }
  };

  const int l = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wr = wv / (BN / WN);  // wave row: token blocks wr, wr+2, wr+4, ... of the tile
  const int wn0 = (wv % (BN / WN)) * WN;

  // DMA source pointers: wave-load i covers tile rows (i*NW + wv)*16 .. +16;
  // lane l fills slot l of the piece: row piece_row(l), chunk piece_chunk(l).
  const int csw = piece_chunk(l) * 16;  // byte offset of the chunk
  const unsigned char* pa[AI];
  const unsigned char* pl[ALO ? AI : 1];
  const unsigned char* pb[BI];
  auto set_ptrs = [&](int e, int m0, int mcount, int n0) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int r = (i * NW + wv) * 16 + piece_row(l);
      const int rr = r < mcount ? r : mcount - 1;
      const int slot = m0 + rr;
      const size_t row = G1 ? (size_t)(perm[slot] / kpairs) : (size_t)slot;
      pa[i] = (const unsigned char*)(A + row * K) + csw;
      if constexpr (ALO) pl[i] = (const unsigned char*)(A_lo + row * K) + csw;
    }
    const bf16* We = W + (size_t)e * Nout * K;
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      if (packed) {
        // packed weights: the 16 rows x 32 K of stage kt are one contiguous
        // 1 KB piece in this copy's LDS order (row blocks past Nout repeat the
        // last one; Nout % 16 == 0)
        const int rb = (n0 + (i * NW + wv) * 16) >> 4;
        const int nrb = Nout >> 4;
        pb[i] = (const unsigned char*)We + (size_t)(rb < nrb ? rb : nrb - 1) * (K / kRK) * 1024 +
                16 * l;
      } else {
        const int r = (i * NW + wv) * 16 + piece_row(l);
        const int n = n0 + r < Nout ? n0 + r : Nout - 1;
        pb[i] = (const unsigned char*)(We + (size_t)n * K) + csw;
      }
    }
  };
  const int wstep = packed ? 1024 : kRowB;  // weight bytes between stages of one row block
  MOE_LDS unsigned char* lds = (MOE_LDS unsigned char*)smem;
  int kb = 0, nks = 0;  // stage range of the current item: [kb, kb + nks)
  // A stage's copies go out in two parts: part 0 (token rows, and their
  // residual rows) right after the mid-stage barrier, part 1 (weight rows) in
  // the first half of the next ring step, so the vector-memory issue is spread
  // over the whole step instead of bursting.
  auto issue_part = [&](int kt, int prt) {
    const int src_kt = kb + (kt < nks ? kt : nks - 1);  // past the last stage: a dead copy
    MOE_LDS unsigned char* st = lds + (kt % RING) * STAGE;
    const int kbyte = src_kt * kRowB;
    if (prt == 0) {
#pragma unroll
      for (int i = 0; i < AI; ++i)
        dma16(pa[i] + kbyte, st + A_OFF + (i * NW + wv) * 1024);
      if constexpr (ALO) {
#pragma unroll
        for (int i = 0; i < AI; ++i)
          dma16(pl[i] + kbyte, st + L_OFF + (i * NW + wv) * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < BI; ++i)
        dma16(pb[i] + (size_t)src_kt * wstep, st + B_OFF + (i * NW + wv) * 1024);
    }
  };
  // prologue of an item: stages 0 .. RING-3 whole, stage RING-2 part 0 (EARLY:
  // stage RING-2 whole as well)
  auto issue_prologue = [&]() {
#pragma unroll
    for (int q = 0; q < RING - 2; ++q) {
      issue_part(q, 0);
      issue_part(q, 1);
    }
    issue_part(RING - 2, 0);
    if constexpr (EARLY) issue_part(RING - 2, 1);
  };

  // Fragment reads (v_mfma_f32_16x16x32_bf16 operands): lane l reads row
  // 16*blk + (l & 15), 16-byte chunk l >> 4 (K 8*(l>>4) .. +8), which sits in
  // slot piece_slot(l & 15, l >> 4) of the block's 1 KB piece.
  const int pos = piece_slot(l & 15, l >> 4) * 16;
  int aoffs[MT], boffs[NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i) aoffs[i] = (2 * i + wr) * 16 * kRowB + pos;
#pragma unroll
  for (int j = 0; j < NTW; ++j) boffs[j] = (wn0 + j * 16) * kRowB + pos;

  bf16x8 af[2][MT], bfr[2][NTW], alf[ALO ? 2 : 1][ALO ? MT : 1];
  // NA: token blocks of this wave that hold rows of the tile (a partly filled
  // tile skips the fragment reads and MFMAs of the empty ones)
  // lo: token blocks [0, NA/2) and the weight blocks; hi: blocks [NA/2, NA)
  auto read_frags_lo = [&](int kt, int set, auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    const unsigned char* st = smem + (kt % RING) * STAGE;
#pragma unroll
    for (int i = 0; i < NA / 2; ++i) af[set][i] = *(const bf16x8*)(st + A_OFF + aoffs[i]);
#pragma unroll
    for (int j = 0; j < NTW; ++j) bfr[set][j] = *(const bf16x8*)(st + B_OFF + boffs[j]);
    if constexpr (ALO) {
#pragma unroll
      for (int i = 0; i < NA / 2; ++i) alf[set][i] = *(const bf16x8*)(st + L_OFF + aoffs[i]);
    }
  };
  auto read_frags_hi = [&](int kt, int set, auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    const unsigned char* st = smem + (kt % RING) * STAGE;
#pragma unroll
    for (int i = NA / 2; i < NA; ++i) af[set][i] = *(const bf16x8*)(st + A_OFF + aoffs[i]);
    if constexpr (ALO) {
#pragma unroll
      for (int i = NA / 2; i < NA; ++i) alf[set][i] = *(const bf16x8*)(st + L_OFF + aoffs[i]);
    }
  };

  // acc[i][j]: token block i x weight block j (weight fragment = A operand,
  // token fragment = B operand of the 16x16x32 MFMA).
  f32x4 acc[MT][NTW];
  auto mma = [&](int set, auto lo_c, auto hi_c) {
    constexpr int LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
#pragma unroll
    for (int i = LO; i < HI; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[set][j], af[set][i], acc[i][j], 0, 0, 0);
    if constexpr (ALO) {
#pragma unroll
      for (int i = LO; i < HI; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[set][j], alf[set][i], acc[i][j], 0, 0, 0);
    }
  };

  // the ring steps of one item, for NA active token blocks: step kt multiplies
  // stage kt (fragments in register set kt & 1, unrolled by two so that the
  // set is static) in two halves of token blocks; the barrier between them
  // makes stage kt+1 visible, and its fragments are read during the second half
  auto kloop = [&](auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    constexpr int H = NA / 2;
    constexpr int NRL = H + NTW + (ALO ? H : 0);  // reads of the next stage (second half)
    constexpr int NRH = (NA - H) * (ALO ? 2 : 1);  // reads of this stage's blocks H.. (first half)
    constexpr int M1 = H * NTW * (ALO ? 2 : 1);    // MFMAs per half
    using lo0 = std::integral_constant<int, 0>;
    using mid = std::integral_constant<int, H>;
    using hi1 = std::integral_constant<int, NA>;
    // copies issued in the first half of a step: part 1 of stage kt+RING-2, or
    // (EARLY) all of stage kt+RING-1
    constexpr int C1 = EARLY ? LPS : BI;
    auto step = [&](int kt, auto set_c) {
      constexpr int SET = decltype(set_c)::value;
      if constexpr (EARLY) {
        // the slot of stage kt-1: every wave finished reading it before the
        // barrier of step kt-1
        issue_part(kt + RING - 1, 0);
        issue_part(kt + RING - 1, 1);
      } else {
        issue_part(kt + RING - 2, 1);
      }
      read_frags_hi(kt, SET, na_c);
      mma(SET, lo0{}, mid{});
      if constexpr (M1 > 0) {
        // those copies and this stage's remaining fragment reads spread over
        // the first half
        constexpr int G1N = M1 / (NRH + C1) > 0 ? M1 / (NRH + C1) : 1;
#pragma unroll
        for (int q = 0; q < NRH; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, G1N, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < C1; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, G1N, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // stage kt+1 has landed (only the stages issued after it may still fly),
      // this wave's reads of stage kt are done, and no wave still reads the
      // slot of stage kt-1
      vm_wait_n<(EARLY ? RING - 2 : RING - 3) * LPS>();
      lgkm_wait0();
      wg_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_frags_lo(kt + 1, SET ^ 1, na_c);  // past the last stage: reads a dead slot, never used
      if constexpr (!EARLY) issue_part(kt + RING - 1, 0);
      mma(SET, mid{}, hi1{});
      if constexpr (M1 > 0) {
        // one MFMA, one fragment read of the next stage, ...; then the
        // token-row copies of stage kt+RING-1
#pragma unroll
        for (int q = 0; q < NRL; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < LPS - C1; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    read_frags_lo(0, 0, na_c);
    int kt = 0;
    for (; kt + 1 < nks; kt += 2) {
      step(kt, std::integral_constant<int, 0>{});
      step(kt + 1, std::integral_constant<int, 1>{});
    }
    if (kt < nks) step(kt, std::integral_constant<int, 0>{});
  };

  int tile, ke, ps, e, m0, mcount, n0;
  if (dyn) {
    const int c = claim();
    if (c < 0) return;
    tile = base_tile + c;
    kb = 0;
    ke = nk;
    ps = -1;
  } else {
    item(0, tile, kb, ke, ps);
  }
  nks = ke - kb;
  ring_decode_tile<MODE, BM, BN>(tile, tiles, M_total, Nout, e, m0, mcount, n0);
  set_ptrs(e, m0, mcount, n0);
  // Every ring step issues exactly LPS loads per wave (part 1 of stage
  // kt+RING-2, then part 0 of stage kt+RING-1; EARLY: stage kt+RING-1 whole;
  // past the last stage the copies land in slots nobody reads), so at the
  // mid-step wait of step kt only the copies of stages kt+2 .. kt+RING-2 (EARLY:
  // kt+RING-1) may still fly: vmcnt <= (RING-3)*LPS (EARLY: (RING-2)*LPS) means
  // stage kt+1 has landed.
  issue_prologue();

  for (int it = 0;;) {
    vm_wait_n<0>();  // this item's first stages (and the last item's stores)
    wg_barrier();
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      // token blocks of this wave row with rows below mcount, rounded up to
      // an even count
      const int nb = (mcount + 15) / 16;
      int na = (nb - wr + 1) / 2;
      na = (na + 1) & ~1;
      na = __builtin_amdgcn_readfirstlane(na < 0 ? 0 : (na > MT ? MT : na));
      if (na >= MT) {
        kloop(std::integral_constant<int, MT>{});
      } else if constexpr (MT == 8) {
        switch (na) {
          case 6: kloop(std::integral_constant<int, 6>{}); break;
          case 4: kloop(std::integral_constant<int, 4>{}); break;
          case 2: kloop(std::integral_constant<int, 2>{}); break;
          default: kloop(std::integral_constant<int, 0>{}); break;
        }
      } else if constexpr (MT == 4) {
        if (na == 2) kloop(std::integral_constant<int, 2>{});
        else kloop(std::integral_constant<int, 0>{});
      } else {
        kloop(std::integral_constant<int, MT>{});
      }
    }
    // all copies (the dead ones too) have landed: the ring is free
    vm_wait_n<0>();
    // This tile's gates and biases, one per thread, go to LDS after the wait
    // below: loaded now, before the next tile's copies go out (vmcnt retires
    // in issue order, so a load issued after them would make the epilogue's
    // stores wait for those copies), and held in one register each instead of
    // per-lane copies live across the K loop.
    float stg = 1.f, stb = 0.f;
    int sdst = -1;
    if constexpr (MODE != kEpiLogit) {
      const int tid = threadIdx.x;
      if (ps < 0) {
        if constexpr (MODE == kEpiGate) {
          if (tid < BM && tid < mcount) {
            stg = gate[m0 + tid];
            if (dmap != nullptr) sdst = dmap[m0 + tid];
          }
        }
        if (bias != nullptr && tid < BN && n0 + tid < Nout)
          stb = (float)((const bf16*)bias)[(size_t)e * Nout + n0 + tid];
      }
    }

    // ---- next item: request its first stages before this item's epilogue
    const int cm0 = m0, cmcount = mcount, cn0 = n0, cps = ps;
    bool more;
    if (dyn) {
      const int c = claim();
      more = c >= 0;
      if (more) {
        tile = base_tile + c;
        kb = 0;
        ke = nk;
        ps = -1;
      }
    } else {
      ++it;
      more = it < n_items;
      if (more) item(it, tile, kb, ke, ps);
    }
    // the gates and biases have landed before the next tile's copies go out
    // (with the work queue the claim's round trip covers most of their
    // latency); every wave finished reading the previous tile's values in its
    // epilogue, before this tile's K loop barriers
    vm_wait_n<0>();
    if constexpr (MODE != kEpiLogit) {
      if (threadIdx.x < BM) sh_gate[threadIdx.x] = stg;
      if constexpr (MODE == kEpiGate)
        if (threadIdx.x < BM) sh_dst[threadIdx.x] = sdst;
      if (threadIdx.x < BN) sh_bias[threadIdx.x] = stb;
      // the stores must have completed before the barrier: s_barrier alone
      // does not order them before another wave's reads (with two workgroups
      // per CU, a wave has read the previous tile's gates for 16 rows without
      // this wait)
      lgkm_wait0();
      wg_barrier();
    }
    if (more) {
      nks = ke - kb;
      ring_decode_tile<MODE, BM, BN>(tile, tiles, M_total, Nout, e, m0, mcount, n0);
      set_ptrs(e, m0, mcount, n0);
      issue_prologue();
    }

    if (cps < 0) {
      ring_epilogue<BM, BN, WM, WN, MODE, SPLIT>(acc, sh_gate, sh_dst, sh_bias, cm0, cmcount, cn0,
                                                 wr, wn0, l, bias, Nout, out, out_lo, ldo, ydir,
                                                 ybf16);
    } else {
      // raw partial accumulators, one float4 per lane and block, lane-major
      // so every store is one contiguous 1 KB
      f32x4* pp = (f32x4*)(part + (size_t)cps * (BM * BN)) + threadIdx.x;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) pp[(i * NTW + j) * NTH] = acc[i][j];
    }
    if (!more) break;
  }
}

// Sums the split-tail partials of each tail tile in workgroup order and
// applies the tile's epilogue. One thread per float4 group of a partial tile
// (4 consecutive output columns of one GEMM lane); the grid strides over
// (XCD, tail tile, group block) with tail tiles that do not exist skipped.
// `grid` is the GEMM launch's grid.
constexpr int kReduceThreads = 256;
template <int BM, int BN, int WM, int WN, int MODE, bool SPLIT>
__global__ __launch_bounds__(kReduceThreads) void ring_reduce_kernel(
    const float* __restrict__ part, int grid, const void* __restrict__ bias,
    const float* __restrict__ gate, const int4* __restrict__ tiles,
    const int32_t* __restrict__ ntiles_p, int K, int Nout, void* __restrict__ out,
    bf16* __restrict__ out_lo, const int32_t* __restrict__ dmap, void* __restrict__ ydir,
    int ybf16) {
#pragma clang fp contract(off)
  constexpr bool G1 = MODE == kEpiGelu;
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int NTH = NW * kWave;
  constexpr int NTW = WN / 16;
  constexpr int GROUPS = BM * BN / 4;               // float4 groups per tile
  constexpr int GB = GROUPS / kReduceThreads;       // group blocks per tile
  const int nk = K / kRK;
  const int ntiles = *ntiles_p;
  const int per = grid >> 3;
  const int nwork = 8 * per * GB;
  for (int w = blockIdx.x; w < nwork; w += gridDim.x) {
    const int xcd = w & 7;
    const int tau = (w >> 3) / GB;
    const int gb = (w >> 3) - tau * GB;
    const RingSplit sp(ntiles, xcd, grid, true);
    if (tau >= sp.tail) continue;
    const int tile = xcd * sp.chunk + sp.rounds * sp.per + tau;
    int e, m0, mcount, n0;
    ring_decode_tile<MODE, BM, BN>(tile, tiles, 0, Nout, e, m0, mcount, n0);
    // group index g = (i*NTW + j)*NTH + tid of the GEMM lane layout
    const int g = gb * kReduceThreads + threadIdx.x;
    const int tid = g % NTH;
    const int ij = g / NTH;
    const int j = ij % NTW, i = ij / NTW;
    const int wv = tid / kWave, lane = tid % kWave;
    const int row = (2 * i + wv / (BN / WN)) * 16 + (lane & 15);
    const int col = n0 + (wv % (BN / WN)) * WN + j * 16 + 4 * (lane >> 4);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    // workgroups whose share holds unit u: lo(j) <= u < lo(j+1), i.e. the
    // largest j with j*U < (u+1)*per (U = tail*nk units in the tail)
    const int U = sp.tail * nk;
    const int u0 = tau * nk, u1 = u0 + nk;
    const int j1 = (int)(((unsigned)(u0 + 1) * per + U - 1) / (unsigned)U) - 1;
    const int j2 = (int)(((unsigned)u1 * per + U - 1) / (unsigned)U) - 1;
    for (int jw = j1; jw <= j2; ++jw) {
      const int lo = sp.lo(jw, nk), hi = sp.lo(jw + 1, nk);
      if (hi <= u0 || lo >= u1 || hi <= lo) continue;
      const int sq = tau - lo / nk;
      const int b = jw * 8 + xcd;
      v += ((const f32x4*)(part + (size_t)(b * 2 + sq) * (BM * BN)))[g];
    }
    if (row >= mcount || col >= Nout) continue;
    const int slot = m0 + row;
    float v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
    if (bias != nullptr) {
      const uint2 bb = *(const uint2*)((const bf16*)bias + (size_t)e * Nout + col);
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
      const float gg = gate[slot];
      const int dst = dmap != nullptr ? dmap[slot] : -1;
      if (dst >= 0)
        store_direct(ydir, ybf16, dst, Nout, col, v0 * gg, v1 * gg, v2 * gg, v3 * gg);
      else
        *(f32x4*)((float*)out + o) = f32x4{v0 * gg, v1 * gg, v2 * gg, v3 * gg};
    }
  }
}

}  // namespace

}  // namespace moe
