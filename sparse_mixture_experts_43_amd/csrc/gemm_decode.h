// Weight-streaming expert GEMM for small per-expert batches (decode-shaped
// layers): LDS-DMA stream kernel and its split-K reduction.
#pragma once

#include "gemm_ring.h"

namespace moe {

namespace {

// ---------------------------------------------------------------- decode bf16, LDS-DMA stream
// Weight streaming for small per-expert batches (<= 64 slots), K % 128 == 0.
// A block (4 waves) owns 64 weight rows of one expert and a K range; weights
// and the expert's slot rows stream through a ring of LDS slots with
// global_load_lds_dwordx4, every wave instruction one contiguous 1 KB run
// (4 rows x 256 bytes), so HBM sees long sequential reads. Row r keeps its
// 16-byte chunk c at position c ^ (r & 15): the 16-row fragment reads are
// bank-conflict free. Each wave multiplies its 16 weight rows against the
// slot groups with v_mfma_f32_16x16x32_bf16. With split-K the blocks write
// fp32 partial sums and a reduce kernel applies bias and the epilogue.
// With packed weights (`packed` != 0, the piece layout of gemm_ring.h) a
// wave's weight copies are the stage's 1 KB pieces of its own 16 rows, which
// land piece by piece and are read with the ring kernel's fragment addressing:
// the same fragments, MFMAs and results.
constexpr int kDKC = 128;             // K per chunk (default)
constexpr int kDRowB = kDKC * 2;      // 256 bytes per row per chunk
constexpr int kDWRows = 64;           // weight rows per block

// Ring depth of the decode stream kernel: as deep as fits two workgroups per
// CU in LDS (80 KB each), at least 3 slots.
constexpr int decode_ring(int xg, bool xlo, int kc = kDKC) {
  const int slot = kDWRows * 2 * kc + 16 * xg * 2 * kc * (xlo ? 2 : 1);
  const int r = (80 * 1024) / slot;
  return r < 3 ? 3 : (r > 6 ? 6 : r);
}

// XG: slot groups of 16 an LDS slot holds (the expert's kept slots, <= 16*XG);
// RING: slots in the ring; KC: K per chunk (rows of 2*KC bytes).
template <bool G1, bool SPLIT, int XG, int RING_, int KC = kDKC>
struct DecodeGeom {
  static constexpr bool XLO = SPLIT && !G1;
  static constexpr int RING = RING_;
  static constexpr int ROWB = 2 * KC;
  static constexpr int CPR = KC / 8;        // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;      // rows per wave DMA instruction
  static constexpr int WLD = 16 / RPI;      // weight DMA instructions per wave per chunk
  static constexpr int XLD = 4 / RPI;       // slot-row DMA instructions per wave per 16-slot group
  static constexpr int W_OFF = 0;
  static constexpr int X_OFF = kDWRows * ROWB;
  static constexpr int L_OFF = X_OFF + 16 * XG * ROWB;
  static constexpr int SLOT = L_OFF + (XLO ? 16 * XG * ROWB : 0);
  static constexpr size_t LDS = (size_t)RING * SLOT;
  static_assert(CPR == 16 || CPR == 32, "128- or 256-wide K chunks");
};

// Persistent: workgroup b takes items b, b + grid, ... of the (expert, 64-row
// block, K share) list, skipping experts that received no slot (their weights
// are never read), and requests the next item's first chunks before the
// current item's epilogue, so no item pays the stream's start-up latency.
template <bool G1, bool SPLIT, int XG, int RING, int KC = kDKC>
__global__ __launch_bounds__(256) void decode_dma_kernel(
    const bf16* __restrict__ X, const bf16* __restrict__ X_lo, const int32_t* __restrict__ perm,
    int kpairs, const int32_t* __restrict__ off, const bf16* __restrict__ W,
    const bf16* __restrict__ bias, const float* __restrict__ gate, int K, int Nout, int nblk_n,
    int nsplit, void* __restrict__ out, bf16* __restrict__ out_lo, float* __restrict__ part,
    int S_cap, int cap, int n_experts, int packed) {
  using Geo = DecodeGeom<G1, SPLIT, XG, RING, KC>;
  constexpr bool XLO = Geo::XLO;
  constexpr int ROWB = Geo::ROWB, CPR = Geo::CPR, RPI = Geo::RPI, WLD = Geo::WLD, XLD = Geo::XLD;
  extern __shared__ __align__(16) unsigned char smem[];
  MOE_LDS unsigned char* lds = (MOE_LDS unsigned char*)smem;
  const int l = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n_items = n_experts * nblk_n * nsplit;
  const int nch_all = K / KC;
  const int per = (nch_all + nsplit - 1) / nsplit;

  // item i -> expert, rows, K share; false when the item holds no work
  int e = 0, n0 = 0, m0 = 0, mcount = 0, c0 = 0, nch = 0, ks = 0, ng = 1;
  auto decode_item = [&](int i) {
    ks = i % nsplit;
    const int rest = i / nsplit;
    e = rest / nblk_n;
    n0 = (rest - e * nblk_n) * kDWRows;
    expert_rows(off, e, S_cap, cap < 16 * XG ? cap : 16 * XG, m0, mcount);
    c0 = ks * per;
    nch = min(nch_all, c0 + per) - c0;
    ng = (mcount + 15) / 16;
    return mcount > 0 && nch > 0;
  };
  auto next_item = [&](int i) {
    for (; i < n_items; i += gridDim.x)
      if (decode_item(i)) return i;
    return n_items;
  };

  // DMA sources: wave-load i covers rows RPI*(4i + wv) .. +RPI; lane l fills
  // row +l/CPR, position l%CPR, which holds chunk (l%CPR) ^ (row & 15).
  const int rsub = l / CPR;
  const unsigned char* pw[WLD];
  const unsigned char* px[XG * XLD];
  const unsigned char* pxl[XLO ? XG * XLD : 1];
  auto set_ptrs = [&]() {
    const int kbeg = c0 * KC;
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      if (packed) {
        // packed weights: wave-load i of wave wv is the 1 KB piece of row
        // block wv (rows n0 + 16 wv ..), K chunk i of the stage
        const int rb = min((n0 >> 4) + wv, (Nout >> 4) - 1);
        pw[i] = (const unsigned char*)(W + (size_t)e * Nout * K) +
                ((size_t)rb * (K / 32) + (size_t)c0 * (KC / 32) + i) * 1024 + 16 * l;
      } else {
        const int r = RPI * (4 * i + wv) + rsub;
        const int c = (l % CPR) ^ (r & 15);
        const int n = min(n0 + r, Nout - 1);
        pw[i] = (const unsigned char*)(W + ((size_t)e * Nout + n) * K + kbeg) + 16 * c;
      }
    }
#pragma unroll
    for (int i = 0; i < XG * XLD; ++i) {
      const int r = RPI * (4 * i + wv) + rsub;
      const int c = (l % CPR) ^ (r & 15);
      const int slot = m0 + min(r, mcount - 1);
      const size_t row = G1 ? (size_t)(perm[slot] / kpairs) : (size_t)slot;
      px[i] = (const unsigned char*)(X + row * K + kbeg) + 16 * c;
      if constexpr (XLO) pxl[i] = (const unsigned char*)(X_lo + row * K + kbeg) + 16 * c;
    }
  };
  // chunk `chunk` of the item into ring slot slot_i % RING; NG groups of slot rows
  auto issue = [&](int slot_i, int chunk, auto ng_c) {
    constexpr int NG = decltype(ng_c)::value;
    MOE_LDS unsigned char* st = lds + (slot_i % RING) * Geo::SLOT;
    const int kb = chunk * ROWB;
    const size_t kw = (size_t)chunk * (packed ? KC * 32 : ROWB);  // weight bytes to the chunk
#pragma unroll
    for (int i = 0; i < WLD; ++i) dma16(pw[i] + kw, st + Geo::W_OFF + (4 * i + wv) * 1024);
#pragma unroll
    for (int i = 0; i < NG * XLD; ++i) {
      dma16(px[i] + kb, st + Geo::X_OFF + (4 * i + wv) * 1024);
      if constexpr (XLO) dma16(pxl[i] + kb, st + Geo::L_OFF + (4 * i + wv) * 1024);
    }
  };
  auto prologue = [&](auto ng_c) {
#pragma unroll
    for (int q = 0; q < RING - 1; ++q) issue(q, q < nch ? q : nch - 1, ng_c);
  };
  // the same with the group count known only at run time
  auto prologue_rt = [&]() {
    if (ng <= 1) {
      prologue(std::integral_constant<int, 1>{});
    } else if constexpr (XG >= 2) {
      if (ng == 2 || XG == 2) {
        prologue(std::integral_constant<int, 2>{});
      } else if constexpr (XG >= 4) {
        if (ng == 3) prologue(std::integral_constant<int, 3>{});
        else prologue(std::integral_constant<int, 4>{});
      }
    }
  };

  int cur_item = next_item(blockIdx.x);
  const int R = 16 * wv + (l & 15);  // weight row of this lane's fragment
  const int Rs = R & 15;
  const int S = l & 15;              // slot row within a group (group base is a multiple of 16)
  const int gq = l >> 4;

  // one item with NG slot groups: stream its chunks, then request the next
  // item's first chunks, then write this item's outputs
  auto run_item = [&](auto ng_c) -> int {
    constexpr int NG = decltype(ng_c)::value;
    constexpr int LPS = WLD + NG * XLD * (XLO ? 2 : 1);  // DMA instructions per wave per chunk
    f32x4 acc[NG];
#pragma unroll
    for (int sg = 0; sg < NG; ++sg) acc[sg] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nch; ++c) {
      vm_wait_n<(RING - 2) * LPS>();
      wg_barrier();
      issue(c + RING - 1, c + RING - 1 < nch ? c + RING - 1 : nch - 1, ng_c);
      const unsigned char* st = smem + (c % RING) * Geo::SLOT;
#pragma unroll
      for (int kq = 0; kq < KC / 32; ++kq) {
        const int ch = 4 * kq + (l >> 4);
        // packed: piece 4 kq + wv, this lane's row l & 15 and 16-byte chunk
        // l >> 4 at the copy's word piece_slot(l & 15, l >> 4)
        const int wo = packed ? (4 * kq + wv) * 1024 + 16 * piece_slot(l & 15, l >> 4)
                              : R * ROWB + 16 * (ch ^ Rs);
        const bf16x8 wf = *(const bf16x8*)(st + Geo::W_OFF + wo);
#pragma unroll
        for (int sg = 0; sg < NG; ++sg) {
          const int xo = (16 * sg + S) * ROWB + 16 * (ch ^ S);
          const bf16x8 xf = *(const bf16x8*)(st + Geo::X_OFF + xo);
          acc[sg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf, acc[sg], 0, 0, 0);
          if constexpr (XLO) {
            const bf16x8 xl = *(const bf16x8*)(st + Geo::L_OFF + xo);
            acc[sg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xl, acc[sg], 0, 0, 0);
          }
        }
      }
    }
    vm_wait_n<0>();  // the dead copies too: the ring is free
    wg_barrier();    // no wave still reads a slot the next item's copies overwrite
    const int ce = e, cn0 = n0, cm0 = m0, cmcount = mcount, cks = ks;
    const int nxt = next_item(cur_item + gridDim.x);
    if (nxt < n_items) {
      set_ptrs();
      prologue_rt();
    }
    // D[row][slot]: lane holds slot column l%16 of each group, rows 4*(l/16) + i.
    float* pp = nsplit > 1 ? part : nullptr;
#pragma unroll
    for (int sg = 0; sg < NG; ++sg) {
      const int sl = 16 * sg + (l & 15);
      if (sl >= cmcount) continue;
      const int slot = cm0 + sl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = cn0 + 16 * wv + 4 * gq + i;
        if (n >= Nout) continue;
        if (pp != nullptr) {
          pp[((size_t)cks * S_cap + slot) * Nout + n] = acc[sg][i];
          continue;
        }
        const float v = acc[sg][i] + (bias != nullptr ? (float)bias[(size_t)ce * Nout + n] : 0.f);
        const size_t o = (size_t)slot * Nout + n;
        if constexpr (G1) {
          const float h = gelu_as(v);
          const bf16 hi = (bf16)h;
          ((bf16*)out)[o] = hi;
          if constexpr (SPLIT) out_lo[o] = (bf16)(h - (float)hi);
        } else {
          ((float*)out)[o] = v * gate[slot];
        }
      }
    }
    return nxt;
  };

  if (cur_item >= n_items) return;
  set_ptrs();
  prologue_rt();
  while (cur_item < n_items) {
    vm_wait_n<0>();  // this item's first chunks (and the last item's stores)
    wg_barrier();
    int nxt;
    if (ng <= 1) {
      nxt = run_item(std::integral_constant<int, 1>{});
    } else if constexpr (XG >= 2) {
      if (ng == 2 || XG == 2) {
        nxt = run_item(std::integral_constant<int, 2>{});
      } else if constexpr (XG >= 4) {
        if (ng == 3) nxt = run_item(std::integral_constant<int, 3>{});
        else nxt = run_item(std::integral_constant<int, 4>{});
      }
    }
    cur_item = nxt;
  }
}

// Split-K reduce: fixed-order sum of the partials, bias and epilogue. One
// block per (expert, 64-row block), threads over (slot, row).
template <bool G1, bool SPLIT>
__global__ __launch_bounds__(256) void decode_reduce_kernel(
    const float* __restrict__ part, int nsplit, int S_cap, int cap, const int32_t* __restrict__ off,
    const bf16* __restrict__ bias, const float* __restrict__ gate, int Nout, int nblk_n,
    void* __restrict__ out, bf16* __restrict__ out_lo) {
  const int e = blockIdx.x / nblk_n;
  const int nb = blockIdx.x - e * nblk_n;
  int m0, mcount;
  expert_rows(off, e, S_cap, cap, m0, mcount);
  const int n0 = nb * kDWRows;
  for (int i = threadIdx.x; i < mcount * kDWRows; i += 256) {
    const int sl = i / kDWRows, n = n0 + i % kDWRows;
    if (n >= Nout) continue;
    const int slot = m0 + sl;
    float v = 0.f;
    for (int q = 0; q < nsplit; ++q) v += part[((size_t)q * S_cap + slot) * Nout + n];
    v += bias != nullptr ? (float)bias[(size_t)e * Nout + n] : 0.f;
    const size_t o = (size_t)slot * Nout + n;
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

}  // namespace

}  // namespace moe
