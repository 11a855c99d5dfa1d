// Capacity-constrained dispatch: histogram, scans, stable bucketing by expert,
// per-expert capacity selection and the slot permutation / inverse map.
//
// Page "Mixture-of-Experts" (beta.fermi.ai wiki), steps 4-5 and the
// capacity-constrained dispatch of its pseudocode: each expert accepts at most
// C (token, expert) pairs; when more arrive, the lowest-scoring ones are
// dropped for that expert (worked example: at E2 the 0.667 request of x2 goes,
// at E3 the 0.286 request of x4). The score is the softmax probability,
// compared through the fp64 key log p = L - logsumexp(L); equal keys keep the
// lower token. Kept pairs are laid out expert by expert, tokens ascending.
//
// The serial append loop of the pseudocode becomes, with no atomics on global
// memory and a deterministic result:
//   hist    : per tile of pairs, each wave counts requests per expert (LDS)
//   scan    : per-expert totals, tile bases, request / kept offsets (1 block)
//   bucket  : each pair is written to its expert's list in token order, with
//             its order-preserving 64-bit key code next to it
//   select  : one block per expert; under capacity: copy; over capacity: an
//             8-pass radix select finds the C-th largest key code, then an
//             ordered block scan keeps the strictly larger codes and the
//             first equal ones in token order.
#include "moe_common.h"

namespace moe {

namespace {

constexpr int kScanThreads = 1024;

__device__ __forceinline__ unsigned long long lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Lanes of this wave whose `e` equals mine (only among `valid` lanes).
__device__ __forceinline__ unsigned long long match_peers(int e, bool valid) {
  unsigned long long peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 10; ++b) {  // expert ids < 1024
    const bool bit = (e >> b) & 1;
    const unsigned long long m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// Block-wide exclusive scan (blockDim.x multiple of 64, <= 1024). `tmp` holds
// 17 ints of LDS. Returns the exclusive prefix; *total gets the block sum.
__device__ int block_scan_excl(int v, int* tmp, int* total) {
  const int l = lane_id();
  const int wv = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (l >= o) x += y;
  }
  __syncthreads();  // tmp may still be read from a previous call
  if (l == kWave - 1) tmp[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int s = (l < nw) ? tmp[l] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(s, o, kWave);
      if (l >= o) s += y;
    }
    if (l < nw) tmp[l] = s;
  }
  __syncthreads();
  const int wbase = wv > 0 ? tmp[wv - 1] : 0;
  *total = tmp[nw - 1];
  return wbase + x - v;
}

// One wave walks one tile of pairs in order; for each pair it returns (via
// `emit`) the pair's rank among the tile's earlier pairs of the same expert.
// Expert ids outside [0, N) are skipped (such pairs are never bucketed; the
// bucket kernel marks them dropped) so that bad ids cannot index out of range.
template <typename Emit>
__device__ void walk_tile(const int32_t* __restrict__ idx, int P, int N, int tile, int* cnt,
                          Emit emit) {
  const int l = lane_id();
  const int p0 = tile * kDispatchTile;
  constexpr int kChunks = kDispatchTile / kWave;
  int ev[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = p0 + c * kWave + l;
    ev[c] = (p < P) ? idx[p] : 0;
  }
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = p0 + c * kWave + l;
    const int e = ev[c];
    const bool valid = p < P && (unsigned)e < (unsigned)N;
    const unsigned long long peers = match_peers(e, valid);
    const int before = __popcll(peers & lanemask_lt());
    int base = 0;
    if (valid) base = cnt[e];
    // all reads of cnt[] in this chunk happen before the leader's update
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      emit(p, e, base + before);
      if (before == 0) cnt[e] = base + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ------------------------------------------------------------ hist
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int P, int N,
                                                   int ntiles, int32_t* __restrict__ tilecnt) {
  extern __shared__ int hsm[];  // [4][N]
  const int wv = threadIdx.x / kWave;
  const int l = lane_id();
  const int tile = blockIdx.x * 4 + wv;
  int* cnt = hsm + wv * N;
  for (int e = l; e < N; e += kWave) cnt[e] = 0;
  __builtin_amdgcn_wave_barrier();
  if (tile >= ntiles) return;
  walk_tile(idx, P, N, tile, cnt, [](int, int, int) {});
  __builtin_amdgcn_wave_barrier();
  for (int e = l; e < N; e += kWave) tilecnt[(size_t)tile * N + e] = cnt[e];
}

// ------------------------------------------------------------ scan
__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const int32_t* __restrict__ tilecnt, int ntiles, int N, int P, int C,
    int32_t* __restrict__ tilebase, int32_t* __restrict__ req, int32_t* __restrict__ cnt,
    int32_t* __restrict__ reqoff, int32_t* __restrict__ off, int32_t* __restrict__ n_dropped) {
  __shared__ int tmp[17];
  __shared__ int carry[2];
  if (threadIdx.x == 0) carry[0] = carry[1] = 0;
  for (int e0 = 0; e0 < N; e0 += kScanThreads) {
    const int e = e0 + threadIdx.x;
    int r = 0;
    if (e < N) {
      for (int t = 0; t < ntiles; ++t) {
        const int c = tilecnt[(size_t)t * N + e];
        tilebase[(size_t)t * N + e] = r;
        r += c;
      }
    }
    const int kept = min(r, C);
    int tot_r, tot_k;
    const int xr = block_scan_excl(r, tmp, &tot_r);
    const int xk = block_scan_excl(kept, tmp, &tot_k);
    if (e < N) {
      req[e] = r;
      cnt[e] = kept;
      reqoff[e] = carry[0] + xr;
      off[e] = carry[1] + xk;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      carry[0] += tot_r;
      carry[1] += tot_k;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    reqoff[N] = carry[0];
    off[N] = carry[1];
    *n_dropped = P - carry[1];
  }
}

// ------------------------------------------------------------ bucket
__global__ __launch_bounds__(256) void bucket_kernel(
    const int32_t* __restrict__ idx, const double* __restrict__ key, int P, int N, int ntiles,
    const int32_t* __restrict__ tilebase, const int32_t* __restrict__ reqoff,
    int32_t* __restrict__ bucket, unsigned long long* __restrict__ codes,
    int32_t* __restrict__ inv) {
  extern __shared__ int bsm[];  // [4][N]
  const int wv = threadIdx.x / kWave;
  const int l = lane_id();
  const int tile = blockIdx.x * 4 + wv;
  int* cnt = bsm + wv * N;
  if (tile < ntiles)
    for (int e = l; e < N; e += kWave) cnt[e] = reqoff[e] + tilebase[(size_t)tile * N + e];
  __builtin_amdgcn_wave_barrier();
  if (tile >= ntiles) return;
  walk_tile(idx, P, N, tile, cnt, [&](int p, int, int pos) {
    bucket[pos] = p;
    codes[pos] = key_code(key[p]);
  });
  for (int c = 0; c < kDispatchTile / kWave; ++c) {
    const int p = tile * kDispatchTile + c * kWave + l;
    if (p < P && (unsigned)idx[p] >= (unsigned)N) inv[p] = -1;
  }
}

// ------------------------------------------------------------ select + scatter
__global__ __launch_bounds__(kScanThreads) void select_kernel(
    const int32_t* __restrict__ bucket, const unsigned long long* __restrict__ codes,
    const float* __restrict__ w, const int32_t* __restrict__ req,
    const int32_t* __restrict__ reqoff, const int32_t* __restrict__ off, int C,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, float* __restrict__ gate) {
  __shared__ int tmp[17];
  __shared__ int hist[256];
  __shared__ unsigned long long sh_prefix;
  __shared__ int sh_want;
  const int e = blockIdx.x;
  const int n = req[e];
  const int base = reqoff[e];
  const int o = off[e];
  const int tid = threadIdx.x;
  if (n <= C) {
    for (int i = tid; i < n; i += kScanThreads) {
      const int p = bucket[base + i];
      perm[o + i] = p;
      gate[o + i] = w[p];
      inv[p] = o + i;
    }
    return;
  }
  // Radix select of the C-th largest code among this expert's n codes.
  unsigned long long prefix = 0ull, pmask = 0ull;
  int want = C;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += kScanThreads) hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kScanThreads) {
      const unsigned long long u = codes[base + i];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns digits 255-4l .. 252-4l (descending); suffix counts from the top
      int c[4], s = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hist[255 - 4 * tid - q];
        s += c[q];
      }
      int incl = s;
#pragma unroll
      for (int off2 = 1; off2 < kWave; off2 <<= 1) {
        const int y = __shfl_up(incl, off2, kWave);
        if (tid >= off2) incl += y;
      }
      int above = incl - s;  // count of digits strictly above this lane's block
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (above < want && above + c[q] >= want) {
          sh_prefix = prefix | ((unsigned long long)(255 - 4 * tid - q) << shift);
          sh_want = want - above;
        }
        above += c[q];
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    want = sh_want;
    pmask |= 255ull << shift;
    __syncthreads();
  }
  // prefix = threshold code U; keep codes > U, and the first `want` codes == U.
  const unsigned long long U = prefix;
  int run_eq = 0, run_kept = 0;
  for (int i0 = 0; i0 < n; i0 += kScanThreads) {
    const int i = i0 + tid;
    unsigned long long u = 0ull;
    int p = -1;
    if (i < n) {
      u = codes[base + i];
      p = bucket[base + i];
    }
    const int eq = (i < n && u == U) ? 1 : 0;
    int tot_eq;
    const int eqr = block_scan_excl(eq, tmp, &tot_eq) + run_eq;
    const int kept = (i < n && (u > U || (eq && eqr < want))) ? 1 : 0;
    int tot_k;
    const int ks = block_scan_excl(kept, tmp, &tot_k) + run_kept;
    if (i < n) {
      if (kept) {
        perm[o + ks] = p;
        gate[o + ks] = w[p];
        inv[p] = o + ks;
      } else {
        inv[p] = -1;
      }
    }
    run_eq += tot_eq;
    run_kept += tot_k;
  }
}

}  // namespace

void carve_dispatch(Carver& c, int P, int N, DispatchScratch* s) {
  const int ntiles = cdiv(P > 0 ? P : 1, kDispatchTile);
  s->tilecnt = c.take<int32_t>((size_t)ntiles * N);
  s->tilebase = c.take<int32_t>((size_t)ntiles * N);
  s->bucket = c.take<int32_t>((size_t)(P > 0 ? P : 1));
  s->reqoff = c.take<int32_t>((size_t)N + 1);
  s->codes = c.take<unsigned long long>((size_t)(P > 0 ? P : 1));
}

hipError_t launch_dispatch(const int32_t* idx, const float* w, const double* key, int T, int N,
                           int k, int C, int32_t* req, int32_t* cnt, int32_t* off, int32_t* perm,
                           int32_t* inv, float* gate, int32_t* n_dropped,
                           const DispatchScratch& s, hipStream_t st) {
  const int P = T * k;
  if (P == 0) return hipSuccess;
  const int ntiles = cdiv(P, kDispatchTile);
  const int nblk = cdiv(ntiles, 4);
  const size_t lds = 4 * (size_t)N * sizeof(int);
  hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(256), lds, st, idx, P, N, ntiles, s.tilecnt);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, st, s.tilecnt, ntiles, N, P, C,
                     s.tilebase, req, cnt, s.reqoff, off, n_dropped);
  hipLaunchKernelGGL(bucket_kernel, dim3(nblk), dim3(256), lds, st, idx, key, P, N, ntiles,
                     s.tilebase, s.reqoff, s.bucket, s.codes, inv);
  hipLaunchKernelGGL(select_kernel, dim3(N), dim3(kScanThreads), 0, st, s.bucket, s.codes, w, req,
                     s.reqoff, off, C, perm, inv, gate);
  return hipGetLastError();
}

}  // namespace moe
