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
//   bucketing : every pair gets its rank among the earlier pairs of the same
//               expert (wave ballots inside a chunk of 64 pairs, running
//               per-expert counters in LDS across chunks, an exclusive scan
//               across waves / tiles), then lands in its expert's list in
//               token order next to its order-preserving 64-bit key code.
//               Small pair counts: one block does it all (fused kernel).
//               Large pair counts: hist (tile counts) -> per-expert column
//               scan -> expert offsets -> bucket.
//   select    : one block per expert; under capacity: copy; over capacity:
//               an 8-pass radix select finds the C-th largest key code, then
//               an ordered block scan keeps the strictly larger codes and the
//               first equal ones in token order.
#include "moe_common.h"

namespace moe {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kFusedMaxPairs = 32768;  // pairs one block buckets by itself

__device__ __forceinline__ unsigned long long lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Lanes of this wave whose `v` equals mine (only among `valid` lanes), for
// values below 2^BITS.
template <int BITS>
__device__ __forceinline__ unsigned long long match_peers(int v, bool valid) {
  unsigned long long peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const bool bit = (v >> b) & 1;
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

// One wave walks pairs [p0, p1) in order, 64 at a time; `cnt` (LDS, per
// expert) holds running counts that start at the caller's bases. For each pair
// `emit(p, e, pos)` gets cnt[e] at the pair's turn. Expert ids outside [0, N)
// are skipped, so bad ids cannot index out of range.
template <typename Emit>
__device__ __forceinline__ void walk_pairs(const int32_t* __restrict__ idx, int p0, int p1, int N,
                                           int* cnt, Emit emit) {
  const int l = lane_id();
  for (int c0 = p0; c0 < p1; c0 += kWave) {
    const int p = c0 + l;
    const int e = (p < p1) ? idx[p] : 0;
    const bool valid = p < p1 && (unsigned)e < (unsigned)N;
    const unsigned long long peers = match_peers<10>(e, valid);  // expert ids < 1024
    const int before = __popcll(peers & lanemask_lt());
    int base = 0;
    if (valid) base = cnt[e];
    // every lane has read cnt[] for this chunk before the leaders update it
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      emit(p, e, base + before);
      if (before == 0) cnt[e] = base + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

__device__ __forceinline__ void write_slot(int32_t* perm, int32_t* inv, float* gate,
                                           const float* w, int p, int s) {
  perm[s] = p;
  gate[s] = w[p];
  inv[p] = s;
}

// ------------------------------------------------------------ fused (small P)
// One block of 16 waves; wave v walks a contiguous range of pairs twice:
// first counting per expert, then (after the block turns counts into bases)
// placing each pair. With no possible overflow (C >= T) the slot of a pair is
// its bucket position, so perm / inv / gate are written here directly.
__global__ __launch_bounds__(kScanThreads) void fused_dispatch_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, const double* __restrict__ key,
    int P, int N, int C, int direct, int32_t* __restrict__ req, int32_t* __restrict__ cnt,
    int32_t* __restrict__ off, int32_t* __restrict__ reqoff, int32_t* __restrict__ n_dropped,
    int32_t* __restrict__ bucket, unsigned long long* __restrict__ codes,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, float* __restrict__ gate) {
  constexpr int NWV = kScanThreads / kWave;
  extern __shared__ int fsm[];  // [NWV][N] counters, then [N] request offsets
  __shared__ int tmp[17];
  __shared__ int carry[2];
  const int wv = threadIdx.x / kWave;
  const int l = lane_id();
  int* my = fsm + wv * N;
  int* sh_reqoff = fsm + NWV * N;
  const int span = cdiv(cdiv(P, NWV), kWave) * kWave;
  const int p0 = min(P, wv * span), p1 = min(P, p0 + span);
  for (int e = l; e < N; e += kWave) my[e] = 0;
  __builtin_amdgcn_wave_barrier();
  walk_pairs(idx, p0, p1, N, my, [](int, int, int) {});
  if (threadIdx.x == 0) carry[0] = carry[1] = 0;
  __syncthreads();
  // per expert: totals, bases across waves, expert offsets
  for (int e0 = 0; e0 < N; e0 += kScanThreads) {
    const int e = e0 + threadIdx.x;
    int r = 0;
    if (e < N) {
      for (int q = 0; q < NWV; ++q) {
        const int c = fsm[q * N + e];
        fsm[q * N + e] = r;
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
      sh_reqoff[e] = carry[0] + xr;
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
  for (int e = l; e < N; e += kWave) my[e] += sh_reqoff[e];
  __builtin_amdgcn_wave_barrier();
  if (direct) {
    walk_pairs(idx, p0, p1, N, my,
               [&](int p, int, int pos) { write_slot(perm, inv, gate, w, p, pos); });
  } else {
    walk_pairs(idx, p0, p1, N, my, [&](int p, int, int pos) {
      bucket[pos] = p;
      codes[pos] = key_code(key[p]);
    });
  }
  for (int p = p0 + l; p < p1; p += kWave)
    if ((unsigned)idx[p] >= (unsigned)N) inv[p] = -1;
}

// ------------------------------------------------------------ large P: hist
// One wave per tile of kDispatchTile pairs; counts land expert-major,
// tcnt[e * ntiles + tile], so the column scan below reads contiguously.
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int P, int N,
                                                   int ntiles, int32_t* __restrict__ tcnt) {
  extern __shared__ int hsm[];  // [4][N]
  const int wv = threadIdx.x / kWave;
  const int l = lane_id();
  const int tile = blockIdx.x * 4 + wv;
  int* c = hsm + wv * N;
  for (int e = l; e < N; e += kWave) c[e] = 0;
  __builtin_amdgcn_wave_barrier();
  if (tile >= ntiles) return;
  const int p0 = tile * kDispatchTile;
  walk_pairs(idx, p0, min(P, p0 + kDispatchTile), N, c, [](int, int, int) {});
  __builtin_amdgcn_wave_barrier();
  for (int e = l; e < N; e += kWave) tcnt[(size_t)e * ntiles + tile] = c[e];
}

// One block per expert: exclusive scan of its tile counts.
__global__ __launch_bounds__(256) void colscan_kernel(const int32_t* __restrict__ tcnt, int ntiles,
                                                      int32_t* __restrict__ tbase,
                                                      int32_t* __restrict__ req) {
  __shared__ int tmp[17];
  const int e = blockIdx.x;
  const int32_t* col = tcnt + (size_t)e * ntiles;
  int32_t* out = tbase + (size_t)e * ntiles;
  int run = 0;
  for (int t0 = 0; t0 < ntiles; t0 += 256) {
    const int t = t0 + threadIdx.x;
    const int v = t < ntiles ? col[t] : 0;
    int tot;
    const int x = block_scan_excl(v, tmp, &tot);
    if (t < ntiles) out[t] = run + x;
    run += tot;
  }
  if (threadIdx.x == 0) req[e] = run;
}

// One block: request and kept offsets over experts.
__global__ __launch_bounds__(kScanThreads) void offsets_kernel(
    const int32_t* __restrict__ req, int N, int P, int C, int32_t* __restrict__ cnt,
    int32_t* __restrict__ reqoff, int32_t* __restrict__ off, int32_t* __restrict__ n_dropped) {
  __shared__ int tmp[17];
  __shared__ int carry[2];
  if (threadIdx.x == 0) carry[0] = carry[1] = 0;
  for (int e0 = 0; e0 < N; e0 += kScanThreads) {
    const int e = e0 + threadIdx.x;
    const int r = e < N ? req[e] : 0;
    const int kept = min(r, C);
    int tot_r, tot_k;
    const int xr = block_scan_excl(r, tmp, &tot_r);
    const int xk = block_scan_excl(kept, tmp, &tot_k);
    if (e < N) {
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

__global__ __launch_bounds__(256) void bucket_kernel(
    const int32_t* __restrict__ idx, const double* __restrict__ key, int P, int N, int ntiles,
    const int32_t* __restrict__ tbase, const int32_t* __restrict__ reqoff,
    int32_t* __restrict__ bucket, unsigned long long* __restrict__ codes,
    int32_t* __restrict__ inv) {
  extern __shared__ int bsm[];  // [4][N]
  const int wv = threadIdx.x / kWave;
  const int l = lane_id();
  const int tile = blockIdx.x * 4 + wv;
  int* c = bsm + wv * N;
  if (tile < ntiles)
    for (int e = l; e < N; e += kWave) c[e] = reqoff[e] + tbase[(size_t)e * ntiles + tile];
  __builtin_amdgcn_wave_barrier();
  if (tile >= ntiles) return;
  const int p0 = tile * kDispatchTile, p1 = min(P, p0 + kDispatchTile);
  walk_pairs(idx, p0, p1, N, c, [&](int p, int, int pos) {
    bucket[pos] = p;
    codes[pos] = key_code(key[p]);
  });
  for (int p = p0 + l; p < p1; p += kWave)
    if ((unsigned)idx[p] >= (unsigned)N) inv[p] = -1;
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
    for (int i = tid; i < n; i += kScanThreads)
      write_slot(perm, inv, gate, w, bucket[base + i], o + i);
    return;
  }
  // Radix select of the C-th largest code among this expert's n codes.
  unsigned long long prefix = 0ull, pmask = 0ull;
  int want = C;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += kScanThreads) hist[b] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += kScanThreads) {
      const int i = i0 + tid;
      const unsigned long long u = i < n ? codes[base + i] : 0ull;
      const bool cand = i < n && (u & pmask) == prefix;
      const int dig = (int)((u >> shift) & 255);
      // lanes with the same digit add once (high digits are shared by most keys)
      const unsigned long long peers = match_peers<8>(dig, cand);
      if (cand && __popcll(peers & lanemask_lt()) == 0) atomicAdd(&hist[dig], __popcll(peers));
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
      if (kept) write_slot(perm, inv, gate, w, p, o + ks);
      else inv[p] = -1;
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
  // an expert receives at most T requests, so with C >= T nothing can drop
  // and bucket order is slot order
  const bool can_drop = C < T;
  const bool fused = P <= kFusedMaxPairs;
  if (fused) {
    const size_t lds = ((size_t)(kScanThreads / kWave) * N + N) * sizeof(int);
    MOE_SET_LDS_ONCE(fused_dispatch_kernel, 160 * 1024);
    hipLaunchKernelGGL(fused_dispatch_kernel, dim3(1), dim3(kScanThreads), lds, st, idx, w, key, P,
                       N, C, can_drop ? 0 : 1, req, cnt, off, s.reqoff, n_dropped, s.bucket,
                       s.codes, perm, inv, gate);
  } else {
    const int ntiles = cdiv(P, kDispatchTile);
    const int nblk = cdiv(ntiles, 4);
    const size_t lds = 4 * (size_t)N * sizeof(int);
    hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(256), lds, st, idx, P, N, ntiles, s.tilecnt);
    hipLaunchKernelGGL(colscan_kernel, dim3(N), dim3(256), 0, st, s.tilecnt, ntiles, s.tilebase,
                       req);
    hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(kScanThreads), 0, st, req, N, P, C, cnt,
                       s.reqoff, off, n_dropped);
    hipLaunchKernelGGL(bucket_kernel, dim3(nblk), dim3(256), lds, st, idx, key, P, N, ntiles,
                       s.tilebase, s.reqoff, s.bucket, s.codes, inv);
  }
  if (can_drop || !fused)
    hipLaunchKernelGGL(select_kernel, dim3(N), dim3(kScanThreads), 0, st, s.bucket, s.codes, w,
                       req, s.reqoff, off, C, perm, inv, gate);
  return hipGetLastError();
}

}  // namespace moe
