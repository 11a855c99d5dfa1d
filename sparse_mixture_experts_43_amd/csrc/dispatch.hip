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
#include "topk.h"

namespace moe {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kFusedMaxPairs = 32768;  // pairs one block buckets by itself
constexpr int kBatch = 8;              // global loads per thread in flight together

__device__ __forceinline__ unsigned long long lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Lanes of this wave whose `v` equals mine (only among `valid` lanes), for
// values below 2^nbits, nbits <= 10 uniform across the wave: expert ids need
// only ceil(log2 N) bits.
__device__ __forceinline__ unsigned long long match_peers_n(int v, bool valid, int nbits) {
  unsigned long long peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (v >> b) & 1;
    const unsigned long long m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// bits of an expert id (N <= 1024)
__device__ __forceinline__ int id_bits(int N) { return N > 1 ? 32 - __clz(N - 1) : 0; }

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
// are skipped, so bad ids cannot index out of range. `idx` is the global
// int32 array or an int16 copy in LDS.
template <typename Id, typename Emit>
__device__ __forceinline__ void walk_pairs(const Id* __restrict__ idx, int p0, int p1, int N,
                                           int* cnt, Emit emit) {
  const int l = lane_id();
  const int nbits = id_bits(N);
  for (int c0 = p0; c0 < p1; c0 += kWave) {
    const int p = c0 + l;
    const int e = (p < p1) ? idx[p] : 0;
    const bool valid = p < p1 && (unsigned)e < (unsigned)N;
    const unsigned long long peers = match_peers_n(e, valid, nbits);
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

// Capacity rank of pair p as an order-preserving 64-bit code (larger = kept
// first): the fp64 log-probability key, or with first-come capacity (fc_k =
// k) the negated token index, so an expert keeps its earliest requests (a
// token asks an expert at most once, so these never tie).
__device__ __forceinline__ unsigned long long rank_code(const double* __restrict__ key, int p,
                                                        int fc_k) {
  return fc_k > 0 ? key_code(-(double)(p / fc_k)) : key_code(key[p]);
}

// ------------------------------------------------------------ fused (small P)
// One block of 16 waves. The expert ids are first copied into LDS as int16
// (-1 for ids outside [0, N)); wave v then walks a contiguous range of pairs
// twice from LDS: first counting per expert, then (after the block turns
// counts into bases) recording each pair's position in place of its id. A last
// parallel pass writes the outputs with coalesced reads of w / key: with no
// possible overflow (C >= T) the slot of a pair is its bucket position, so
// perm / inv / gate are written directly; otherwise the request-ordered
// bucket and its keys.
__global__ __launch_bounds__(kScanThreads) void fused_dispatch_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, const double* __restrict__ key,
    int P, int N, int C, int direct, int fc_k, int32_t* __restrict__ req,
    int32_t* __restrict__ cnt,
    int32_t* __restrict__ off, int32_t* __restrict__ reqoff, int32_t* __restrict__ n_dropped,
    int32_t* __restrict__ bucket, unsigned long long* __restrict__ codes,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, float* __restrict__ gate) {
  constexpr int NWV = kScanThreads / kWave;
  extern __shared__ int fsm[];  // [NWV][N] counters, [N] request offsets, then int16 ids[P]
  __shared__ int tmp[17];
  __shared__ int carry[2];
  const int wv = threadIdx.x / kWave;
  const int l = lane_id();
  int* my = fsm + wv * N;
  int* sh_reqoff = fsm + NWV * N;
  int16_t* sid = (int16_t*)(fsm + NWV * N + N);
  // global loads in batches of kBatch per thread, issued before any is used
  for (int q0 = 0; q0 < P; q0 += kBatch * kScanThreads) {
    int ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = q0 + u * kScanThreads + (int)threadIdx.x;
      ev[u] = p < P ? idx[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = q0 + u * kScanThreads + (int)threadIdx.x;
      if (p < P) sid[p] = (unsigned)ev[u] < (unsigned)N ? (int16_t)ev[u] : (int16_t)-1;
    }
  }
  const int span = cdiv(cdiv(P, NWV), kWave) * kWave;
  const int p0 = min(P, wv * span), p1 = min(P, p0 + span);
  for (int e = l; e < N; e += kWave) my[e] = 0;
  __syncthreads();
  // this wave's requests per expert (order-free: one LDS add per pair on the
  // wave's own counters; the positions below follow pair order)
  for (int p = p0 + l; p < p1; p += kWave) {
    const int e = sid[p];
    if (e >= 0) atomicAdd(&my[e], 1);
  }
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
  // positions (< P <= 32768) replace the ids of valid pairs
  walk_pairs(sid, p0, p1, N, my, [&](int p, int, int pos) { sid[p] = (int16_t)pos; });
  __syncthreads();
  for (int q0 = 0; q0 < P; q0 += kBatch * kScanThreads) {
    int sv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = q0 + u * kScanThreads + (int)threadIdx.x;
      sv[u] = p < P ? (int)sid[p] : -1;
    }
    if (direct) {
      float wv_[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int p = q0 + u * kScanThreads + (int)threadIdx.x;
        wv_[u] = sv[u] >= 0 ? w[p] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int p = q0 + u * kScanThreads + (int)threadIdx.x;
        if (p >= P) continue;
        const int s = sv[u];
        if (s < 0) {
          inv[p] = -1;
        } else {
          perm[s] = p;
          gate[s] = wv_[u];
          inv[p] = s;
        }
      }
    } else {
      // the pairs in bucket order only: the selection that follows computes
      // their rank codes from `key` and writes inv for every pair it sees
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int p = q0 + u * kScanThreads + (int)threadIdx.x;
        if (p >= P) continue;
        const int s = sv[u];
        if (s < 0) inv[p] = -1;
        else bucket[s] = p;
      }
    }
  }
}

// ------------------------------------------------------------ route + dispatch (few tokens)
// Few tokens (T <= 64, N <= 64, k <= 16): the split-K router leaves S partial
// logit tiles part[s][r][n] (r < Tp = 16 cdiv(T, 16), n < NP). One block adds
// them (splitk_logit, as the router's own top-k kernel does, so both give the
// same bits), adds the bias and runs the top-k of every row (logits and key to
// global memory, the picks and weights to LDS as well), then dispatches the
// P = T*k <= 1024 pairs from LDS:
//   wave c owns pairs 64c .. 64c+63; per expert one ballot gives the chunk's
//   count and each pair's rank among the chunk's pairs of that expert;
//   wave 0 (lane = expert) adds the chunk counts in chunk order (the chunk
//   bases), scans requests and kept counts over the experts and writes
//   req / cnt / reqoff / off / n_dropped;
//   a pair's bucket position is its expert's request offset + the counts of
//   the earlier chunks + its rank: expert-major, pair order within an expert,
//   the layout the other dispatch paths produce.
// With no possible overflow (C >= T) the position is the slot (perm, gate,
// inv written here); otherwise the request-ordered bucket, which the
// selection that follows turns into slots. One launch and three global round
// trips fewer than router + dispatch.
constexpr int kRouteDispatchPairs = 64 * kMaxK;
template <int NT>
__global__ __launch_bounds__(kScanThreads) void route_dispatch_kernel(
    const float* __restrict__ part, int S, int Tp, const float* __restrict__ bias, int T, int N,
    int k, float* __restrict__ logits, int32_t* __restrict__ idx, float* __restrict__ w,
    double* __restrict__ key, int C, int direct, int32_t* __restrict__ req,
    int32_t* __restrict__ cnt, int32_t* __restrict__ off, int32_t* __restrict__ reqoff,
    int32_t* __restrict__ n_dropped, int32_t* __restrict__ bucket, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, float* __restrict__ gate) {
  constexpr int NP = NT * 16;
  constexpr int kRows = 64;
  constexpr int NWV = kScanThreads / kWave;
  static_assert(NWV * kWave >= kRouteDispatchPairs, "one 64-pair chunk per wave");
  __shared__ float Ls[kRows][NP + 4];
  __shared__ int32_t s_idx[kRouteDispatchPairs];
  __shared__ float s_w[kRouteDispatchPairs];
  __shared__ int s_cc[NWV][kWave];  // per chunk and expert: count, then base
  __shared__ int s_roff[kWave];
  const int l = lane_id();
  const int wv = threadIdx.x / kWave;
  const size_t stride = (size_t)Tp * NP;
  for (int i = threadIdx.x; i < kRows * NP; i += kScanThreads) {
    const int r = i / NP, n = i - r * NP;
    float v = 0.f;
    if (r < Tp) {
      // (fewer loads in flight where four waves per SIMD leave 128 VGPRs to
      // the wider top-k)
      v = splitk_logit<NT == 1 ? 32 : 16>(part + (size_t)r * NP + n, S, stride);
      v += (bias != nullptr && n < N) ? bias[n] : 0.f;
    }
    Ls[r][n] = v;
  }
  __syncthreads();
  if constexpr (NT == 1) {
    // 16 waves x 4 rows (16-lane groups) cover the 64 rows; waves past the
    // last token skip (their reductions stay inside the wave)
    if (wv * 4 < T) {
      const int r = wv * 4 + (l >> 4);
      topk_row16(&Ls[r][0], r < T, N, k, r, logits, s_idx, s_w, key);
    }
  } else {
    for (int r = wv; r < T; r += NWV) topk_row(&Ls[r][0], N, k, r, logits, s_idx, s_w, key);
  }
  __syncthreads();
  const int P = T * k;
  const int p = wv * kWave + l;
  const bool in = p < P;
  if (in) {
    idx[p] = s_idx[p];
    w[p] = s_w[p];
  }
  const int e = in ? s_idx[p] : -1;
  const bool ok = in && (unsigned)e < (unsigned)N;
  const unsigned long long lt = lanemask_lt();
  int rank = 0, ccount = 0;
  for (int ex = 0; ex < N; ++ex) {
    const unsigned long long m = __ballot(ok && e == ex);
    if (l == ex) ccount = __popcll(m);
    if (ok && e == ex) rank = __popcll(m & lt);
  }
  s_cc[wv][l] = ccount;
  __syncthreads();
  if (wv == 0) {
    int run = 0;
    for (int q = 0; q < NWV; ++q) {
      const int c = s_cc[q][l];
      s_cc[q][l] = run;
      run += c;
    }
    const int kept = run < C ? run : C;
    int ir = run, ik = kept;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int yr = __shfl_up(ir, o, kWave), yk = __shfl_up(ik, o, kWave);
      if (l >= o) {
        ir += yr;
        ik += yk;
      }
    }
    if (l < N) {
      req[l] = run;
      cnt[l] = kept;
      reqoff[l] = ir - run;
      off[l] = ik - kept;
    }
    s_roff[l] = ir - run;
    if (l == kWave - 1) {
      reqoff[N] = ir;
      off[N] = ik;
      *n_dropped = P - ik;
    }
  }
  __syncthreads();
  if (in) {
    if (!ok) {
      inv[p] = -1;
    } else {
      const int pos = s_roff[e] + s_cc[wv][e] + rank;
      if (direct) {
        perm[pos] = p;
        gate[pos] = s_w[p];
        inv[p] = pos;
      } else {
        bucket[pos] = p;
      }
    }
  }
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
    const int32_t* __restrict__ idx, const double* __restrict__ key, int fc_k, int P, int N,
    int ntiles,
    const int32_t* __restrict__ tbase, const int32_t* __restrict__ reqoff,
    const int32_t* __restrict__ req, int C,
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
    codes[pos] = rank_code(key, p, fc_k);
  });
  // invalid pairs, and every pair of an expert over capacity (the selection
  // then writes only its kept ones): coalesced here, scattered there
  for (int p = p0 + l; p < p1; p += kWave) {
    const int e = idx[p];
    if ((unsigned)e >= (unsigned)N || req[e] > C) inv[p] = -1;
  }
}

// ------------------------------------------------------------ select + scatter
// One block per expert. An expert within capacity writes its slots in bucket
// (token) order. Over capacity, the C-th largest U of the order-preserving
// 64-bit images of the fp64 keys is found by radix selection: the bits above
// the highest bit in which the expert's keys differ are common (block min/max);
// 256-bin passes on 8-bit digits from there down each pick the bin holding
// the C-th largest key, and once the remaining candidates fit in a short LDS
// list they are compacted into it, so the later passes scan only them; the
// passes stop early once the picked bin holds exactly the keys still wanted.
// The pairs with key above U and the first (lowest-token) ones equal to U are
// kept, in token order. The dispatch kernels before it have already marked
// every pair of an over-capacity expert dropped (inv = -1), so only the kept
// pairs are written here. Up to kSelLds keys are held in LDS.
constexpr int kSelLds = 16384;
constexpr int kSelList = 1024;  // compacted candidates

// Threshold digit of a histogram of `bins` (<= 2048) bins: the digit whose
// suffix count (from the top) first reaches `want`; run by one wave.
__device__ __forceinline__ void hist_pick(const int* hist, int bins, int want, int* out_dig,
                                          int* out_want) {
  const int l = lane_id();
  const int per = (bins + kWave - 1) / kWave;  // bins per lane, descending from the top
  int s = 0;
  for (int q = 0; q < per; ++q) {
    const int b = bins - 1 - (l * per + q);
    if (b >= 0) s += hist[b];
  }
  int incl = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (l >= o) incl += y;
  }
  int above = incl - s;
  for (int q = 0; q < per; ++q) {
    const int b = bins - 1 - (l * per + q);
    if (b < 0) break;
    const int c = hist[b];
    if (above < want && above + c >= want) {
      *out_dig = b;
      *out_want = want - above;
    }
    above += c;
  }
}

constexpr int kSelWaves = kScanThreads / kWave;
struct SelShared {
  int tmp[17];
  int hist[256];
  int whist[kSelWaves][256];  // per-wave sub-histograms
  unsigned long long list[kSelList];
  unsigned long long red[2][16];
  int dig, want, cnt;
};

// codes == nullptr: the rank codes are computed from the pairs' keys
// (rank_code of bucket[i]) instead of read.
template <bool LDSC>
__device__ __forceinline__ void select_body(
    const int32_t* __restrict__ bucket, const unsigned long long* __restrict__ codes,
    const double* __restrict__ key, int fc_k,
    const float* __restrict__ w, int n, int base, int o, int C, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, float* __restrict__ gate, unsigned long long* __restrict__ sc,
    SelShared& shm) {
  auto gcode = [&](int i) -> unsigned long long {
    return codes != nullptr ? codes[base + i] : rank_code(key, bucket[base + i], fc_k);
  };
  int* tmp = shm.tmp;
  int* hist = shm.hist;
  unsigned long long* list = shm.list;
  auto& red = shm.red;
  int& sh_dig = shm.dig;
  int& sh_want = shm.want;
  int& sh_cnt = shm.cnt;
  const int tid = threadIdx.x;
  const int l = lane_id(), wv = tid / kWave;
  // the keys (into LDS when they fit) and their block min and max, whose
  // common prefix every key shares
  unsigned long long mn = ~0ull, mx = 0ull;
  if constexpr (LDSC) {
    for (int i0 = 0; i0 < n; i0 += 4 * kScanThreads) {
      unsigned long long v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + q * kScanThreads + tid;
        v[q] = i < n ? gcode(i) : 0ull;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + q * kScanThreads + tid;
        if (i < n) {
          sc[i] = v[q];
          mn = v[q] < mn ? v[q] : mn;
          mx = v[q] > mx ? v[q] : mx;
        }
      }
    }
  } else {
    for (int i = tid; i < n; i += kScanThreads) {
      const unsigned long long u = gcode(i);
      mn = u < mn ? u : mn;
      mx = u > mx ? u : mx;
    }
  }
  auto code = [&](int i) -> unsigned long long { return LDSC ? sc[i] : gcode(i); };
#pragma unroll
  for (int off2 = 32; off2 > 0; off2 >>= 1) {
    const unsigned long long a = __shfl_xor(mn, off2, kWave), b2 = __shfl_xor(mx, off2, kWave);
    mn = a < mn ? a : mn;
    mx = b2 > mx ? b2 : mx;
  }
  if (l == 0) {
    red[0][wv] = mn;
    red[1][wv] = mx;
  }
  __syncthreads();
  mn = red[0][0];
  mx = red[1][0];
  for (int q = 1; q < kScanThreads / kWave; ++q) {
    mn = red[0][q] < mn ? red[0][q] : mn;
    mx = red[1][q] > mx ? red[1][q] : mx;
  }

  unsigned long long prefix, pmask;
  int want = C;
  if (mn == mx) {
    prefix = mn;  // every key equal: keep the first C by token
  } else {
    // 8-bit digits from the highest differing bit down; each pass scans the
    // candidates (all keys sharing the prefix so far), from the compacted
    // list once they fit in it
    int s_hi = 63 - __clzll((long long)(mn ^ mx));  // highest differing bit
    pmask = s_hi >= 63 ? 0ull : ~((2ull << s_hi) - 1ull);
    prefix = mn & pmask;
    bool compact = false;
    int lsize = 0;  // keys in the compacted list
    while (true) {
      const int sh = s_hi >= 7 ? s_hi - 7 : 0;  // digit = bits [sh, s_hi]
      const int bins = 1 << (s_hi - sh + 1);
      const unsigned long long dmask = (unsigned long long)(bins - 1);
      __syncthreads();  // earlier readers of hist / list are done
      for (int b2 = tid; b2 < kSelWaves * 256; b2 += kScanThreads) (&shm.whist[0][0])[b2] = 0;
      __syncthreads();
      const int nn = compact ? lsize : n;
      int* hw = shm.whist[wv];  // this wave's sub-histogram: no contention between waves
      for (int i0 = 0; i0 < nn; i0 += kScanThreads) {
        const int i = i0 + tid;
        const unsigned long long u = i < nn ? (compact ? list[i] : code(i)) : 0ull;
        const bool cand = i < nn && (u & pmask) == prefix;
        const int dig = (int)((u >> sh) & dmask);
        // one LDS atomic per candidate on its wave's own sub-histogram
        // (measured faster than first adding equal digits once per wave)
        if (cand) atomicAdd(&hw[dig], 1);
      }
      __syncthreads();
      for (int b2 = tid; b2 < bins; b2 += kScanThreads) {
        int sum = 0;
#pragma unroll
        for (int q = 0; q < kSelWaves; ++q) sum += shm.whist[q][b2];
        hist[b2] = sum;
      }
      __syncthreads();
      if (tid < kWave) hist_pick(hist, bins, want, &sh_dig, &sh_want);
      __syncthreads();
      prefix |= (unsigned long long)sh_dig << sh;
      pmask |= dmask << sh;
      want = sh_want;
      const int m_next = hist[sh_dig];
      // every candidate left in the bin is kept: the bin's lowest code, the
      // prefix with zeros below, already splits kept from dropped
      if (sh == 0 || m_next == want) break;
      s_hi = sh - 1;
      if (!compact && m_next <= kSelList) {
        // the remaining candidates fit in the list: compact them once
        if (tid == 0) sh_cnt = 0;
        __syncthreads();
        for (int i0 = 0; i0 < n; i0 += kScanThreads) {
          const int i = i0 + tid;
          const unsigned long long u = i < n ? code(i) : 0ull;
          if (i < n && (u & pmask) == prefix) list[atomicAdd(&sh_cnt, 1)] = u;
        }
        __syncthreads();
        compact = true;
        lsize = m_next;
      }
    }
  }
  // prefix = threshold code U; keep codes > U, and the first `want` codes == U.
  // Each wave takes a contiguous segment of the expert's requests (token
  // order), its lanes consecutive elements, ranks from ballot prefixes. A
  // wave keeps all its codes > U and, of its codes == U, as many as the
  // `want` left after the equal codes of the waves before it.
  const unsigned long long U = prefix;
  const bool stage = C <= 2 * kSelList;  // kept pair ids gathered in the candidate list
  int* kept_p = (int*)list;
  const int seg = ((n + kSelWaves - 1) / kSelWaves + kWave - 1) / kWave * kWave;
  const int s_beg = wv * seg, s_end = min(n, s_beg + seg);
  const unsigned long long lt = lanemask_lt();
  int n_eq = 0, n_gt = 0;
  for (int i0 = s_beg; i0 < s_end; i0 += kWave) {
    const int i = i0 + l;
    const unsigned long long u = i < s_end ? code(i) : 0ull;
    n_eq += __popcll(__ballot(i < s_end && u == U));
    n_gt += __popcll(__ballot(i < s_end && u > U));
  }
  int tot;
  const int eq_before = block_scan_excl(l == 0 ? n_eq : 0, tmp, &tot);
  const int eq_w = __shfl(eq_before, 0, kWave);  // equal keys before this wave's segment
  const int eq_keep = want - eq_w < 0 ? 0 : (want - eq_w > n_eq ? n_eq : want - eq_w);
  const int kept_before = block_scan_excl(l == 0 ? n_gt + eq_keep : 0, tmp, &tot);
  {
    int r = eq_w;
    int ks = o + __shfl(kept_before, 0, kWave);
    // the segment's pair ids first (all loads in flight), then the writes
    constexpr int kPre = kSelLds / kSelWaves / kWave;  // iterations of an LDS-sized segment
    int pre[kPre];
#pragma unroll
    for (int q = 0; q < kPre; ++q) {
      const int i = s_beg + q * kWave + l;
      pre[q] = i < s_end ? bucket[base + i] : 0;
    }
    for (int i0 = s_beg, q = 0; i0 < s_end; i0 += kWave, ++q) {
      const int i = i0 + l;
      const bool in = i < s_end;
      const unsigned long long u = in ? code(i) : 0ull;
      const int p = !in ? 0 : (q < kPre ? pre[q < kPre ? q : 0] : bucket[base + i]);
      const unsigned long long eqm = __ballot(in && u == U);
      const bool keep = in && (u > U || (u == U && r + __popcll(eqm & lt) < want));
      const unsigned long long km = __ballot(keep);
      if (keep) {
        const int slot = ks + __popcll(km & lt);
        inv[p] = slot;
        if (stage) {
          kept_p[slot - o] = p;
        } else {
          perm[slot] = p;
          gate[slot] = w[p];
        }
      } else if (in && codes == nullptr) {
        // dropped by the capacity limit (the bucketing kernels of the
        // multi-block path mark these pairs themselves, in parallel)
        inv[p] = -1;
      }
      ks += __popcll(km);
      r += __popcll(eqm);
    }
  }
  // The expert keeps exactly C pairs, in slots o .. o + C - 1. When C fits
  // the (by now unused) candidate list, the kept pair ids were gathered there
  // and perm and the gates are written after the loop: coalesced stores and
  // one batch of weight loads instead of a dependent load per iteration. (Not
  // read back from perm: global memory written by this kernel can be stale in
  // the CU's L1, which workgroups that ran there earlier may have filled.)
  if (stage) {
    __syncthreads();
    for (int i = tid; i < C; i += kScanThreads) {
      const int p = kept_p[i];
      perm[o + i] = p;
      gate[o + i] = w[p];
    }
  }
}

__global__ __launch_bounds__(kScanThreads) void select_kernel(
    const int32_t* __restrict__ bucket, const unsigned long long* __restrict__ codes,
    const double* __restrict__ key, int fc_k,
    const float* __restrict__ w, const int32_t* __restrict__ req,
    const int32_t* __restrict__ reqoff, const int32_t* __restrict__ off, int C,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, float* __restrict__ gate) {
  extern __shared__ __align__(16) unsigned long long sel_codes[];
  const int e = blockIdx.x;
  const int n = req[e];
  const int base = reqoff[e];
  const int o = off[e];
  if (n <= C) {
    for (int i = threadIdx.x; i < n; i += kScanThreads)
      write_slot(perm, inv, gate, w, bucket[base + i], o + i);
    return;
  }
  __shared__ SelShared shm;
  if (n <= kSelLds)
    select_body<true>(bucket, codes, key, fc_k, w, n, base, o, C, perm, inv, gate, sel_codes, shm);
  else
    select_body<false>(bucket, codes, key, fc_k, w, n, base, o, C, perm, inv, gate, nullptr, shm);
}

// ------------------------------------------------------------ survivor renormalisation
// One thread per token: a token that lost some but not all of its picks gets
// each kept pick's gate = w / (sum of its kept w), the kept weights summed in
// fp32 in pick order (wiki page, worked example: x4 keeps only E2, weight 1.0).
// Tokens that kept every pick keep their weights bit for bit.
__global__ __launch_bounds__(256) void renorm_kernel(const float* __restrict__ w,
                                                     const int32_t* __restrict__ inv, int T,
                                                     int k, float* __restrict__ gate) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int32_t* it = inv + (size_t)t * k;
  const float* wt = w + (size_t)t * k;
  float sum = 0.f;
  int kept = 0;
  for (int j = 0; j < k; ++j)
    if (it[j] >= 0) {
      sum += wt[j];
      ++kept;
    }
  if (kept == 0 || kept == k) return;
  for (int j = 0; j < k; ++j)
    if (it[j] >= 0) gate[it[j]] = wt[j] / sum;
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

template <int NT>
void launch_route_dispatch(const RoutePartials& rp, int T, int N, int k, int C, int direct,
                           int32_t* req, int32_t* cnt, int32_t* off, int32_t* perm, int32_t* inv,
                           float* gate, int32_t* n_dropped, const DispatchScratch& s,
                           hipStream_t st) {
  hipLaunchKernelGGL(route_dispatch_kernel<NT>, dim3(1), dim3(kScanThreads), 0, st, rp.part,
                     rp.S, rp.Tp, rp.bias, T, N, k, rp.logits, rp.idx, rp.w, rp.key, C, direct,
                     req, cnt, off, s.reqoff, n_dropped, s.bucket, perm, inv, gate);
}

hipError_t launch_dispatch(const int32_t* idx, const float* w, const double* key, int T, int N,
                           int k, int C, int flags, int32_t* req, int32_t* cnt, int32_t* off,
                           int32_t* perm, int32_t* inv, float* gate, int32_t* n_dropped,
                           const DispatchScratch& s, hipStream_t st, const RoutePartials* rp) {
  const int P = T * k;
  if (P == 0) return hipSuccess;
  // an expert receives at most T requests, so with C >= T nothing can drop
  // and bucket order is slot order
  const bool can_drop = C < T;
  const bool fused = P <= kFusedMaxPairs;
  const int fc_k = (flags & kFlagFirstCome) ? k : 0;
  if (rp != nullptr) {
    // few tokens: the router's top-k runs in the dispatch block (P <= 64 * 16)
    if (T > 64 || rp->NP > 64 || P > kRouteDispatchPairs || rp->idx != idx || rp->w != w ||
        rp->key != key)
      return hipErrorInvalidValue;
    const int direct = can_drop ? 0 : 1;
    switch (rp->NP / 16) {
      case 1: launch_route_dispatch<1>(*rp, T, N, k, C, direct, req, cnt, off, perm, inv, gate, n_dropped, s, st); break;
      case 2: launch_route_dispatch<2>(*rp, T, N, k, C, direct, req, cnt, off, perm, inv, gate, n_dropped, s, st); break;
      case 3: launch_route_dispatch<3>(*rp, T, N, k, C, direct, req, cnt, off, perm, inv, gate, n_dropped, s, st); break;
      default: launch_route_dispatch<4>(*rp, T, N, k, C, direct, req, cnt, off, perm, inv, gate, n_dropped, s, st); break;
    }
  } else if (fused) {
    const size_t lds = ((size_t)(kScanThreads / kWave) * N + N) * sizeof(int) +
                       (size_t)P * sizeof(int16_t);
    MOE_SET_LDS_ONCE(fused_dispatch_kernel, 160 * 1024);
    hipLaunchKernelGGL(fused_dispatch_kernel, dim3(1), dim3(kScanThreads), lds, st, idx, w, key, P,
                       N, C, can_drop ? 0 : 1, fc_k, req, cnt, off, s.reqoff, n_dropped, s.bucket,
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
    hipLaunchKernelGGL(bucket_kernel, dim3(nblk), dim3(256), lds, st, idx, key, fc_k, P, N,
                       ntiles, s.tilebase, s.reqoff, req, C, s.bucket, s.codes, inv);
  }
  if (can_drop || !fused)
  {
    // LDS for the keys of one expert; at most T requests reach an expert
    const int nmax = T < kSelLds ? T : kSelLds;
    const size_t lds = (size_t)nmax * sizeof(unsigned long long);
    MOE_SET_LDS_ONCE(select_kernel, 160 * 1024);
    // (the fused path leaves the rank codes to the selection)
    hipLaunchKernelGGL(select_kernel, dim3(N), dim3(kScanThreads), lds, st, s.bucket,
                       fused ? nullptr : s.codes, key, fc_k, w, req, s.reqoff, off, C, perm, inv,
                       gate);
  }
  // nothing can drop when C >= T: the weights stay as they are
  if ((flags & kFlagRenorm) && can_drop)
    hipLaunchKernelGGL(renorm_kernel, dim3(cdiv(T, 256)), dim3(256), 0, st, w, inv, T, k, gate);
  return hipGetLastError();
}

}  // namespace moe
