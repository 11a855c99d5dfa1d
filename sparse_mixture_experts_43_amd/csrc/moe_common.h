// Shared device helpers and host-side launch declarations of libmoe.
// gfx950 (CDNA4) only: wave64, bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kWave = 64;
constexpr int kMaxN = 1024;
constexpr int kMaxK = 16;

enum Dtype : int { kF32 = 0, kBF16 = 1 };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// Exact GELU, z * Phi(z) = z * (1 + erf(z / sqrt(2))) / 2, with the device
// library's single-precision erf.
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, wave_shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += wave_shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += wave_shfl_xor(v, o);
  return v;
}

// Order-preserving map of an fp64 key to uint64 (larger key -> larger code).
// -0.0 is folded onto +0.0 first so that equal keys give equal codes.
__device__ __forceinline__ unsigned long long key_code(double k) {
  if (k == 0.0) k = 0.0;
  unsigned long long b = (unsigned long long)__double_as_longlong(k);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Slot rows [m0, m0 + mcount) of expert e for an expert GEMM planned for at
// most S_cap slots in all and `cap` per expert. Offsets from moe_dispatch with
// the same sizes and capacity factor are within both bounds already; other
// offsets are clamped so every access stays inside the plan's buffers (the
// rows past the bounds are then not computed).
__device__ __forceinline__ void expert_rows(const int32_t* __restrict__ off, int e, int S_cap,
                                            int cap, int& m0, int& mcount) {
  int a = off[e], b = off[e + 1];
  a = a < 0 ? 0 : (a > S_cap ? S_cap : a);
  b = b < a ? a : (b > S_cap ? S_cap : b);
  m0 = a;
  mcount = b - a < cap ? b - a : cap;
}

// ---------------------------------------------------------------- host side
// Raise a kernel's dynamic-LDS limit to all the LDS a workgroup may have
// (160 KB on gfx950) minus its static LDS. Once per call site (idempotent; a
// race between threads only repeats the call).
inline void allow_max_dynamic_lds(const void* func) {
  hipFuncAttributes a{};
  if (hipFuncGetAttributes(&a, func) != hipSuccess) return;
  const int limit = 160 * 1024 - (int)a.sharedSizeBytes;
  (void)hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, limit);
}
#define MOE_SET_LDS_ONCE(kern, lds)                    \
  do {                                                 \
    static bool done_ = false;                         \
    if (!done_) {                                      \
      allow_max_dynamic_lds((const void*)(kern));      \
      done_ = true;                                    \
    }                                                  \
    (void)(lds);                                       \
  } while (0)

// Capacity per the documented formula (moe.h).
int capacity_host(int T, int N, int k, double cf);

// Workspace carve: every piece 256-byte aligned.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    off = align_up(off, 256);
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

// Dispatch scratch (sizes depend on T*k and N only).
struct DispatchScratch {
  int32_t* tilecnt;   // [ntiles, N] requests per expert in each tile of pairs
  int32_t* tilebase;  // [ntiles, N] requests per expert in earlier tiles
  int32_t* bucket;    // [T*k] pairs grouped by expert, token order
  int32_t* reqoff;    // [N+1] exclusive scan of requests per expert
  unsigned long long* codes;  // [T*k] order-preserving key codes, bucket order
};
constexpr int kDispatchTile = 512;  // pairs per histogram tile (one wave each)
void carve_dispatch(Carver& c, int P, int N, DispatchScratch* s);

// Expert FFN scratch.
struct FfnScratch {
  void* hidden;       // [S_max, d_ff] activation dtype
  void* hidden_lo;    // [S_max, d_ff] bf16 residual of the hidden layer (split mode) or null
  int32_t* tiles;     // GEMM tile tables (int4 entries) for both GEMMs
  int32_t* counts;    // [20]: tile counts written by the schedule kernel, then the
                      // GEMMs' per-XCD work-queue counters (zeroed by it)
  float* part;        // split-K partial sums of the decode GEMMs, or null
  int32_t* direct;    // [S_max]: direct-row map (DirectRows), tiled bf16 paths only
};
// Direct rows: when the combine would only copy a token's single kept pick,
// the second expert GEMM writes that row of y itself and the combine leaves
// it alone. The schedule kernel writes map[slot] = token when the slot's
// token kept no other pick (counted from inv), else -1. The caller fills y,
// y_dtype and inv; launch_expert_ffn sets map and used when its path writes
// direct rows (tiled bf16 on the LDS ring), else leaves used false.
struct DirectRows {
  void* y = nullptr;
  int y_dtype = 0;
  const int32_t* inv = nullptr;  // [T*k] pair -> slot or -1
  int32_t* map = nullptr;
  bool used = false;
};
constexpr int kFlagHiddenSplit = 1;  // MOE_FLAG_HIDDEN_SPLIT
constexpr int kFlagYF32 = 2;         // MOE_FLAG_Y_F32
constexpr int kFlagFirstCome = 4;    // MOE_FLAG_FIRST_COME
constexpr int kFlagRenorm = 8;       // MOE_FLAG_RENORM_SURVIVORS
constexpr int kFlagIdentity = 16;    // MOE_FLAG_IDENTITY_FALLBACK
constexpr int kFlagExpertChoice = 32;  // MOE_FLAG_EXPERT_CHOICE
constexpr int kFlagPacked = 64;        // MOE_FLAG_PACKED_WEIGHTS
void carve_ffn(Carver& c, int T, int d, int d_ff, int N, int k, int C, int S_max, int dtype,
               int flags, FfnScratch* s);

// Profiling marks: records the event registered for `slot` (if any) on `st`.
// Slots: 0 before the router, 1 after the router, 2 after dispatch, 3 before
// the first expert GEMM, 4 after it, 5 after the second expert GEMM, 6 after
// the combine.
void profile_mark(int slot, hipStream_t st);

// Split-K router state for few tokens (T <= 64, N <= 64, bf16, d % 128 == 0):
// partial logit tiles part[s][r][n] (fp32, s < S, r < Tp = 16 cdiv(T, 16),
// n < NP = 16 cdiv(N, 16)) in the router scratch, and where the routing that
// finishes from them writes its results.
struct RoutePartials {
  const float* part = nullptr;
  int S = 0, Tp = 0, NP = 0;
  const float* bias = nullptr;
  float* logits = nullptr;
  int32_t* idx = nullptr;
  float* w = nullptr;
  double* key = nullptr;
};

// Launchers (return hipError_t of the last launch).
size_t route_scratch_bytes(int d, int N, int dtype);  // transposed router weight
hipError_t launch_route(const void* x, const void* W_g, const float* bias, int T, int d, int N,
                        int k, int dtype, float* logits, int32_t* idx, float* w, double* key,
                        void* scratch, hipStream_t st);
// Few tokens (the RoutePartials shapes): only the split-K router's first
// kernel, and *rp filled for launch_dispatch, which finishes the routing. For
// other shapes nothing is launched and rp->part stays null.
hipError_t launch_route_partials(const void* x, const void* W_g, const float* bias, int T, int d,
                                 int N, int dtype, float* logits, int32_t* idx, float* w,
                                 double* key, void* scratch, hipStream_t st, RoutePartials* rp);
// flags: kFlagFirstCome, kFlagRenorm.
// Expert choice: from fp32 logits [T, N], every pair t*N + e as a candidate:
// idx = e, w = p[t,e], key = log p[t,e] (fp64).
hipError_t launch_route_expert_choice(const float* logits, int T, int N, int32_t* idx, float* w,
                                     double* key, hipStream_t st);
// With `rp` (the split-K router's partial logits, few tokens) the dispatch
// block first finishes the routing: it adds the partials, runs the top-k and
// writes rp->logits / idx / w / key (the same arrays as idx / w / key here).
hipError_t launch_dispatch(const int32_t* idx, const float* w, const double* key, int T, int N,
                           int k, int C, int flags, int32_t* req, int32_t* cnt, int32_t* off,
                           int32_t* perm, int32_t* inv, float* gate, int32_t* n_dropped,
                           const DispatchScratch& s, hipStream_t st,
                           const RoutePartials* rp = nullptr);
// Routing statistics: scratch bytes and launch (stats: [2N + 2] fp32).
size_t stats_scratch_bytes(int T, int N);
hipError_t launch_routing_stats(const float* logits, const int32_t* idx, int T, int N, int k,
                                float* stats, void* scratch, hipStream_t st);
// Second expert GEMM left as K-split fp32 partials (decode path): the combine
// finishes the slot outputs, gate * (sum_q part[q] + b2), in the same order of
// operations as the split-K reduction would.
struct SplitK {
  const float* part = nullptr;  // [nsplit][S_cap][d]
  int nsplit = 1;
  int S_cap = 0;
  const void* bias = nullptr;   // b2 [N, d] activation dtype, or null
  bool f32 = false;             // fp32 activations (bias, x) instead of bf16
  const float* gate = nullptr;  // slot gates
  const int32_t* off = nullptr; // expert offsets [N+1] (slot -> expert for the bias)
  int N = 0;
};
// defer: when not null and the plan splits the second GEMM's K, its reduction
// is skipped and described in *defer (nsplit > 1) for launch_combine_splitk.
hipError_t launch_expert_ffn(const void* x, const int32_t* perm, const int32_t* off,
                             const float* gate, const void* W1, const void* b1, const void* W2,
                             const void* b2, int T, int d, int d_ff, int N, int k, int C,
                             int S_max, int dtype, int flags, void* slot_out,
                             const FfnScratch& s, hipStream_t st, SplitK* defer = nullptr,
                             DirectRows* dr = nullptr);
// y_dtype: dtype of y; x (x_dtype, [T, d]) is read for tokens with no kept
// pick when not null (identity fallback), else such tokens get zeros; sh (fp32
// [T, d], a shared expert's output) is added to every token when not null.
// skip_single: tokens that kept exactly one pick are left alone (their rows
// were written by the second expert GEMM: DirectRows).
hipError_t launch_combine(const void* slot_out, const int32_t* inv, int T, int d, int k,
                          int y_dtype, const void* x, int x_dtype, const float* sh, void* y,
                          hipStream_t st, bool skip_single = false);
hipError_t launch_combine_splitk(const SplitK& sk, const int32_t* inv, int T, int d, int k,
                                 int y_dtype, const void* x, int x_dtype, const float* sh,
                                 void* y, hipStream_t st);
// Weights [N, rows, K] bf16 -> the packed piece layout of gemm_ring.h (same
// size; rows % 16 == 0, K % 32 == 0).
hipError_t launch_pack_weights(const void* W, int N, int rows, int K, void* out, hipStream_t st);
// Shared expert: the grouped expert FFN run as one expert that holds every
// token (slot t = token t, weight 1); out fp32 [T, d]. Scratch from
// carve_shared (the identity dispatch plus the FFN scratch).
struct SharedScratch {
  int32_t* perm;  // [T]
  int32_t* off;   // [2]
  float* gate;    // [T]
  FfnScratch fs;
};
void carve_shared(Carver& c, int T, int d, int d_fs, int dtype, int flags, SharedScratch* s);
hipError_t launch_shared_expert(const void* x, const void* W1s, const void* b1s, const void* W2s,
                                const void* b2s, int T, int d, int d_fs, int dtype, int flags,
                                float* out, const SharedScratch& s, hipStream_t st);

}  // namespace moe
