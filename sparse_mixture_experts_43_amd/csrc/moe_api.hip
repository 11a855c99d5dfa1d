// C ABI of libmoe: argument checks, workspace carving and the launch sequence
// of the MoE layer forward (declarations and contracts in include/moe.h).
#include "../../include/moe.h"
#include "moe_common.h"

#include <math.h>

#include <mutex>

namespace moe {

static thread_local int g_last_hip = 0;
constexpr int kProfileSlots = 7;
static thread_local void* g_prof[kProfileSlots] = {};

void profile_mark(int slot, hipStream_t st) {
  if (slot >= 0 && slot < kProfileSlots && g_prof[slot] != nullptr)
    hipEventRecord((hipEvent_t)g_prof[slot], st);
}

int capacity_host(int T, int N, int k, double cf) {
  if (T <= 0) return 0;
  if (!(cf > 0.0)) return T;  // no limit
  const double c = cf * (double)k * (double)T / (double)N;
  double g = c - 1e-6 * (c > 1.0 ? c : 1.0);
  double ci = ceil(g);
  if (ci < 1.0) ci = 1.0;
  if (ci > (double)T) ci = (double)T;
  return (int)ci;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static int check_shape(int T, int d, int d_ff, int N, int k, int dtype, bool need_dff) {
  if (T < 0 || N < 1 || N > kMaxN || k < 1 || k > N || k > kMaxK) return MOE_ERR_INVALID_ARG;
  if (d < 8 || d > 65536 || (d % 8) != 0) return MOE_ERR_UNSUPPORTED;
  if (need_dff && (d_ff < 8 || d_ff > 65536 || (d_ff % 8) != 0)) return MOE_ERR_UNSUPPORTED;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const long long big = (long long)T * (long long)(k > N ? k : N);
  if (big >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip = (int)e;
  return MOE_ERR_HIP;
}

// Pieces of the moe_forward workspace.
struct ForwardWs {
  float* logits;
  int32_t* idx;
  float* w;
  double* key;
  int32_t *req, *cnt, *off, *ndrop;
  int32_t *perm, *inv;
  float* gate;
  void* slot_out;
  void* wgt;  // transposed router weight
  DispatchScratch ds;
  FfnScratch fs;
  size_t bytes;
};

static void carve_forward(void* base, int T, int d, int d_ff, int N, int k, int C, int dtype,
                          int flags, ForwardWs* f) {
  Carver c(base);
  const size_t P = (size_t)(T > 0 ? T : 1) * k;
  const int S_max = (int)((long long)T * k < (long long)N * C ? (long long)T * k : (long long)N * C);
  f->logits = c.take<float>((size_t)(T > 0 ? T : 1) * N);
  f->idx = c.take<int32_t>(P);
  f->w = c.take<float>(P);
  f->key = c.take<double>(P);
  f->req = c.take<int32_t>(N);
  f->cnt = c.take<int32_t>(N);
  f->off = c.take<int32_t>((size_t)N + 1);
  f->ndrop = c.take<int32_t>(1);
  f->perm = c.take<int32_t>(P);
  f->inv = c.take<int32_t>(P);
  f->gate = c.take<float>(P);
  f->slot_out = c.take<float>((size_t)(S_max > 0 ? S_max : 1) * d);
  f->wgt = c.take<unsigned char>(route_scratch_bytes(d, N, dtype));
  carve_dispatch(c, T * k, N, &f->ds);
  carve_ffn(c, T, d, d_ff, N, k, C, S_max, dtype, flags, &f->fs);
  f->bytes = align_up(c.off, 256);
}

static size_t dispatch_bytes(int T, int N, int k) {
  Carver c(nullptr);
  DispatchScratch ds;
  carve_dispatch(c, T * k, N, &ds);
  return align_up(c.off, 256);
}

static size_t shared_bytes(int T, int d, int d_fs, int dtype, int flags) {
  Carver c(nullptr);
  SharedScratch ss;
  carve_shared(c, T, d, d_fs, dtype, flags, &ss);
  return align_up(c.off, 256);
}

static size_t ffn_bytes(int T, int d, int d_ff, int N, int k, int C, int dtype, int flags) {
  Carver c(nullptr);
  FfnScratch fs;
  const int S_max = (int)((long long)T * k < (long long)N * C ? (long long)T * k : (long long)N * C);
  carve_ffn(c, T, d, d_ff, N, k, C, S_max, dtype, flags, &fs);
  return align_up(c.off, 256);
}

// ---------------------------------------------------------------- no-alloc scratch
// Scratch of moe_forward_noalloc: one static device array, which each GPU the
// library's code is loaded on holds until the process ends. In host code the
// array's name is not a device address: its address on the current device
// comes from hipGetSymbolAddress, looked up once per device and cached; only
// that address is ever handed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_status(e != hipSuccess ? e : hipErrorUnknown);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// MOE_FLAG_PACKED_WEIGHTS: bf16 experts with d and d_ff multiples of 128
// (every expert GEMM path then reads the piece layout).
static int check_packed(int flags, int d, int d_ff, int dtype) {
  if (!(flags & MOE_FLAG_PACKED_WEIGHTS)) return MOE_OK;
  return dtype == MOE_BF16 && d % 128 == 0 && d_ff % 128 == 0 ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

// The layer forward behind moe_forward (caller workspace) and
// moe_forward_noalloc (noalloc: the device's static scratch array, whose
// address replaces workspace once the sizes are known to fit).
static int forward_impl(const void* x, const void* W_g, const float* logit_bias, const void* W1,
                        const void* b1, const void* W2, const void* b2, int T, int d, int d_ff,
                        int N, int k, double capacity_factor, int dtype, int flags,
                        const float* shared_out, void* y, float* logits_opt,
                        int32_t* topk_idx_opt, int32_t* inv_opt, int32_t* req_counts_opt,
                        int32_t* counts_opt, int32_t* n_dropped_opt, void* workspace,
                        size_t ws_bytes, void* stream, bool noalloc) {
  int st = check_shape(T, d, d_ff, N, k, dtype, true);
  if (st != MOE_OK) return st;
  if (isnan(capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (flags & ~(MOE_FLAG_HIDDEN_SPLIT | MOE_FLAG_Y_F32 | MOE_FLAG_FIRST_COME |
                MOE_FLAG_RENORM_SURVIVORS | MOE_FLAG_IDENTITY_FALLBACK | MOE_FLAG_EXPERT_CHOICE |
                MOE_FLAG_PACKED_WEIGHTS))
    return MOE_ERR_INVALID_ARG;
  st = check_packed(flags, d, d_ff, dtype);
  if (st != MOE_OK) return st;
  const bool ec = (flags & MOE_FLAG_EXPERT_CHOICE) != 0;
  if (ec && ((flags & (MOE_FLAG_FIRST_COME | MOE_FLAG_RENORM_SURVIVORS)) || topk_idx_opt))
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !W_g || !W1 || !W2 || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(W_g, 16) || !aligned(W1, 16) || !aligned(W2, 16) ||
      !aligned(y, 16) || (b1 && !aligned(b1, 16)) || (b2 && !aligned(b2, 16)) ||
      (logit_bias && !aligned(logit_bias, 4)) || (logits_opt && !aligned(logits_opt, 4)) ||
      (shared_out && !aligned(shared_out, 16)))
    return MOE_ERR_UNSUPPORTED;
  const int C = capacity_host(T, N, k, capacity_factor);
  // pairs per token: k picks, or with expert choice every expert (pair t*N + e)
  const int kp = ec ? N : k;
  ForwardWs f;
  carve_forward(nullptr, T, d, d_ff, N, kp, C, dtype, flags, &f);
  if (noalloc) {
    if (f.bytes > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
    const int ss = noalloc_scratch(&workspace);
    if (ss != MOE_OK) return ss;
    ws_bytes = kNoAllocScratchBytes;
  }
  if (!workspace || !aligned(workspace, 256) || ws_bytes < f.bytes) return MOE_ERR_WORKSPACE;
  carve_forward(workspace, T, d, d_ff, N, kp, C, dtype, flags, &f);
  if (logits_opt) f.logits = logits_opt;
  if (topk_idx_opt) f.idx = topk_idx_opt;
  if (inv_opt) f.inv = inv_opt;
  if (req_counts_opt) f.req = req_counts_opt;
  if (counts_opt) f.cnt = counts_opt;
  if (n_dropped_opt) f.ndrop = n_dropped_opt;
  const int S_max =
      (int)((long long)T * kp < (long long)N * C ? (long long)T * kp : (long long)N * C);
  hipStream_t s = (hipStream_t)stream;
  profile_mark(0, s);
  // expert choice: the router's logits (its top-1 outputs are scratch), then
  // every pair as a candidate
  // few tokens: the split-K router leaves partial logits, and the dispatch
  // block adds them and runs the top-k (one launch fewer)
  RoutePartials rp;
  hipError_t e = ec ? hipSuccess
                    : launch_route_partials(x, W_g, logit_bias, T, d, N, dtype, f.logits, f.idx,
                                            f.w, f.key, f.wgt, s, &rp);
  if (e == hipSuccess && rp.part == nullptr)
    e = launch_route(x, W_g, logit_bias, T, d, N, ec ? 1 : k, dtype, f.logits, f.idx, f.w, f.key,
                     f.wgt, s);
  if (e == hipSuccess && ec) e = launch_route_expert_choice(f.logits, T, N, f.idx, f.w, f.key, s);
  if (e != hipSuccess) return hip_status(e);
  profile_mark(1, s);
  e = launch_dispatch(f.idx, f.w, f.key, T, N, kp, C, flags, f.req, f.cnt, f.off, f.perm, f.inv,
                      f.gate, f.ndrop, f.ds, s, rp.part != nullptr ? &rp : nullptr);
  if (e != hipSuccess) return hip_status(e);
  profile_mark(2, s);
  SplitK sk;  // a K-split second GEMM hands its partials straight to the combine
  const int y_dtype = (flags & MOE_FLAG_Y_F32) ? MOE_F32 : dtype;
  const void* xf = (flags & MOE_FLAG_IDENTITY_FALLBACK) ? x : nullptr;
  // A token that kept exactly one pick outputs that pick's gate-scaled row,
  // unless the identity fallback or a shared expert adds to it: then the
  // second expert GEMM may write the row into y itself (DirectRows).
  DirectRows dr;
  if (!ec && xf == nullptr && shared_out == nullptr) {
    dr.y = y;
    dr.y_dtype = y_dtype;
    dr.inv = f.inv;
  }
  e = launch_expert_ffn(x, f.perm, f.off, f.gate, W1, b1, W2, b2, T, d, d_ff, N, kp, C, S_max,
                        dtype, flags, f.slot_out, f.fs, s, &sk, &dr);
  if (e != hipSuccess) return hip_status(e);
  e = sk.nsplit > 1
          ? launch_combine_splitk(sk, f.inv, T, d, kp, y_dtype, xf, dtype, shared_out, y, s)
          : launch_combine(f.slot_out, f.inv, T, d, kp, y_dtype, xf, dtype, shared_out, y, s,
                           dr.used);
  profile_mark(6, s);
  return hip_status(e);
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_version(void) { return 103; }

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (null pointer, size or limit)";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype, alignment or shape";
    case MOE_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case MOE_ERR_HIP: return "HIP launch failed (see moe_last_hip_error)";
    default: return "unknown status";
  }
}

int moe_last_hip_error(void) { return g_last_hip; }

int moe_set_profile_events(void* const* events, int n) {
  if (n < 0 || n > kProfileSlots || (n > 0 && events == nullptr)) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < kProfileSlots; ++i) g_prof[i] = (i < n) ? events[i] : nullptr;
  return MOE_OK;
}

int moe_capacity(int T, int N, int k, double capacity_factor) {
  if (T < 0 || N < 1 || k < 1 || k > N || isnan(capacity_factor)) return MOE_ERR_INVALID_ARG;
  return capacity_host(T, N, k, capacity_factor);
}

size_t moe_workspace_bytes(int T, int d, int d_ff, int N, int k, double capacity_factor,
                           int dtype) {
  if (check_shape(T, d, d_ff, N, k, dtype, true) != MOE_OK || isnan(capacity_factor)) return 0;
  // enough for every flag combination (the plans with and without the split
  // hidden layer differ in tiling and scratch)
  const int C = capacity_host(T, N, k, capacity_factor);
  ForwardWs f, g;
  carve_forward(nullptr, T, d, d_ff, N, k, C, dtype, MOE_FLAG_HIDDEN_SPLIT | MOE_FLAG_Y_F32, &f);
  carve_forward(nullptr, T, d, d_ff, N, k, C, dtype, MOE_FLAG_Y_F32, &g);
  size_t b = f.bytes > g.bytes ? f.bytes : g.bytes;
  // expert choice: every (token, expert) pair is a candidate
  ForwardWs ec;
  carve_forward(nullptr, T, d, d_ff, N, N, C, dtype, MOE_FLAG_HIDDEN_SPLIT | MOE_FLAG_Y_F32, &ec);
  b = b > ec.bytes ? b : ec.bytes;
  const size_t sb = align_up(stats_scratch_bytes(T, N), 256);  // moe_routing_stats
  return b > sb ? b : sb;
}

size_t moe_shared_workspace_bytes(int T, int d, int d_fs, int dtype) {
  if (check_shape(T, d, d_fs, 1, 1, dtype, true) != MOE_OK) return 0;
  const size_t a = shared_bytes(T, d, d_fs, dtype, MOE_FLAG_HIDDEN_SPLIT);
  const size_t b = shared_bytes(T, d, d_fs, dtype, 0);
  return a > b ? a : b;
}

int moe_shared_expert(const void* x, const void* W1s, const void* b1s, const void* W2s,
                      const void* b2s, int T, int d, int d_fs, int dtype, int flags, float* out,
                      void* workspace, size_t ws_bytes, void* stream) {
  int st = check_shape(T, d, d_fs, 1, 1, dtype, true);
  if (st != MOE_OK) return st;
  if (flags & ~MOE_FLAG_HIDDEN_SPLIT) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !W1s || !W2s || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(W1s, 16) || !aligned(W2s, 16) || !aligned(out, 16) ||
      (b1s && !aligned(b1s, 16)) || (b2s && !aligned(b2s, 16)))
    return MOE_ERR_UNSUPPORTED;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < shared_bytes(T, d, d_fs, dtype, flags))
    return MOE_ERR_WORKSPACE;
  Carver c(workspace);
  SharedScratch ss;
  carve_shared(c, T, d, d_fs, dtype, flags, &ss);
  // the expert FFN's profiling marks belong to moe_forward's sequence
  void* saved[kProfileSlots];
  for (int i = 0; i < kProfileSlots; ++i) {
    saved[i] = g_prof[i];
    g_prof[i] = nullptr;
  }
  const hipError_t e = launch_shared_expert(x, W1s, b1s, W2s, b2s, T, d, d_fs, dtype, flags, out,
                                            ss, (hipStream_t)stream);
  for (int i = 0; i < kProfileSlots; ++i) g_prof[i] = saved[i];
  return hip_status(e);
}

int moe_route(const void* x, const void* W_g, const float* logit_bias, int T, int d, int N, int k,
              int dtype, float* logits, int32_t* topk_idx, float* topk_w, double* topk_key,
              void* workspace, size_t ws_bytes, void* stream) {
  int st = check_shape(T, d, 8, N, k, dtype, false);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !W_g || !logits || !topk_idx || !topk_w || !topk_key) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(W_g, 16) || !aligned(logits, 4) || !aligned(topk_idx, 4) ||
      !aligned(topk_w, 4) || !aligned(topk_key, 8) || (logit_bias && !aligned(logit_bias, 4)))
    return MOE_ERR_UNSUPPORTED;
  const size_t need = route_scratch_bytes(d, N, dtype);
  if (need > 0 && (!workspace || !aligned(workspace, 256) || ws_bytes < need))
    return MOE_ERR_WORKSPACE;
  return hip_status(launch_route(x, W_g, logit_bias, T, d, N, k, dtype, logits, topk_idx, topk_w,
                                 topk_key, workspace, (hipStream_t)stream));
}

int moe_routing_stats(const float* logits, const int32_t* topk_idx, int T, int N, int k,
                      float* stats, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_shape(T, 8, 8, N, k, MOE_F32, false);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !stats) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(stats, 4))
    return MOE_ERR_UNSUPPORTED;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < stats_scratch_bytes(T, N))
    return MOE_ERR_WORKSPACE;
  return hip_status(launch_routing_stats(logits, topk_idx, T, N, k, stats, workspace,
                                         (hipStream_t)stream));
}

int moe_dispatch(const int32_t* topk_idx, const float* topk_w, const double* topk_key, int T,
                 int N, int k, double capacity_factor, int flags, int32_t* req_counts,
                 int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, float* slot_gate,
                 int32_t* n_dropped, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_shape(T, 8, 8, N, k, MOE_F32, false);
  if (st != MOE_OK) return st;
  if (isnan(capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (flags & ~(MOE_FLAG_FIRST_COME | MOE_FLAG_RENORM_SURVIVORS)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !topk_w || (!topk_key && !(flags & MOE_FLAG_FIRST_COME)) || !req_counts ||
      !counts || !offsets || !perm || !inv || !slot_gate || !n_dropped)
    return MOE_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256) || ws_bytes < dispatch_bytes(T, N, k))
    return MOE_ERR_WORKSPACE;
  const int C = capacity_host(T, N, k, capacity_factor);
  Carver c(workspace);
  DispatchScratch ds;
  carve_dispatch(c, T * k, N, &ds);
  return hip_status(launch_dispatch(topk_idx, topk_w, topk_key, T, N, k, C, flags, req_counts,
                                    counts, offsets, perm, inv, slot_gate, n_dropped, ds,
                                    (hipStream_t)stream));
}

int moe_expert_ffn(const void* x, const int32_t* perm, const int32_t* offsets,
                   const float* slot_gate, const void* W1, const void* b1, const void* W2,
                   const void* b2, int T, int d, int d_ff, int N, int k, double capacity_factor,
                   int dtype, int flags, void* slot_out, void* workspace, size_t ws_bytes,
                   void* stream) {
  int st = check_shape(T, d, d_ff, N, k, dtype, true);
  if (st != MOE_OK) return st;
  if (flags & ~(MOE_FLAG_HIDDEN_SPLIT | MOE_FLAG_Y_F32 | MOE_FLAG_PACKED_WEIGHTS))
    return MOE_ERR_INVALID_ARG;
  st = check_packed(flags, d, d_ff, dtype);
  if (st != MOE_OK) return st;
  if (isnan(capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !perm || !offsets || !slot_gate || !W1 || !W2 || !slot_out) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(W1, 16) || !aligned(W2, 16) || !aligned(slot_out, 16) ||
      (b1 && !aligned(b1, 16)) || (b2 && !aligned(b2, 16)))
    return MOE_ERR_UNSUPPORTED;
  const int C = capacity_host(T, N, k, capacity_factor);
  if (!workspace || !aligned(workspace, 256) ||
      ws_bytes < ffn_bytes(T, d, d_ff, N, k, C, dtype, flags))
    return MOE_ERR_WORKSPACE;
  const int S_max = (int)((long long)T * k < (long long)N * C ? (long long)T * k : (long long)N * C);
  Carver c(workspace);
  FfnScratch fs;
  carve_ffn(c, T, d, d_ff, N, k, C, S_max, dtype, flags, &fs);
  return hip_status(launch_expert_ffn(x, perm, offsets, slot_gate, W1, b1, W2, b2, T, d, d_ff, N,
                                      k, C, S_max, dtype, flags, slot_out, fs,
                                      (hipStream_t)stream));
}

int moe_pack_weights(const void* W, int N, int rows, int K, int dtype, void* W_packed,
                     void* stream) {
  if (N < 0 || rows < 0 || K < 0 || dtype < MOE_F32 || dtype > MOE_BF16)
    return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 || rows % 16 != 0 || K % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((size_t)N * rows * K == 0) return MOE_OK;
  if (!W || !W_packed) return MOE_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(W_packed, 16)) return MOE_ERR_UNSUPPORTED;
  const size_t bytes = (size_t)N * rows * K * 2;
  const char* a = (const char*)W;
  const char* b = (const char*)W_packed;
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;  // overlapping buffers
  return hip_status(launch_pack_weights(W, N, rows, K, W_packed, (hipStream_t)stream));
}

int moe_combine(const void* slot_out, const int32_t* inv, const void* x, const float* shared_out,
                int T, int d, int k, int dtype, int flags, void* y, void* stream) {
  if (T < 0 || k < 1 || k > kMaxK || d < 8 || d > 65536 || (d % 8) != 0) {
    return (T < 0 || k < 1 || k > kMaxK) ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED;
  }
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (flags & ~(MOE_FLAG_Y_F32 | MOE_FLAG_IDENTITY_FALLBACK)) return MOE_ERR_INVALID_ARG;
  if ((long long)T * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  const bool fallback = (flags & MOE_FLAG_IDENTITY_FALLBACK) != 0;
  if (!slot_out || !inv || !y || (fallback && !x)) return MOE_ERR_INVALID_ARG;
  if (!aligned(slot_out, 16) || !aligned(y, 16) || (fallback && !aligned(x, 16)) ||
      (shared_out && !aligned(shared_out, 16)))
    return MOE_ERR_UNSUPPORTED;
  const int y_dtype = (flags & MOE_FLAG_Y_F32) ? MOE_F32 : dtype;
  return hip_status(launch_combine(slot_out, inv, T, d, k, y_dtype, fallback ? x : nullptr, dtype,
                                   shared_out, y, (hipStream_t)stream));
}

int moe_forward(const void* x, const void* W_g, const float* logit_bias, const void* W1,
                const void* b1, const void* W2, const void* b2, int T, int d, int d_ff, int N,
                int k, double capacity_factor, int dtype, int flags, const float* shared_out,
                void* y, float* logits_opt,
                int32_t* topk_idx_opt, int32_t* inv_opt, int32_t* req_counts_opt,
                int32_t* counts_opt, int32_t* n_dropped_opt, void* workspace, size_t ws_bytes,
                void* stream) {
  return forward_impl(x, W_g, logit_bias, W1, b1, W2, b2, T, d, d_ff, N, k, capacity_factor,
                      dtype, flags, shared_out, y, logits_opt, topk_idx_opt, inv_opt,
                      req_counts_opt, counts_opt, n_dropped_opt, workspace, ws_bytes, stream,
                      false);
}

int moe_forward_noalloc(const void* x, const void* W_g, const float* logit_bias, const void* W1,
                        const void* b1, const void* W2, const void* b2, int T, int d, int d_ff,
                        int N, int k, double capacity_factor, int dtype, int flags,
                        const float* shared_out, void* y, float* logits_opt,
                        int32_t* topk_idx_opt, int32_t* inv_opt, int32_t* req_counts_opt,
                        int32_t* counts_opt, int32_t* n_dropped_opt, void* stream) {
  return forward_impl(x, W_g, logit_bias, W1, b1, W2, b2, T, d, d_ff, N, k, capacity_factor,
                      dtype, flags, shared_out, y, logits_opt, topk_idx_opt, inv_opt,
                      req_counts_opt, counts_opt, n_dropped_opt, nullptr, 0, stream, true);
}

}  // extern "C"
