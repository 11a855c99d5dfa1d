/*
 * moe.h - C ABI of libmoe: forward pass of one sparse Mixture-of-Experts layer
 * on an AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages define it (page "Mixture-of-Experts", beta.fermi.ai
 * wiki, "Step-by-step mechanism for one MoE layer", steps 1-7, and its
 * MoE_Layer pseudocode; page "Mixture of Experts (MoE): Architecture, Routing,
 * and Scaling", "Core Architecture"):
 *
 *   1. router logits L = x W_g (+ optional per-expert logit bias), softmax over N
 *   2. top-k experts per token                    (ties: lower expert id first)
 *   3. combine weights = top-k softmax scores renormalised to sum to 1
 *   4. capacity C per expert; at an over-full expert the lowest-scoring
 *      requests are dropped (rank: softmax probability, ties: lower token)
 *   5. dispatch: kept (token, expert) pairs grouped by expert
 *   6. each expert's FFN  o = W2 GELU(W1 x + b1) + b2     (exact erf GELU)
 *   7. combine: y[t] = sum over kept picks j of w[t,j] * o[t,j]; a dropped pick
 *      contributes zero; a token with every pick dropped gets y[t] = 0.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Return value: MOE_OK (0) or a negative MOE_ERR_* code. On error nothing
 *    has been launched. MOE_ERR_HIP means a launch failed; the HIP error code
 *    is then available from moe_last_hip_error() (per calling thread).
 *  - Every tensor pointer is a DEVICE pointer owned by the caller. The library
 *    never allocates or frees device memory and keeps no state between calls.
 *    Scratch memory comes from the caller's `workspace` (device memory of at
 *    least moe_workspace_bytes(...) bytes, 256-byte aligned). The one
 *    exception is moe_forward_noalloc, whose scratch is a static device array
 *    of MOE_NOALLOC_SCRATCH_BYTES per GPU (see there).
 *  - Inputs are never written. Outputs are fully overwritten (rows past the
 *    kept-slot count S of slot-indexed outputs are left untouched).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*; NULL = the default stream). No call synchronises and no call
 *    reads data-dependent sizes back to the host: S, the per-expert counts
 *    and the drop count stay in device memory.
 *  - Layouts are row-major and contiguous; base pointers 16-byte aligned.
 *      x      [T, d]            activation dtype
 *      W_g    [d, N]            activation dtype (router weight, L = x W_g)
 *      W1     [N, d_ff, d]      activation dtype (nn.Linear(d, d_ff) weight per expert)
 *      b1     [N, d_ff]         activation dtype, may be NULL
 *      W2     [N, d, d_ff]      activation dtype (nn.Linear(d_ff, d) weight per expert)
 *      b2     [N, d]            activation dtype, may be NULL
 *      logit_bias [N]           fp32, may be NULL
 *      y      [T, d]            activation dtype
 *      W1s    [d_fs, d], b1s [d_fs], W2s [d, d_fs], b2s [d]: a shared expert
 *                               (activation dtype; biases may be NULL)
 *    Router logits and combine weights are fp32; rank keys are fp64.
 *  - dtype: MOE_F32 (all activation tensors fp32) or MOE_BF16 (bf16 storage,
 *    fp32 accumulation).
 *  - Limits: 1 <= N <= 1024; 1 <= k <= min(N, 16); d and d_ff multiples of 8,
 *    1 <= d, d_ff <= 65536; 0 <= T and T * max(k, N) < 2^31. T = 0 is a
 *    successful no-op. Violations return MOE_ERR_INVALID_ARG or
 *    MOE_ERR_UNSUPPORTED.
 *  - capacity_factor: C = ceil(cf * k * T / N - 1e-6 * max(1, cf * k * T / N))
 *    clamped to [1, T] (capacity formula in "Communication cost in distributed
 *    settings" of the wiki page; the small guard absorbs the representation
 *    error of cf). cf <= 0 means no limit (C = T).
 *  - Results are deterministic: no floating-point atomics anywhere (integer
 *    atomics only count and hand out tiles, which does not change any value
 *    computed), so equal inputs give bit-identical outputs from run to run.
 *  - Thread safety: concurrent calls are safe when they use distinct
 *    workspaces and outputs. Calls that share a workspace must be ordered on
 *    one stream.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null required pointer, bad size or limit */
#define MOE_ERR_UNSUPPORTED (-2) /* dtype, alignment or shape outside the limits */
#define MOE_ERR_WORKSPACE (-3)   /* workspace missing, too small or misaligned */
#define MOE_ERR_HIP (-4)         /* a HIP launch failed; see moe_last_hip_error() */

#define MOE_F32 0
#define MOE_BF16 1

/* flags (bitwise or; 0 = defaults). Each entry point lists the ones it honours
 * and rejects unknown bits with MOE_ERR_INVALID_ARG. */
#define MOE_FLAG_HIDDEN_SPLIT 1 /* bf16 only: carry each hidden activation h into the
                                   second GEMM as bf16(h) plus the bf16 residual
                                   h - bf16(h) (about 16 significant bits instead of
                                   8) at twice the second GEMM's matrix-core work */
#define MOE_FLAG_Y_F32 2        /* y is written as fp32 whatever `dtype` is */
/* Drop-policy variants (wiki page "Mixture-of-Experts": the MoE_Layer
 * pseudocode and the worked example's final combine). Defaults: capacity by
 * score, pre-drop weights (partial combine), y[t] = 0 for a fully dropped
 * token. */
#define MOE_FLAG_FIRST_COME 4        /* capacity keeps each expert's first C requests in
                                        token order (the pseudocode's arrival order)
                                        instead of the C highest-scoring ones */
#define MOE_FLAG_RENORM_SURVIVORS 8  /* a token that lost a pick but kept others gets its
                                        kept weights divided by their sum (the worked
                                        example: weight 1.0 on E2 for x4) */
#define MOE_FLAG_IDENTITY_FALLBACK 16 /* a token that lost every pick gets y[t] = x[t]
                                         (the pseudocode's fallback) */
/* Expert-choice routing (page "Mixture of Experts: Scaling Language Models with
 * Sparse Activation", "Expert Choice Routing"; page "Mixture of Experts (MoE):
 * Architecture, Routing, and Scaling", "Expert Choice Routing (ECR)"),
 * moe_forward only: every expert takes the C tokens with the highest softmax
 * probability p[t,e] (equal probabilities: lower token), C from the capacity
 * formula with k read as the average number of experts per token (cf <= 0:
 * C = T, every expert takes every token); the combine weight is p[t,e]; a token
 * no expert took gets 0, or x[t] with MOE_FLAG_IDENTITY_FALLBACK. Pairs are
 * indexed t*N + e: inv_opt is then [T*N], req_counts are T, n_dropped counts the
 * pairs not taken. Not combinable with FIRST_COME / RENORM_SURVIVORS or a
 * topk_idx_opt output. */
#define MOE_FLAG_EXPERT_CHOICE 32
/* W1 and W2 (moe_forward, moe_forward_noalloc, moe_expert_ffn) are in the
 * packed layout written by moe_pack_weights. bf16 only, d and d_ff multiples
 * of 128; else MOE_ERR_UNSUPPORTED. The results are bit-identical to the same
 * call with the unpacked weights: only the order of the bytes in memory
 * changes, so that the expert GEMMs read each weight tile stage as one
 * contiguous kilobyte instead of 64 bytes from each of 16 rows. */
#define MOE_FLAG_PACKED_WEIGHTS 64

/* Library ABI version (major*100 + minor). */
int moe_version(void);

/* Human-readable text of a status code (static string). */
const char* moe_strerror(int status);

/* HIP error code (hipError_t as int) of the last failed launch on this thread. */
int moe_last_hip_error(void);

/* Expert capacity C for T tokens, N experts, top-k and capacity factor cf
 * (formula above). Returns 0 for T = 0, a negative MOE_ERR_* code for bad
 * arguments. Wiki page, "Communication cost in distributed settings". */
int moe_capacity(int T, int N, int k, double capacity_factor);

/* Device workspace, in bytes, that is enough for any entry point below called
 * with these sizes and any flags (256-byte aligned pieces are carved from it).
 * Returns 0 on invalid arguments. */
size_t moe_workspace_bytes(int T, int d, int d_ff, int N, int k, double capacity_factor, int dtype);

/* Device workspace, in bytes, that is enough for moe_shared_expert with these
 * sizes and any flags. Returns 0 on invalid arguments. */
size_t moe_shared_workspace_bytes(int T, int d, int d_fs, int dtype);

/* Shared expert (page "Mixture of Experts: Scaling Language Models with Sparse
 * Activation", "Comparing MoE Architectures": shared experts that see every
 * token next to the sparsely activated routed ones; page "Mixture of Experts
 * (MoE): Architecture, Routing, and Scaling", "Expert Choice Routing (ECR)":
 * tokens no expert took are still processed by a shared expert). The same FFN as step 6 with its own weights,
 * applied to every token with weight 1:
 *   in : x [T,d]; W1s [d_fs,d], b1s [d_fs] or NULL, W2s [d,d_fs], b2s [d] or NULL
 *   out: out [T,d] fp32, out[t] = W2s GELU(W1s x[t] + b1s) + b2s (hidden
 *        activations rounded to the activation dtype, as in moe_expert_ffn)
 * Pass `out` as shared_out to moe_combine / moe_forward to add it to the
 * routed output before y is rounded. d_fs follows d_ff's limits. flags:
 * MOE_FLAG_HIDDEN_SPLIT (bf16). Needs workspace of
 * moe_shared_workspace_bytes(...) bytes; records no profiling events. */
int moe_shared_expert(const void* x, const void* W1s, const void* b1s, const void* W2s,
                      const void* b2s, int T, int d, int d_fs, int dtype, int flags, float* out,
                      void* workspace, size_t ws_bytes, void* stream);

/* Steps 1-3 (wiki page, steps 1-3; "Inside the Router" on the corecocept page
 * for keeping logits at higher precision).
 *   in : x [T,d], W_g [d,N], logit_bias [N] fp32 or NULL
 *   out: logits   [T,N] fp32, L = x W_g + bias (fp32 accumulation)
 *        topk_idx [T,k] int32, expert ids in descending logit order,
 *                 equal logits ordered by lower expert id
 *        topk_w   [T,k] fp32, renormalised softmax scores, sum_j = 1
 *        topk_key [T,k] fp64, log softmax probability L[t,e] - logsumexp_t(L)
 *                 computed in fp64 from the fp32 logits (the capacity rank)
 * Needs workspace for bf16 (a transposed copy of W_g, or for T <= 64 and
 * N <= 64 the fp32 partial logits of a K split, at most the same size;
 * moe_workspace_bytes is enough); fp32 needs none (workspace may be NULL). */
int moe_route(const void* x, const void* W_g, const float* logit_bias,
              int T, int d, int N, int k, int dtype,
              float* logits, int32_t* topk_idx, float* topk_w, double* topk_key,
              void* workspace, size_t ws_bytes, void* stream);

/* Forward routing statistics (wiki page, step 8 and "The load-balancing
 * auxiliary loss"; page "Mixture of Experts (MoE): Architecture, Routing, and
 * Scaling", "Auxiliary Load Balancing Loss" and "Importance Loss and Z-Loss").
 *   in : logits [T,N] fp32 and topk_idx [T,k] as produced by moe_route
 *   out: stats [2N + 2] fp32:
 *          stats[e]       f_e, share of the T*k top-k picks (before capacity)
 *                         that chose expert e (sums to 1; the k-hot mask averaged
 *                         over tokens, as in some pages' code, is k * f_e)
 *          stats[N + e]   P_e, mean over tokens of the softmax probability of e
 *          stats[2N]      N * sum_e f_e * P_e (the load-balancing loss without its
 *                         coefficient; 1 when routing is uniform)
 *          stats[2N + 1]  mean over tokens of logsumexp_t(L)^2 (the router
 *                         z-loss without its coefficient)
 * Evaluated in fp64 with fixed-order sums (bit-reproducible). Needs workspace
 * (moe_workspace_bytes is enough). */
int moe_routing_stats(const float* logits, const int32_t* topk_idx, int T, int N, int k,
                      float* stats, void* workspace, size_t ws_bytes, void* stream);

/* Steps 4-5 (wiki page, steps 4-5 and the capacity-constrained dispatch of
 * its pseudocode; worked example with N=4, k=2, T=5, C=2).
 * Pair index p = t*k + j names token t's j-th pick.
 *   in : topk_idx, topk_w, topk_key as produced by moe_route
 *   out: req_counts [N]   requests per expert before capacity
 *        counts     [N]   kept pairs per expert = min(req_counts, C)
 *        offsets    [N+1] exclusive scan of counts; S = offsets[N]
 *        perm       [T*k] slot -> pair index; slots grouped by expert
 *                         ascending, tokens ascending inside an expert;
 *                         first S entries valid
 *        inv        [T*k] pair -> slot, or -1 when the pair was dropped
 *        slot_gate  [T*k] combine weight topk_w of each slot; first S valid
 *        n_dropped  [1]   T*k - S
 * At an expert with more than C requests the C pairs with the largest key
 * are kept (equal keys: lower token first).
 * flags: MOE_FLAG_FIRST_COME (keep the first C requests in token order; the
 * keys are then not read) and MOE_FLAG_RENORM_SURVIVORS (slot_gate of a token
 * that lost a pick = its topk_w / sum of its kept topk_w, in fp32, kept picks
 * summed in pick order) are honoured. Needs workspace. */
int moe_dispatch(const int32_t* topk_idx, const float* topk_w, const double* topk_key,
                 int T, int N, int k, double capacity_factor, int flags,
                 int32_t* req_counts, int32_t* counts, int32_t* offsets,
                 int32_t* perm, int32_t* inv, float* slot_gate, int32_t* n_dropped,
                 void* workspace, size_t ws_bytes, void* stream);

/* Step 6 with the gate of step 7 folded in (page "Mixture of Experts (MoE):
 * Architecture, Routing, and Scaling", "Core Architecture": FFN(x) =
 * W2 GELU(W1 x + b1) + b2).
 *   in : x [T,d]; perm, offsets, slot_gate from moe_dispatch; W1, b1, W2, b2
 *   out: slot_out [T*k, d] fp32 (either dtype); for each slot s < S of expert
 *        e and token t = perm[s] / k:
 *          slot_out[s] = slot_gate[s] * (W2[e] GELU(W1[e] x[t] + b1[e]) + b2[e])
 *        (hidden activations are rounded to the activation dtype; the
 *        gate-scaled outputs stay fp32 so that only y is rounded once more).
 * flags: MOE_FLAG_HIDDEN_SPLIT (bf16) and MOE_FLAG_PACKED_WEIGHTS are honoured;
 * MOE_FLAG_Y_F32 has no effect here. T, k, capacity_factor bound S (S <= min(T*k, N*C)) for launch
 * sizing: perm, offsets and slot_gate must come from moe_dispatch called with
 * the same T, N, k and capacity_factor. With other offsets the kernels clamp
 * each expert's rows to C and all rows to min(T*k, N*C), so every access
 * stays inside the buffers, but the rows past those bounds are not computed
 * (their slot_out rows are left as they were). Needs workspace (the hidden
 * activations live there). */
int moe_expert_ffn(const void* x, const int32_t* perm, const int32_t* offsets,
                   const float* slot_gate,
                   const void* W1, const void* b1, const void* W2, const void* b2,
                   int T, int d, int d_ff, int N, int k, double capacity_factor, int dtype,
                   int flags, void* slot_out, void* workspace, size_t ws_bytes, void* stream);

/* Expert weights in the packed layout of MOE_FLAG_PACKED_WEIGHTS, written once
 * (at load time) and then passed to the FFN entry points with that flag. The
 * operation is a reordering only (no arithmetic; the pages' FFN of page "Mixture
 * of Experts (MoE): Architecture, Routing, and Scaling", "Core Architecture",
 * is unchanged).
 *   in : W [N, rows, K] bf16, row-major (W1: rows = d_ff, K = d; W2: rows = d,
 *        K = d_ff), 16-byte aligned
 *   out: W_packed, the same N*rows*K*2 bytes, caller-owned, 16-byte aligned,
 *        not overlapping W: for each expert e, row block rb (16 rows) and K
 *        chunk kc (32 values) a 1 KB piece at byte
 *        ((e*rows/16 + rb)*K/32 + kc)*1024 whose 16-byte word w holds the 8
 *        values W[e][rb*16 + r(w)][kc*32 + 8*c(w) ..+8], with h = w/16,
 *        g = (w/4)%4, r(w) = (g%2) + 2*h + 8*(g/2) and c(w) = (w%4) ^ h.
 * dtype must be MOE_BF16, rows % 16 == 0 and K % 128 == 0
 * (MOE_ERR_UNSUPPORTED otherwise). Asynchronous on `stream`; no workspace. */
int moe_pack_weights(const void* W, int N, int rows, int K, int dtype, void* W_packed,
                     void* stream);

/* Step 7 (wiki page, step 7; weighted combine of the pseudocode).
 *   in : slot_out [T*k, d] fp32 (already gate-scaled), inv [T*k]; x [T,d] in
 *        `dtype` (read only with MOE_FLAG_IDENTITY_FALLBACK, else may be NULL);
 *        shared_out [T,d] fp32 from moe_shared_expert, or NULL
 *   out: y [T,d] in `dtype` (fp32 with MOE_FLAG_Y_F32), y[t] = sum over
 *        j = 0..k-1 with inv[t*k+j] >= 0 of slot_out[inv[t*k+j]], summed in
 *        fp32 in increasing j; for a token with no kept pick 0, or x[t] with
 *        MOE_FLAG_IDENTITY_FALLBACK; then + shared_out[t] when given (fp32),
 *        and one rounding to y's dtype.
 * flags: MOE_FLAG_Y_F32, MOE_FLAG_IDENTITY_FALLBACK. Needs no workspace. */
int moe_combine(const void* slot_out, const int32_t* inv, const void* x, const float* shared_out,
                int T, int d, int k, int dtype, int flags, void* y, void* stream);

/* Whole layer, steps 1-7, as one enqueue of the calls above on `stream`.
 *   out: y [T,d] (required) in `dtype`, or fp32 with MOE_FLAG_Y_F32; optional
 *        copies of intermediate results, each NULL to skip: logits_opt [T,N]
 *        fp32, topk_idx_opt [T,k], inv_opt [T*k], req_counts_opt [N],
 *        counts_opt [N], n_dropped_opt [1].
 *   in : shared_out [T,d] fp32 (moe_shared_expert's output) or NULL: added
 *        to every token in the combine, as in moe_combine.
 * flags: every MOE_FLAG_* above (unknown bits: MOE_ERR_INVALID_ARG).
 * Needs workspace of moe_workspace_bytes(...) bytes. */
int moe_forward(const void* x, const void* W_g, const float* logit_bias,
                const void* W1, const void* b1, const void* W2, const void* b2,
                int T, int d, int d_ff, int N, int k, double capacity_factor, int dtype,
                int flags, const float* shared_out, void* y,
                float* logits_opt, int32_t* topk_idx_opt, int32_t* inv_opt,
                int32_t* req_counts_opt, int32_t* counts_opt, int32_t* n_dropped_opt,
                void* workspace, size_t ws_bytes, void* stream);

/* Size of the static per-GPU scratch array behind moe_forward_noalloc: 64 MiB. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results, flags and errors are those of moe_forward without
 * `workspace` / `ws_bytes`; the same kernels run and give the same bits.
 * Scratch: one static device array of MOE_NOALLOC_SCRATCH_BYTES per GPU,
 * reserved when the library's code is loaded on that GPU and held until the
 * process ends; its address on the current device is looked up on the first
 * call there (make that first call outside graph capture, as the first
 * moe_forward of a shape should be) and cached. Nothing is allocated or freed
 * (no hipMalloc, hipFree or allocating library call) by this entry point.
 * Limit: a call whose moe_forward workspace for these sizes and flags
 * (moe_workspace_bytes gives an upper bound) exceeds the array returns
 * MOE_ERR_WORKSPACE before any launch; decode-sized calls fit (for example
 * 32 tokens of the Mixtral-shaped layer, d = 4096, d_ff = 14336, N = 8,
 * top-2, with any flags).
 * Every call on one GPU uses that GPU's one array, which keeps the last call's
 * contents; no part of it needs to start at zero (every kernel writes what it
 * later reads, and the work-queue counters are zeroed by the launch sequence).
 * Calls that overlap on one GPU (other streams, or other host threads, without
 * ordering between them) race on the array and give wrong results: order them
 * on one stream. */
int moe_forward_noalloc(const void* x, const void* W_g, const float* logit_bias,
                        const void* W1, const void* b1, const void* W2, const void* b2,
                        int T, int d, int d_ff, int N, int k, double capacity_factor, int dtype,
                        int flags, const float* shared_out, void* y,
                        float* logits_opt, int32_t* topk_idx_opt, int32_t* inv_opt,
                        int32_t* req_counts_opt, int32_t* counts_opt, int32_t* n_dropped_opt,
                        void* stream);

/* Instrumentation for timing (not part of the layer): registers up to 7
 * hipEvent_t handles (as void*, entries may be NULL) for the calling thread;
 * n = 0 clears. While registered, moe_forward records event i on its stream
 * at these points of its launch sequence: 0 before the router, 1 after the
 * router, 2 after dispatch, 3 before the first expert GEMM, 4 after it,
 * 5 after the second expert GEMM, 6 after the combine (moe_expert_ffn alone
 * records 3-5). The caller owns the events. Returns MOE_ERR_INVALID_ARG for
 * n outside [0, 7] or a NULL array with n > 0. */
int moe_set_profile_events(void* const* events, int n);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
