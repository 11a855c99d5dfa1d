"""CPU oracle for the forward pass of one sparse Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg
do. It shares no code with the HIP library.

Plain numpy in float64, evaluated on the exact values of the (bf16- or fp32-)
rounded inputs. Each function follows one step of the layer as the pages
describe it. Page names used in the citations:

  [Wiki]     "Mixture-of-Experts" (beta.fermi.ai wiki): step-by-step mechanism
             (steps 1-8), the MoE_Layer pseudocode, the capacity formula in
             "Communication cost in distributed settings", and the worked
             example (N=4, k=2, T=5, C=2).
  [Arch]     "Mixture of Experts (MoE): Architecture, Routing, and Scaling"
             (syntave.com): "Core Architecture" (FFN formula, SparseMoE
             snippet), "Expert Capacity and Capacity Factor".
  [Scaling]  "Mixture of Experts: Scaling Language Models with Sparse
             Activation" (tempatgunting.com): "Routing Mechanisms" (TopKRouter).
  [Rise]     "The Rise of Mixture-of-Experts Models" (gradflow): "The Gating
             Mechanism" (TopKRouter, MoELayer).
  [Explained] "Mixture of Experts: How Sparse Routing Scales Transformers"
             (corecocept.com): "Inside the Router".

Readings taken where the pages are silent or disagree (each is listed with its
reason in the design notes of the repository):

  R1 top-k order: experts ordered by logit descending, ties to the lower
     expert index. Softmax is strictly increasing, so choosing by logit and by
     softmax score gives the same set.
  R2 capacity C = ceil(cf*k*T/N - 1e-6*max(1, cf*k*T/N)), clamped to [1, T];
     cf <= 0 means no limit (C = T). [Wiki] capacity formula (with k).
  R3 the overflow rank at an expert is the raw softmax probability p[t,e],
     compared through the float64 log-domain key kappa = L[t,e] - lse_t;
     equal keys keep the lower token index. [Wiki] step 4 and worked example.
  R4 a dropped (token, expert) pair contributes zero; kept pairs keep their
     pre-drop combine weight (partial combine, [Wiki] pseudocode combine step).
  R5 a token whose every pick is dropped outputs 0 (the residual belongs to
     the enclosing block).
  R6 GELU is the exact erf form (nn.GELU default in [Arch] and [Rise]).
  R7 slots are ordered by expert ascending, tokens ascending inside an expert
     (the append order of the [Wiki] pseudocode).
  R15 routing statistics: f_e = share of the T*k top-k picks (before capacity)
     that chose expert e, so sum_e f_e = 1 ([Wiki] normalisation; the code of
     [Scaling] and [Rise] averages the k-hot mask over tokens, which is k*f_e);
     P_e = mean over tokens of the full softmax probability; aux = N * sum_e
     f_e P_e without the training coefficient (1 at uniform routing); z = mean
     over tokens of lse_t^2 without its coefficient.
  R16 drop-policy variants, each off by default: (a) first-come capacity keeps
     each expert's first C requests in token order (the arrival order of the
     [Wiki] pseudocode's dispatch loop); (b) survivor renormalisation divides a
     token's kept weights by their sum when it lost a pick ([Wiki] worked
     example: weight 1.0 on E2's output for x4); (c) identity fallback gives a
     token that lost every pick y[t] = x[t] (the [Wiki] pseudocode's fallback).
  R17 expert-choice routing: every expert takes the C tokens with the highest
     softmax probability p[t,e] (equal probabilities: lower token), C from the
     capacity formula with k read as the average number of experts per token
     (cf <= 0: every token, C = T); the combine weight is p[t,e] itself; a token
     no expert took gets 0 (or x[t] with the identity fallback). [Scaling]
     "Expert Choice Routing", [Arch] "Expert Choice Routing (ECR)".
  R18 shared expert: an always-on FFN of its own weights, applied to every
     token with weight 1 and added to the routed output (after the identity
     fallback, which replaces only the routed part). [Scaling] "Comparing MoE
     Architectures" (shared experts that see every token next to sparsely
     activated routed ones), [Arch]
     "Expert Choice Routing (ECR)" (unselected tokens processed by a shared
     expert).

Every function here is pinned by tests under tests/ against facts the pages
or the mathematics fix (see tests/test_oracle_pins.py). The bf16 rounding of
the GPU path's intermediates is not modelled: it is covered by tolerance only
(parity unpinned for that rounding path).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np
import torch

__all__ = [
    "to_f64",
    "router_logits",
    "route_topk",
    "capacity",
    "capacity_dispatch",
    "gelu",
    "expert_ffn_rows",
    "expert_slots_out",
    "combine",
    "moe_forward",
    "Routing",
    "Dispatch",
    "RoutingStats",
    "routing_stats",
    "renormalise_survivors",
    "expert_choice_dispatch",
    "moe_forward_expert_choice",
    "shared_expert_out",
]


def to_f64(t) -> Optional[np.ndarray]:
    """Exact float64 copy of a CPU tensor / array (bf16 and fp32 widen exactly)."""
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


# --------------------------------------------------------------------------
# Step 1: router logits.  [Wiki] step 1 (logits = X W_g, W_g in R^{d x N});
# [Arch] "Core Architecture" (router is a linear layer d_model x E).
# The optional per-expert logit bias is part of the synthetic workloads.
# --------------------------------------------------------------------------
def router_logits(x, W_g, logit_bias=None) -> np.ndarray:
    X = to_f64(x)
    W = to_f64(W_g)
    L = X @ W
    if logit_bias is not None:
        L = L + to_f64(logit_bias)[None, :]
    return L


@dataclass
class Routing:
    idx: np.ndarray  # [T, k] int32, experts in descending logit order
    w: np.ndarray  # [T, k] float64, renormalised combine weights
    key: np.ndarray  # [T, k] float64, kappa = L[t, idx] - lse_t = log p[t, idx]
    probs: np.ndarray  # [T, N] float64, full softmax
    lse: np.ndarray  # [T] float64


# --------------------------------------------------------------------------
# Steps 1-3: softmax over N, top-k, renormalise over the selected k.
# [Wiki] steps 1-3 and the routing loop of the pseudocode; [Arch] SparseMoE
# forward (softmax, topk, divide by the sum); [Explained] "Inside the Router".
# --------------------------------------------------------------------------
def route_topk(L, k: int) -> Routing:
    L = np.asarray(L, dtype=np.float64)
    if L.ndim != 2:
        raise ValueError("logits must be [T, N]")
    T, N = L.shape
    if not (1 <= k <= N):
        raise ValueError("need 1 <= k <= N")
    if not np.all(np.isfinite(L)):
        raise ValueError("non-finite logits are outside the method's domain")
    # R1: stable sort of -L keeps equal logits in ascending expert order.
    order = np.argsort(-L, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    m = L.max(axis=1)
    ex = np.exp(L - m[:, None])
    s = ex.sum(axis=1)
    probs = ex / s[:, None]
    lse = m + np.log(s)
    rows = np.arange(T)[:, None]
    p_sel = probs[rows, idx]
    w = p_sel / p_sel.sum(axis=1, keepdims=True)
    key = L[rows, idx] - lse[:, None]
    return Routing(idx=idx, w=w, key=key, probs=probs, lse=lse)


# --------------------------------------------------------------------------
# Forward routing statistics: [Wiki] step 8 and "The load-balancing auxiliary
# loss" (f_e, P_e, N * sum f_e P_e, minimum 1 when f = P = 1/N); [Arch]
# "Auxiliary Load Balancing Loss" and "Importance Loss and Z-Loss" (z-loss over
# the tokens' log-sum-exp); [Scaling] "Training Dynamics and Stability" (z-loss
# as the batch mean of the squared log-sum-exp).  Reading R15.
# --------------------------------------------------------------------------
@dataclass
class RoutingStats:
    f: np.ndarray  # [N] share of the T*k top-k picks that chose each expert (sum 1)
    P: np.ndarray  # [N] mean softmax probability of each expert over the tokens (sum 1)
    aux: float  # N * sum_e f_e * P_e
    z: float  # mean over tokens of lse_t^2


def routing_stats(L, idx) -> RoutingStats:
    L = np.asarray(L, dtype=np.float64)
    idx = np.asarray(idx)
    T, N = L.shape
    k = idx.shape[1]
    m = L.max(axis=1)
    lse = m + np.log(np.exp(L - m[:, None]).sum(axis=1))
    probs = np.exp(L - lse[:, None])
    f = np.bincount(idx.reshape(-1), minlength=N).astype(np.float64) / (T * k)
    P = probs.mean(axis=0)
    return RoutingStats(f=f, P=P, aux=float(N * np.dot(f, P)), z=float(np.mean(lse * lse)))


# --------------------------------------------------------------------------
# Capacity C.  [Wiki] "Communication cost in distributed settings":
# C = gamma * k * T / N.  Reading R2 for rounding and "no limit".
# --------------------------------------------------------------------------
def capacity(T: int, N: int, k: int, capacity_factor: float) -> int:
    if T <= 0:
        return 0
    if capacity_factor is None or capacity_factor <= 0:
        return T
    c = capacity_factor * k * T / N
    c = math.ceil(c - 1e-6 * max(1.0, c))
    return int(min(max(c, 1), T))


@dataclass
class Dispatch:
    C: int
    req_counts: np.ndarray  # [N] int32 requests per expert before capacity
    counts: np.ndarray  # [N] int32 kept per expert
    offsets: np.ndarray  # [N+1] int32 exclusive scan of counts
    perm: np.ndarray  # [S] int32 pair index t*k + j of each slot
    inv: np.ndarray  # [T*k] int32 slot of each pair, -1 when dropped
    slot_gate: np.ndarray  # [S] float64 combine weight of each slot
    n_dropped: int

    @property
    def S(self) -> int:
        return int(self.offsets[-1])

    def slot_token(self, k: int) -> np.ndarray:
        return self.perm // k

    def slot_expert(self) -> np.ndarray:
        N = len(self.counts)
        return np.repeat(np.arange(N, dtype=np.int32), self.counts)


# --------------------------------------------------------------------------
# Step 4 (capacity) and step 5 (dispatch order).
# [Wiki] step 4: an expert accepts at most C tokens; the lowest-scoring
# overflow is dropped for that expert (worked example: E2 drops x2 at 0.667,
# E3 drops x4 at 0.286).  Readings R3 (rank by the float64 log-probability
# key, ties to the lower token) and R7 (slot order).
# --------------------------------------------------------------------------
def capacity_dispatch(idx, key, w, N: int, C: int, first_come: bool = False) -> Dispatch:
    """``first_come`` (reading R16a): keep each expert's first C requests in token
    order instead of the C highest keys."""
    idx = np.asarray(idx)
    key = np.asarray(key, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, k = idx.shape
    P = T * k
    inv = np.full(P, -1, dtype=np.int32)
    req = np.zeros(N, dtype=np.int32)
    cnt = np.zeros(N, dtype=np.int32)
    perm_parts = []
    for e in range(N):
        t_e, j_e = np.nonzero(idx == e)  # token-major order
        req[e] = len(t_e)
        if len(t_e) == 0:
            perm_parts.append(np.zeros(0, dtype=np.int64))
            continue
        kap = key[t_e, j_e]
        # primary: key descending; secondary: token ascending (first-come:
        # token ascending only)
        rank = np.arange(len(t_e)) if first_come else np.lexsort((t_e, -kap))
        keep = np.sort(rank[:C])  # back to token-ascending order (R7)
        cnt[e] = len(keep)
        perm_parts.append(t_e[keep].astype(np.int64) * k + j_e[keep])
    perm = np.concatenate(perm_parts).astype(np.int32) if perm_parts else np.zeros(0, np.int32)
    offsets = np.zeros(N + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(cnt)
    inv[perm] = np.arange(len(perm), dtype=np.int32)
    slot_gate = w.reshape(-1)[perm] if len(perm) else np.zeros(0)
    return Dispatch(C=C, req_counts=req, counts=cnt, offsets=offsets, perm=perm, inv=inv,
                    slot_gate=slot_gate, n_dropped=int(P - len(perm)))


def renormalise_survivors(disp: Dispatch, w, k: int) -> Dispatch:
    """Reading R16b: a token that lost at least one pick but kept some gets its
    kept weights divided by their sum ([Wiki] worked example: x4 keeps only
    E2, with weight 1.0). Tokens that kept every pick are left unchanged."""
    w = np.asarray(w, dtype=np.float64).reshape(-1, k)
    gate = disp.slot_gate.copy()
    inv = disp.inv.reshape(-1, k)
    for t in range(inv.shape[0]):
        kept = inv[t] >= 0
        if kept.all() or not kept.any():
            continue
        tot = w[t, kept].sum()
        for j in np.nonzero(kept)[0]:
            gate[inv[t, j]] = w[t, j] / tot
    return Dispatch(C=disp.C, req_counts=disp.req_counts, counts=disp.counts,
                    offsets=disp.offsets, perm=disp.perm, inv=disp.inv, slot_gate=gate,
                    n_dropped=disp.n_dropped)


# --------------------------------------------------------------------------
# Expert-choice routing ([Scaling] "Expert Choice Routing": each expert picks
# its top tokens from the batch, every expert the same number; [Arch] "Expert
# Choice Routing (ECR)": tokens no expert picks get zero).  Reading R17.
# Pairs are indexed p = t*N + e (every token is a candidate of every expert),
# so the Dispatch below uses k = N in its pair bookkeeping.
# --------------------------------------------------------------------------
def expert_choice_dispatch(L, C: int) -> Dispatch:
    L = np.asarray(L, dtype=np.float64)
    T, N = L.shape
    m = L.max(axis=1)
    lse = m + np.log(np.exp(L - m[:, None]).sum(axis=1))
    key = L - lse[:, None]  # log p[t, e]
    p = np.exp(key)
    inv = np.full(T * N, -1, dtype=np.int32)
    cnt = np.zeros(N, dtype=np.int32)
    parts = []
    toks = np.arange(T)
    for e in range(N):
        rank = np.lexsort((toks, -key[:, e]))  # probability descending, then token
        keep = np.sort(rank[:C])  # token-ascending slot order
        cnt[e] = len(keep)
        parts.append(keep.astype(np.int64) * N + e)
    perm = np.concatenate(parts).astype(np.int32)
    offsets = np.zeros(N + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(cnt)
    inv[perm] = np.arange(len(perm), dtype=np.int32)
    return Dispatch(C=C, req_counts=np.full(N, T, dtype=np.int32), counts=cnt, offsets=offsets,
                    perm=perm, inv=inv, slot_gate=p.reshape(-1)[perm],
                    n_dropped=int(T * N - len(perm)))


def moe_forward_expert_choice(x, W_g, logit_bias, W1, b1, W2, b2, k: int,
                              capacity_factor: float, logits: Optional[np.ndarray] = None,
                              tokens: Optional[Sequence[int]] = None,
                              identity_fallback: bool = False, shared=None):
    """Layer forward with expert-choice routing (reading R17). ``k`` is the
    average number of experts per token behind C; ``logits`` / ``tokens`` /
    ``shared`` as in moe_forward (the shared expert also serves the tokens no
    expert took, reading R18). Returns dict with y, logits, dispatch (pairs
    t*N + e)."""
    X = x
    T = X.shape[0]
    N = W_g.shape[1]
    d = W_g.shape[0]
    L = router_logits(X, W_g, logit_bias) if logits is None else np.asarray(logits, np.float64)
    C = capacity(T, N, k, capacity_factor)
    disp = expert_choice_dispatch(L, C)
    xf = X if identity_fallback else None
    if tokens is None:
        O = expert_slots_out(X, disp, N, W1, b1, W2, b2)
        y = combine(O, disp, T, N, d, x_fallback=xf)
    else:
        toks = np.asarray(tokens, dtype=np.int64)
        pairs = (toks[:, None] * N + np.arange(N)[None, :]).reshape(-1)
        slots = disp.inv[pairs]
        slots = slots[slots >= 0]
        O = expert_slots_out(X, disp, N, W1, b1, W2, b2, slots=slots)
        y = combine(O, disp, T, N, d, tokens=toks, x_fallback=xf)
    if shared is not None:
        y = y + shared_expert_out(X, shared, tokens)
    return {"y": y, "logits": L, "dispatch": disp}


# --------------------------------------------------------------------------
# Step 6: expert FFN.  [Arch] "Core Architecture": FFN(x) = W2 GELU(W1 x + b1)
# + b2, with nn.Linear(d, d_ff) / nn.Linear(d_ff, d) weights stored [out, in];
# [Rise] MoELayer experts (Linear, GELU, Linear).  Reading R6: exact GELU.
# --------------------------------------------------------------------------
def gelu(z):
    """Exact GELU, z * Phi(z) = z * (1 + erf(z / sqrt 2)) / 2, in float64."""
    z = np.asarray(z, dtype=np.float64)
    erf = torch.special.erf(torch.from_numpy(z / math.sqrt(2.0))).numpy()
    return z * 0.5 * (1.0 + erf)


def expert_ffn_rows(X_rows, W1_e, b1_e, W2_e, b2_e, return_hidden: bool = False):
    """Apply one expert to a batch of token rows. W1_e [d_ff, d], W2_e [d, d_ff]."""
    Xr = to_f64(X_rows)
    Z = Xr @ to_f64(W1_e).T
    if b1_e is not None:
        Z = Z + to_f64(b1_e)[None, :]
    H = gelu(Z)
    O = H @ to_f64(W2_e).T
    if b2_e is not None:
        O = O + to_f64(b2_e)[None, :]
    return (O, H) if return_hidden else O


def expert_slots_out(x, disp: Dispatch, k: int, W1, b1, W2, b2,
                     slots: Optional[np.ndarray] = None, return_hidden: bool = False):
    """Step 6 over dispatched slots: out[s] = FFN_{e(s)}(x[tok(s)]) (not gate-scaled).

    ``slots`` restricts the evaluation to a subset of slot ids (sampled checks
    on large workloads). Returns a dict slot -> row when ``slots`` is given,
    else an [S, d] array. [Wiki] pseudocode expert-compute loop.
    """
    N = len(disp.counts)
    exp_of_slot = disp.slot_expert()
    tok_of_slot = disp.slot_token(k)
    want = np.arange(disp.S) if slots is None else np.asarray(slots, dtype=np.int64)
    out = {}
    hid = {}
    for e in range(N):
        sel = want[exp_of_slot[want] == e] if len(want) else want
        if len(sel) == 0:
            continue
        tok = tok_of_slot[sel]
        rows = (x[torch.as_tensor(tok, dtype=torch.long)] if isinstance(x, torch.Tensor)
                else np.asarray(x)[tok])
        O, H = expert_ffn_rows(rows, W1[e], None if b1 is None else b1[e],
                               W2[e], None if b2 is None else b2[e], return_hidden=True)
        for i, s in enumerate(sel):
            out[int(s)] = O[i]
            hid[int(s)] = H[i]
    if slots is not None:
        return (out, hid) if return_hidden else out
    d = to_f64(W2[0]).shape[0]
    O_all = np.zeros((disp.S, d))
    H_all = np.zeros((disp.S, to_f64(W1[0]).shape[0])) if return_hidden else None
    for s, row in out.items():
        O_all[s] = row
        if return_hidden:
            H_all[s] = hid[s]
    return (O_all, H_all) if return_hidden else O_all


# --------------------------------------------------------------------------
# Step 7: weighted combine back to token order.  [Wiki] step 7 and the
# pseudocode's Y[t] += w * o; [Arch] SparseMoE outputs[mask] += weight * out.
# Readings R4 (dropped pair contributes zero) and R5 (all dropped -> 0).
# --------------------------------------------------------------------------
def combine(slot_out, disp: Dispatch, T: int, k: int, d: int,
            tokens: Optional[Sequence[int]] = None, x_fallback=None) -> np.ndarray:
    """y[t] = sum over kept j of w[t,j] * out[slot(t,j)]; rows for ``tokens`` only if given.

    ``slot_out`` is either an [S, d] array or a dict slot -> row. ``x_fallback``
    (reading R16c): a token whose every pick was dropped gets x[t] instead of 0.
    """
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    y = np.zeros((len(toks), d))
    for i, t in enumerate(toks):
        if x_fallback is not None and np.all(disp.inv[t * k:(t + 1) * k] < 0):
            y[i] = to_f64(x_fallback[int(t)])
            continue
        for j in range(k):
            s = disp.inv[t * k + j]
            if s < 0:
                continue
            y[i] += disp.slot_gate[s] * np.asarray(slot_out[int(s)], dtype=np.float64)
    return y


def shared_expert_out(x, shared, tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Reading R18: FFN_s(x_t) for every token (or the given ones); ``shared``
    is (W1s [d_fs, d], b1s or None, W2s [d, d_fs], b2s or None)."""
    W1s, b1s, W2s, b2s = shared
    X = to_f64(x)
    if tokens is not None:
        X = X[np.asarray(tokens, dtype=np.int64)]
    return expert_ffn_rows(X, W1s, b1s, W2s, b2s)


def moe_forward(x, W_g, logit_bias, W1, b1, W2, b2, k: int, capacity_factor: float,
                logits: Optional[np.ndarray] = None, C: Optional[int] = None,
                tokens: Optional[Sequence[int]] = None, first_come: bool = False,
                renorm_survivors: bool = False, identity_fallback: bool = False,
                shared=None):
    """Whole layer forward ([Wiki] MoE_Layer, steps 1-7).

    ``logits``: when given (e.g. another implementation's fp32 router logits,
    widened exactly), routing starts from them instead of from X W_g.
    ``C``: explicit capacity (the worked example gives C directly).
    ``tokens``: evaluate the output rows for these tokens only; routing and
    capacity still use every token, since capacity ranks across tokens.
    ``first_come``, ``renorm_survivors``, ``identity_fallback``: the drop-policy
    variants of reading R16. ``shared``: a shared expert's (W1s, b1s, W2s, b2s),
    added to every token's output (reading R18).

    Returns dict with y ([T,d] or [len(tokens), d]), logits, routing, dispatch.
    """
    X = x
    T = X.shape[0]
    N = W_g.shape[1]
    d = W_g.shape[0]
    L = router_logits(X, W_g, logit_bias) if logits is None else np.asarray(logits, np.float64)
    r = route_topk(L, k)
    if C is None:
        C = capacity(T, N, k, capacity_factor)
    disp = capacity_dispatch(r.idx, r.key, r.w, N, C, first_come=first_come)
    if renorm_survivors:
        disp = renormalise_survivors(disp, r.w, k)
    xf = X if identity_fallback else None
    if tokens is None:
        O = expert_slots_out(X, disp, k, W1, b1, W2, b2)
        y = combine(O, disp, T, k, d, x_fallback=xf)
    else:
        toks = np.asarray(tokens, dtype=np.int64)
        pairs = (toks[:, None] * k + np.arange(k)[None, :]).reshape(-1)
        slots = disp.inv[pairs]
        slots = slots[slots >= 0]
        O = expert_slots_out(X, disp, k, W1, b1, W2, b2, slots=slots)
        y = combine(O, disp, T, k, d, tokens=toks, x_fallback=xf)
    if shared is not None:
        y = y + shared_expert_out(X, shared, tokens)
    return {"y": y, "logits": L, "routing": r, "dispatch": disp}
