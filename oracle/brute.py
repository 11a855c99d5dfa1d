"""Brute-force statement of the MoE layer for tiny inputs.

TEST INFRASTRUCTURE ONLY (see oracle/moe_ref.py). Shares no code with the HIP
library and none with oracle/moe_ref.py either: it is a second, structurally
different statement of the same layer, used to check the slot-based oracle.

It follows the expert-loop form of the pages' snippets ([Scaling] MoELayer,
[Arch] SparseMoE, [Rise] MoELayer): every expert runs on every token (dense),
and a mask keeps the (token, expert) pairs the router chose and capacity kept.
Capacity selection here is done with pure-Python sorting on the softmax
probability itself (not the log-domain key), one expert at a time, exactly as
the [Wiki] worked example ranks requests. Expert modules are torch.nn layers in
float64 (nn.Linear stores weights [out, in]; nn.GELU() is the erf form).

The drop-policy variants are stated the same way: first-come capacity as the
[Wiki] pseudocode's dispatch loop (tokens in order, each token's picks in
order, an expert's buffer accepts while it holds fewer than C), survivor
renormalisation and identity fallback as plain per-token loops. The routing
statistics are stated with pure-Python sums over tokens and picks.

Only for small T, d, d_ff, N (pure-Python loops over tokens and experts).
"""
from __future__ import annotations

import math
from typing import Callable, List, Optional

import numpy as np
import torch


def _f64(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().to(torch.float64)
    return torch.as_tensor(np.asarray(t, dtype=np.float64))


def make_experts(W1, b1, W2, b2) -> List[Callable]:
    """nn.Sequential(Linear(d, d_ff), GELU(), Linear(d_ff, d)) per expert, float64."""
    W1, W2 = _f64(W1), _f64(W2)
    b1, b2 = _f64(b1), _f64(b2)
    N, d_ff, d = W1.shape
    experts = []
    for e in range(N):
        l1 = torch.nn.Linear(d, d_ff, bias=b1 is not None, dtype=torch.float64)
        l2 = torch.nn.Linear(d_ff, d, bias=b2 is not None, dtype=torch.float64)
        with torch.no_grad():
            l1.weight.copy_(W1[e])
            l2.weight.copy_(W2[e])
            if b1 is not None:
                l1.bias.copy_(b1[e])
            if b2 is not None:
                l2.bias.copy_(b2[e])
        experts.append(torch.nn.Sequential(l1, torch.nn.GELU(), l2))
    return experts


def brute_moe(x, logits, k: int, C: Optional[int], experts: List[Callable],
              first_come: bool = False, renorm: bool = False, identity: bool = False):
    """Dense-then-mask MoE forward.

    logits: [T, N] router logits (float64 or exactly widened fp32).
    C: per-expert capacity, or None for no limit.
    experts: list of callables mapping a float64 [M, d] tensor to [M, d].
    first_come / renorm / identity: the drop-policy variants.
    Returns (y [T, d] float64 numpy, kept set {(t, e)}, picks {t: [(e, w)]}).
    """
    X = _f64(x)
    L = _f64(logits)
    T, N = L.shape
    probs = torch.softmax(L, dim=-1)
    picks = {}
    for t in range(T):
        row = [(float(L[t, e]), e) for e in range(N)]
        # highest logit first; equal logits: lower expert id first
        row.sort(key=lambda p: (-p[0], p[1]))
        chosen = [e for _, e in row[:k]]
        tot = sum(float(probs[t, e]) for e in chosen)
        picks[t] = [(e, float(probs[t, e]) / tot) for e in chosen]
    kept = set()
    if first_come:
        buffers = {e: [] for e in range(N)}
        for t in range(T):
            for e, _ in picks[t]:
                if C is None or len(buffers[e]) < C:
                    buffers[e].append(t)
                    kept.add((t, e))
    else:
        for e in range(N):
            reqs = [(float(probs[t, e]), t) for t in range(T)
                    if any(pe == e for pe, _ in picks[t])]
            reqs.sort(key=lambda r: (-r[0], r[1]))  # highest score first, then lower token
            lim = len(reqs) if C is None else C
            for _, t in reqs[:lim]:
                kept.add((t, e))
    gates = {}
    for t in range(T):
        survivors = [(e, w) for e, w in picks[t] if (t, e) in kept]
        scale = 1.0
        if renorm and survivors and len(survivors) < len(picks[t]):
            scale = 1.0 / sum(w for _, w in survivors)
        for e, w in survivors:
            gates[(t, e)] = w * scale
    dense = [experts[e](X).detach() for e in range(N)]  # every expert on every token
    y = torch.zeros_like(X)
    for e in range(N):
        mask = torch.tensor([(t, e) in kept for t in range(T)], dtype=torch.bool)
        gate = torch.tensor([gates.get((t, e), 0.0) for t in range(T)], dtype=torch.float64)
        y += (mask.to(torch.float64) * gate)[:, None] * dense[e]
    if identity:
        for t in range(T):
            if not any((t, e) in kept for e, _ in picks[t]):
                y[t] = X[t]
    return y.numpy(), kept, picks


def brute_routing_stats(logits, k: int):
    """(f, P, aux, z) with pure-Python loops: f_e = picks of e / (T*k), P_e =
    mean softmax probability, aux = N * sum f_e P_e, z = mean lse^2."""
    L = _f64(logits)
    T, N = L.shape
    counts = [0] * N
    psum = [0.0] * N
    zsum = 0.0
    for t in range(T):
        row = [float(L[t, e]) for e in range(N)]
        m = max(row)
        lse = m + math.log(sum(math.exp(v - m) for v in row))
        zsum += lse * lse
        for e in range(N):
            psum[e] += math.exp(row[e] - lse)
        order = sorted(range(N), key=lambda e: (-row[e], e))
        for e in order[:k]:
            counts[e] += 1
    f = [c / (T * k) for c in counts]
    P = [s / T for s in psum]
    return f, P, N * sum(a * b for a, b in zip(f, P)), zsum / T


def brute_expert_choice(x, logits, C: int, experts: List[Callable], identity: bool = False):
    """Expert-choice layer with pure-Python selection: each expert sorts all
    tokens by its softmax probability (ties: lower token) and takes the first
    C; y[t] = sum over the experts that took t of p[t,e] * E_e(x_t)."""
    X = _f64(x)
    L = _f64(logits)
    T, N = L.shape
    probs = torch.softmax(L, dim=-1)
    taken = {}
    for e in range(N):
        col = sorted(range(T), key=lambda t: (-float(probs[t, e]), t))
        for t in col[:C]:
            taken.setdefault(t, []).append(e)
    dense = [experts[e](X).detach() for e in range(N)]
    y = torch.zeros_like(X)
    for t in range(T):
        if t not in taken:
            if identity:
                y[t] = X[t]
            continue
        for e in taken[t]:
            y[t] += float(probs[t, e]) * dense[e][t]
    return y.numpy(), {(t, e) for t, es in taken.items() for e in es}
