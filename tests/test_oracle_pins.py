"""Pins of the CPU oracle against facts the pages and the mathematics fix.

CPU only. Every pin calls the oracle through the module object ``M`` so that
``test_every_mutant_is_caught`` can plant a plausible mistake in the oracle
(a dropped term, a wrong sign or index, a transposed operand, a wrong tie
rule) and check that at least one pin fails for it.

Pins used (none of them re-types the oracle's own formula):
  * the worked example of the "Mixture-of-Experts" wiki page (N=4, k=2, T=5,
    C=2): drop set, final dispatch and the partial combine of x2 and x4;
  * the router with the per-expert logit bias as a torch nn.Linear(d, N)
    (weight W_g^T, bias the logit bias) in float64;
  * the capacity formula of the same page at the five workloads' numbers;
  * textbook values of the exact GELU, z * Phi(z);
  * the top-k-on-logits-then-softmax router of the "Scaling Language Models
    with Sparse Activation" and "Rise of Mixture-of-Experts Models" pages,
    evaluated with torch.topk and torch.softmax;
  * k = N with no capacity limit equals the dense softmax-weighted mixture of
    all experts (wiki page, router distribution G(x));
  * N = 1, k = 1 equals a plain nn.Sequential(Linear, GELU, Linear);
  * a brute-force dense-then-mask statement (oracle/brute.py) that ranks
    capacity by the softmax probability with pure-Python sorting;
  * the linear-expert closed form of the practice exercise on the "How Sparse
    Routing Scales Transformers" page;
  * dispatch invariants (counts <= C, slot bookkeeping, score order at cuts);
  * routing statistics: the wiki page's closed form (aux = 1 when f = P = 1/N,
    here from circulant logits), a collapsed router (aux -> N), the code form
    of the "Scaling" and "Rise" pages (k-hot mask averaged over tokens, i.e.
    k * f) evaluated with torch ops, torch.logsumexp for the z term, and
    pure-Python sums (oracle/brute.py);
  * drop policies: the worked example's survivor renormalisation (weight 1.0
    on E2 for x4, on E4 for x2), first-come capacity as the pseudocode's
    arrival-order loop (worked example and brute force), identity fallback
    for a token that loses every pick;
  * expert-choice routing: with no capacity limit every expert takes every
    token, which is the dense softmax mixture of all experts; every expert
    takes exactly min(C, T) tokens; pure-Python selection per expert
    (oracle/brute.py), with and without the identity fallback;
  * shared expert: with one routed expert and top-1 the layer is the sum of
    two plain nn.Sequential MLPs; with every routed pick dropped it is the
    shared MLP alone (plus the input row under the identity fallback).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.moe_ref as M
from oracle.brute import brute_expert_choice, brute_moe, brute_routing_stats, make_experts

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_layer(rng, T, d, d_ff, N, bias=True):
    x = torch.from_numpy(rng.standard_normal((T, d)))
    W_g = torch.from_numpy(rng.standard_normal((d, N)) * 0.5)
    W1 = torch.from_numpy(rng.standard_normal((N, d_ff, d)) / math.sqrt(d))
    W2 = torch.from_numpy(rng.standard_normal((N, d, d_ff)) / math.sqrt(d_ff))
    b1 = torch.from_numpy(rng.standard_normal((N, d_ff)) * 0.1) if bias else None
    b2 = torch.from_numpy(rng.standard_normal((N, d)) * 0.1) if bias else None
    return x, W_g, W1, b1, W2, b2


# ---------------------------------------------------------------- pins ----
def pin_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    N, k, T, C = g["N"], g["k"], g["T"], g["C"]
    assert M.capacity(T, N, k, g["capacity_factor_giving_C"]) == C
    L = np.full((T, N), -30.0)
    for t, picks in g["picks"].items():
        for e, p in picks.items():
            L[int(t), int(e)] = math.log(p)
    r = M.route_topk(L, k)
    for t, picks in g["picks"].items():
        assert set(r.idx[int(t)].tolist()) == {int(e) for e in picks}
    disp = M.capacity_dispatch(r.idx, r.key, r.w, N, C)
    assert disp.req_counts.tolist() == [len(g["requests_per_expert"][str(e)]) for e in range(N)]
    toks = disp.slot_token(k)
    for e in range(N):
        seg = toks[disp.offsets[e]:disp.offsets[e + 1]].tolist()
        assert seg == g["final_dispatch"][str(e)], (e, seg)
    dropped = sorted((int(p // k), int(r.idx[p // k, p % k])) for p in np.nonzero(disp.inv < 0)[0])
    assert dropped == sorted(tuple(p) for p in g["dropped_pairs"])
    # combine: x2 is served by E4 only, x4 by E2 only, each with its pre-drop weight
    X = np.arange(1, T * 3 + 1, dtype=np.float64).reshape(T, 3)
    out = {s: X[toks[s]] * (1 + int(e)) for e in range(N)
           for s in range(disp.offsets[e], disp.offsets[e + 1])}
    y = M.combine(out, disp, T, k, 3)
    for t, e in g["tokens_served_by_one_expert"].items():
        t = int(t)
        w_te = g["picks"][str(t)][str(e)]
        np.testing.assert_allclose(y[t], w_te * (1 + e) * X[t], rtol=1e-9)
    for t in range(T):
        if str(t) not in g["tokens_served_by_one_expert"]:
            ref = sum(p * (1 + int(e)) for e, p in g["picks"][str(t)].items()) * X[t]
            np.testing.assert_allclose(y[t], ref, rtol=1e-9)


def pin_capacity_formula():
    # C = capacity_factor * k * T / N at the five workloads
    assert M.capacity(256, 8, 2, 1.25) == 80
    assert M.capacity(8192, 64, 1, 1.0) == 128
    assert M.capacity(16384, 256, 8, 1.25) == 640
    assert M.capacity(4096, 8, 2, 0.0) == 4096  # no limit
    assert M.capacity(32, 8, 2, -1.0) == 32
    assert M.capacity(10, 4, 2, 1.0) == 5
    assert M.capacity(10, 4, 1, 1.0) == 3  # 2.5 rounds up
    assert M.capacity(7, 64, 1, 1.0) == 1  # clamped to at least one slot


def pin_gelu_textbook():
    # z * Phi(z) with Phi the standard normal CDF (textbook values)
    z = np.array([0.0, 1.0, -1.0, 2.0, -3.0, 0.5])
    phi = np.array([0.5, 0.8413447460685429, 0.15865525393145707, 0.9772498680518208,
                    0.0013498980316300933, 0.6914624612740131])
    np.testing.assert_allclose(M.gelu(z), z * phi, rtol=1e-14, atol=1e-300)


def pin_router_logits_linear():
    # Router step of the wiki page (logits = x W_g) with the workloads' per-
    # expert logit bias, stated as the pages' router module: a torch
    # nn.Linear(d, N) whose weight is W_g^T and whose bias is the logit bias,
    # evaluated in float64. A zero bias must give x W_g exactly as a Linear
    # without bias does.
    rng = np.random.default_rng(17)
    for (T, d, N) in ((7, 5, 4), (33, 16, 9), (64, 8, 64)):
        x = torch.from_numpy(rng.standard_normal((T, d)))
        W_g = torch.from_numpy(rng.standard_normal((d, N)) * 0.3)
        b = torch.from_numpy(rng.standard_normal(N) * 0.7)
        lin = torch.nn.Linear(d, N, bias=True, dtype=torch.float64)
        lin0 = torch.nn.Linear(d, N, bias=False, dtype=torch.float64)
        with torch.no_grad():
            lin.weight.copy_(W_g.T)
            lin.bias.copy_(b)
            lin0.weight.copy_(W_g.T)
            ref = lin(x).numpy()
            ref0 = lin0(x).numpy()
        np.testing.assert_allclose(M.router_logits(x, W_g, b), ref, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(M.router_logits(x, W_g, None), ref0, rtol=1e-13, atol=1e-13)
        # through the layer: the bias moves the top-1 choice to the favoured expert
        big = torch.full((N,), -50.0, dtype=torch.float64)
        big[N - 1] = 50.0
        r = M.route_topk(M.router_logits(x, W_g, big), 1)
        assert np.all(r.idx[:, 0] == N - 1)


def pin_topk_then_softmax_router():
    rng = np.random.default_rng(1)
    L = rng.standard_normal((64, 16)) * 2.0
    for k in (1, 2, 4, 16):
        r = M.route_topk(L, k)
        vals, ids = torch.topk(torch.from_numpy(L), k, dim=-1)
        assert np.array_equal(r.idx, ids.numpy())
        np.testing.assert_allclose(r.w, torch.softmax(vals, dim=-1).numpy(), rtol=1e-12)
        np.testing.assert_allclose(r.w.sum(axis=1), 1.0, rtol=1e-12)
        full = torch.softmax(torch.from_numpy(L), dim=-1).numpy()
        np.testing.assert_allclose(np.exp(r.key), np.take_along_axis(full, ids.numpy(), 1),
                                   rtol=1e-12)


def pin_topk_ties_lower_expert():
    L = np.array([[0.0, 1.0, 3.0, 1.0, 3.0, 2.0]])
    r = M.route_topk(L, 3)
    assert r.idx[0].tolist() == [2, 4, 5]
    r = M.route_topk(np.array([[1.0, 1.0, 1.0, 1.0]]), 2)
    assert r.idx[0].tolist() == [0, 1]
    np.testing.assert_allclose(r.w, 0.5, rtol=1e-15)


def pin_k1_gates_exactly_one():
    rng = np.random.default_rng(2)
    r = M.route_topk(rng.standard_normal((100, 7)), 1)
    assert np.all(r.w == 1.0)


def pin_dense_mixture_k_equals_n():
    rng = np.random.default_rng(3)
    T, d, d_ff, N = 12, 6, 10, 5
    x, W_g, W1, b1, W2, b2 = _rand_layer(rng, T, d, d_ff, N)
    res = M.moe_forward(x, W_g, None, W1, b1, W2, b2, k=N, capacity_factor=0.0)
    experts = make_experts(W1, b1, W2, b2)
    G = torch.softmax(x @ W_g, dim=-1)
    ref = sum(G[:, e:e + 1] * experts[e](x) for e in range(N)).detach().numpy()
    np.testing.assert_allclose(res["y"], ref, rtol=1e-11, atol=1e-12)


def pin_single_expert_is_mlp():
    rng = np.random.default_rng(4)
    for (T, d, d_ff) in ((9, 8, 8), (5, 4, 12)):
        x, W_g, W1, b1, W2, b2 = _rand_layer(rng, T, d, d_ff, 1)
        res = M.moe_forward(x, W_g, None, W1, b1, W2, b2, k=1, capacity_factor=0.0)
        mlp = torch.nn.Sequential(torch.nn.Linear(d, d_ff, dtype=torch.float64), torch.nn.GELU(),
                                  torch.nn.Linear(d_ff, d, dtype=torch.float64))
        with torch.no_grad():
            mlp[0].weight.copy_(W1[0]); mlp[0].bias.copy_(b1[0])
            mlp[2].weight.copy_(W2[0]); mlp[2].bias.copy_(b2[0])
        np.testing.assert_allclose(res["y"], mlp(x).detach().numpy(), rtol=1e-12, atol=1e-13)


BRUTE_CASES = [
    # T, d, d_ff, N, k, capacity_factor, bias
    (20, 6, 10, 4, 2, 0.8, True),
    (33, 8, 8, 5, 1, 1.0, False),
    (17, 5, 7, 6, 3, 0.5, True),
    (40, 4, 6, 8, 2, 1.25, False),
    (25, 6, 9, 3, 3, 0.0, True),
    (30, 3, 5, 16, 4, 0.3, False),
]


def pin_brute_force():
    for i, (T, d, d_ff, N, k, cf, bias) in enumerate(BRUTE_CASES):
        rng = np.random.default_rng(100 + i)
        x, W_g, W1, b1, W2, b2 = _rand_layer(rng, T, d, d_ff, N, bias)
        # skew one expert so capacity binds
        lb = np.zeros(N); lb[0] = 1.5
        res = M.moe_forward(x, W_g, lb, W1, b1, W2, b2, k=k, capacity_factor=cf)
        C = M.capacity(T, N, k, cf) if cf > 0 else None
        yb, kept, _ = brute_moe(x, res["logits"], k, C, make_experts(W1, b1, W2, b2))
        disp = res["dispatch"]
        kept_oracle = {(int(p // k), int(res["routing"].idx[p // k, p % k])) for p in disp.perm}
        assert kept_oracle == kept, (i, sorted(kept_oracle ^ kept))
        np.testing.assert_allclose(res["y"], yb, rtol=1e-11, atol=1e-12)


def pin_linear_experts_closed_form():
    # Practice exercise: experts x -> x * (i + 1), a random 4x8 gate, 200 tokens, k = 2.
    rng = np.random.default_rng(5)
    T, d, N, k = 200, 4, 8, 2
    X = rng.standard_normal((T, d))
    w_gate = rng.standard_normal((d, N))
    for skew in (False, True):
        Wg = w_gate.copy()
        if skew:
            Wg[:, 0] *= 5.0
        L = M.router_logits(X, Wg)
        r = M.route_topk(L, k)
        disp = M.capacity_dispatch(r.idx, r.key, r.w, N, M.capacity(T, N, k, 0.0))
        assert disp.n_dropped == 0
        toks, exps = disp.slot_token(k), disp.slot_expert()
        out = X[toks] * (exps[:, None] + 1.0)
        y = M.combine(out, disp, T, k, d)
        ref = X * (r.w * (r.idx + 1.0)).sum(axis=1, keepdims=True)
        np.testing.assert_allclose(y, ref, rtol=1e-12)
        hist = disp.req_counts
        assert hist.sum() == T * k
        if not skew:
            assert hist.max() <= 2 * (T * k / N)  # roughly even
        else:
            assert hist.argmax() == 0  # expert 0 got the head start


def pin_dispatch_invariants():
    rng = np.random.default_rng(6)
    for (T, N, k, cf) in ((500, 8, 2, 1.0), (300, 32, 4, 0.7), (64, 4, 1, 1.0), (50, 6, 6, 0.4)):
        L = rng.standard_normal((T, N)) + np.linspace(2.0, 0.0, N)[None, :]
        r = M.route_topk(L, k)
        C = M.capacity(T, N, k, cf)
        disp = M.capacity_dispatch(r.idx, r.key, r.w, N, C)
        req = np.bincount(r.idx.reshape(-1), minlength=N)
        assert np.array_equal(disp.req_counts, req)
        assert np.all(disp.counts <= C)
        assert np.array_equal(disp.counts, np.minimum(req, C))
        assert disp.S == T * k - disp.n_dropped
        assert np.array_equal(disp.inv[disp.perm], np.arange(disp.S))
        assert np.sum(disp.inv >= 0) == disp.S
        toks = disp.slot_token(k)
        for e in range(N):
            seg = slice(disp.offsets[e], disp.offsets[e + 1])
            assert np.all(np.diff(toks[seg]) > 0)
            assert np.all(r.idx.reshape(-1)[disp.perm[seg]] == e)
            kept_keys = r.key.reshape(-1)[disp.perm[seg]]
            pairs_e = np.nonzero(r.idx.reshape(-1) == e)[0]
            dropped = pairs_e[disp.inv[pairs_e] < 0]
            if len(dropped) and len(kept_keys):
                assert kept_keys.min() >= r.key.reshape(-1)[dropped].max()
        np.testing.assert_array_equal(disp.slot_gate, r.w.reshape(-1)[disp.perm])


def pin_capacity_ties_lower_token():
    # identical rows: equal keys; capacity 2 at the shared expert keeps tokens 0 and 1
    L = np.tile(np.array([[2.0, 0.0, -1.0]]), (4, 1))
    r = M.route_topk(L, 1)
    disp = M.capacity_dispatch(r.idx, r.key, r.w, 3, 2)
    assert disp.perm.tolist() == [0, 1]
    assert disp.inv.tolist() == [0, 1, -1, -1]


def pin_routing_stats_uniform():
    # circulant logits: token t prefers expert t mod N, then (t+1) mod N; with
    # k = 2 every expert gets the same share of picks and, by symmetry, the same
    # mean probability: f = P = 1/N and aux = N * N * (1/N)^2 = 1 (wiki page)
    N, reps, k = 8, 3, 2
    T = N * reps
    L = np.zeros((T, N))
    for t in range(T):
        L[t, t % N] = 3.0
        L[t, (t + 1) % N] = 2.0
    r = M.route_topk(L, k)
    st = M.routing_stats(L, r.idx)
    np.testing.assert_allclose(st.f, 1.0 / N, rtol=1e-15)
    np.testing.assert_allclose(st.P, 1.0 / N, rtol=1e-12)
    assert abs(st.aux - 1.0) < 1e-12
    lse = math.log(math.exp(3.0) + math.exp(2.0) + (N - 2))
    assert abs(st.z - lse * lse) < 1e-12
    # all-zero logits: lse = log N for every token
    st0 = M.routing_stats(np.zeros((5, N)), np.zeros((5, 1), dtype=np.int32))
    assert abs(st0.z - math.log(N) ** 2) < 1e-12


def pin_routing_stats_collapse():
    # every token strongly prefers expert 0: f = (1, 0, ...), aux = N * P_0 -> N
    N, T = 6, 40
    L = np.zeros((T, N))
    L[:, 0] = 40.0
    r = M.route_topk(L, 1)
    st = M.routing_stats(L, r.idx)
    assert st.f.tolist() == [1.0] + [0.0] * (N - 1)
    p0 = 1.0 / (1.0 + (N - 1) * math.exp(-40.0))
    assert abs(st.aux - N * p0) < 1e-12


def pin_routing_stats_code_form():
    # the load-balance snippets of the "Scaling" and "Rise" pages: a k-hot mask
    # averaged over tokens (sums to k) times the mean softmax, times N; the
    # z term with torch.logsumexp
    rng = np.random.default_rng(7)
    for (T, N, k) in ((50, 8, 2), (33, 16, 4), (20, 5, 1)):
        L = rng.standard_normal((T, N)) * 1.5 + np.linspace(1.0, 0.0, N)[None, :]
        r = M.route_topk(L, k)
        st = M.routing_stats(L, r.idx)
        Lt = torch.from_numpy(L)
        probs = torch.softmax(Lt, dim=-1)
        mask = torch.zeros_like(probs)
        mask.scatter_(-1, torch.from_numpy(r.idx.astype(np.int64)), 1.0)
        code = N * (mask.mean(dim=0) * probs.mean(dim=0)).sum().item()
        assert abs(code - k * st.aux) < 1e-12 * max(1.0, code)
        np.testing.assert_allclose(st.P, probs.mean(dim=0).numpy(), rtol=1e-12)
        zt = (torch.logsumexp(Lt, dim=-1) ** 2).mean().item()
        assert abs(zt - st.z) < 1e-12 * max(1.0, zt)
        fb, Pb, auxb, zb = brute_routing_stats(L, k)
        np.testing.assert_allclose(st.f, fb, rtol=1e-15)
        np.testing.assert_allclose(st.P, Pb, rtol=1e-12)
        assert abs(st.aux - auxb) < 1e-12 and abs(st.z - zb) < 1e-12 * max(1.0, zb)


def _worked_example_routing():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    N, k, T, C = g["N"], g["k"], g["T"], g["C"]
    L = np.full((T, N), -30.0)
    for t, picks in g["picks"].items():
        for e, p in picks.items():
            L[int(t), int(e)] = math.log(p)
    return g, N, k, T, C, M.route_topk(L, k)


def pin_first_come_worked_example():
    # the wiki pseudocode's dispatch loop (tokens in order, an expert's buffer
    # accepts while it holds fewer than C) on the worked example's requests:
    # E2 gets x1, x2, x4 and keeps x1, x2; E3 gets x1, x4, x5 and keeps x1, x4
    g, N, k, T, C, r = _worked_example_routing()
    disp = M.capacity_dispatch(r.idx, r.key, r.w, N, C, first_come=True)
    toks = disp.slot_token(k)
    segs = {e: toks[disp.offsets[e]:disp.offsets[e + 1]].tolist() for e in range(N)}
    assert segs == {0: [2, 4], 1: [0, 1], 2: [0, 3], 3: [1, 2]}, segs
    dropped = sorted((int(p // k), int(r.idx[p // k, p % k])) for p in np.nonzero(disp.inv < 0)[0])
    assert dropped == [(3, 1), (4, 2)]


def pin_renorm_worked_example():
    # "renormalize over the surviving expert alone (weight 1.0 on E2's output)"
    # for x4; x2 likewise keeps only E4, with weight 1.0
    g, N, k, T, C, r = _worked_example_routing()
    disp = M.renormalise_survivors(M.capacity_dispatch(r.idx, r.key, r.w, N, C), r.w, k)
    toks = disp.slot_token(k)
    X = np.arange(1, T * 3 + 1, dtype=np.float64).reshape(T, 3)
    out = {s: X[toks[s]] * (1 + int(e)) for e in range(N)
           for s in range(disp.offsets[e], disp.offsets[e + 1])}
    y = M.combine(out, disp, T, k, 3)
    for t, e in g["tokens_served_by_one_expert"].items():
        t = int(t)
        np.testing.assert_allclose(y[t], 1.0 * (1 + e) * X[t], rtol=1e-12)
    for t in range(T):
        if str(t) not in g["tokens_served_by_one_expert"]:
            ref = sum(p * (1 + int(e)) for e, p in g["picks"][str(t)].items()) * X[t]
            np.testing.assert_allclose(y[t], ref, rtol=1e-9)


def pin_identity_fallback():
    # four identical tokens, one expert each, capacity 1: tokens 1..3 lose their
    # only pick and keep their input (the pseudocode's fallback); token 0 is served
    rng = np.random.default_rng(8)
    T, d, d_ff, N = 4, 5, 7, 3
    x, W_g, W1, b1, W2, b2 = _rand_layer(rng, T, d, d_ff, N)
    x = x[:1].repeat(T, 1)
    res = M.moe_forward(x, W_g, None, W1, b1, W2, b2, k=1, capacity_factor=0.0, C=1,
                        identity_fallback=True)
    e0 = int(res["routing"].idx[0, 0])
    ref0 = make_experts(W1, b1, W2, b2)[e0](x[:1]).detach().numpy()[0]
    np.testing.assert_allclose(res["y"][0], ref0, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(res["y"][1:], x[1:].numpy())
    plain = M.moe_forward(x, W_g, None, W1, b1, W2, b2, k=1, capacity_factor=0.0, C=1)
    assert np.all(plain["y"][1:] == 0.0)


def pin_brute_force_policies():
    for i, (T, d, d_ff, N, k, cf, bias) in enumerate(BRUTE_CASES[:4]):
        rng = np.random.default_rng(200 + i)
        x, W_g, W1, b1, W2, b2 = _rand_layer(rng, T, d, d_ff, N, bias)
        lb = np.zeros(N); lb[0] = 2.5
        C = M.capacity(T, N, k, cf) if cf > 0 else None
        for fc, rn, idn in ((True, False, False), (False, True, False), (False, False, True),
                            (True, True, True)):
            res = M.moe_forward(x, W_g, lb, W1, b1, W2, b2, k=k, capacity_factor=cf,
                                first_come=fc, renorm_survivors=rn, identity_fallback=idn)
            yb, kept, _ = brute_moe(x, res["logits"], k, C, make_experts(W1, b1, W2, b2),
                                    first_come=fc, renorm=rn, identity=idn)
            disp = res["dispatch"]
            kept_oracle = {(int(p // k), int(res["routing"].idx[p // k, p % k])) for p in disp.perm}
            assert kept_oracle == kept, (i, fc, rn, idn)
            np.testing.assert_allclose(res["y"], yb, rtol=1e-11, atol=1e-12)


def pin_expert_choice_dense():
    # no capacity limit: every expert takes every token with weight p[t, e],
    # the dense softmax mixture of all experts
    rng = np.random.default_rng(9)
    T, d, d_ff, N = 14, 6, 9, 5
    x, W_g, W1, b1, W2, b2 = _rand_layer(rng, T, d, d_ff, N)
    res = M.moe_forward_expert_choice(x, W_g, None, W1, b1, W2, b2, k=2, capacity_factor=0.0)
    experts = make_experts(W1, b1, W2, b2)
    G = torch.softmax(x @ W_g, dim=-1)
    ref = sum(G[:, e:e + 1] * experts[e](x) for e in range(N)).detach().numpy()
    np.testing.assert_allclose(res["y"], ref, rtol=1e-11, atol=1e-12)


def pin_expert_choice_balance_and_brute():
    for i, (T, d, d_ff, N, k, cf, bias) in enumerate(BRUTE_CASES[:5]):
        rng = np.random.default_rng(300 + i)
        x, W_g, W1, b1, W2, b2 = _rand_layer(rng, T, d, d_ff, N, bias)
        lb = np.zeros(N); lb[0] = 2.0
        for identity in (False, True):
            res = M.moe_forward_expert_choice(x, W_g, lb, W1, b1, W2, b2, k=k, capacity_factor=cf,
                                              identity_fallback=identity)
            C = M.capacity(T, N, k, cf)
            disp = res["dispatch"]
            # perfect balance by construction: every expert takes min(C, T) tokens
            assert np.all(disp.counts == min(C, T))
            yb, taken = brute_expert_choice(x, res["logits"], C, make_experts(W1, b1, W2, b2),
                                            identity=identity)
            kept = {(int(p // N), int(p % N)) for p in disp.perm}
            assert kept == taken, (i, identity)
            np.testing.assert_allclose(res["y"], yb, rtol=1e-11, atol=1e-12)


def _mlp(W1, b1, W2, b2):
    d_ff, d = W1.shape
    m = torch.nn.Sequential(torch.nn.Linear(d, d_ff, dtype=torch.float64), torch.nn.GELU(),
                            torch.nn.Linear(d_ff, d, dtype=torch.float64))
    with torch.no_grad():
        m[0].weight.copy_(W1); m[0].bias.copy_(b1)
        m[2].weight.copy_(W2); m[2].bias.copy_(b2)
    return m


def pin_shared_expert():
    rng = np.random.default_rng(10)
    T, d, d_ff, d_fs = 9, 6, 8, 5
    x, W_g, W1, b1, W2, b2 = _rand_layer(rng, T, d, d_ff, 1)
    W1s = torch.from_numpy(rng.standard_normal((d_fs, d)) / math.sqrt(d))
    W2s = torch.from_numpy(rng.standard_normal((d, d_fs)) / math.sqrt(d_fs))
    b1s = torch.from_numpy(rng.standard_normal(d_fs) * 0.1)
    b2s = torch.from_numpy(rng.standard_normal(d) * 0.1)
    shared = (W1s, b1s, W2s, b2s)
    ref_s = _mlp(W1s, b1s, W2s, b2s)(x).detach().numpy()
    # one routed expert, top-1: routed MLP + shared MLP
    res = M.moe_forward(x, W_g, None, W1, b1, W2, b2, k=1, capacity_factor=0.0, shared=shared)
    ref = _mlp(W1[0], b1[0], W2[0], b2[0])(x).detach().numpy() + ref_s
    np.testing.assert_allclose(res["y"], ref, rtol=1e-12, atol=1e-13)
    # every routed pick but the first dropped (capacity 1): the shared MLP alone,
    # or the input row plus it under the identity fallback
    for identity in (False, True):
        res = M.moe_forward(x, W_g, None, W1, b1, W2, b2, k=1, capacity_factor=0.0, C=1,
                            shared=shared, identity_fallback=identity)
        tail = ref_s[1:] + (x[1:].numpy() if identity else 0.0)
        np.testing.assert_allclose(res["y"][1:], tail, rtol=1e-12, atol=1e-13)
    # the sampled-token form agrees with the full form
    res_t = M.moe_forward(x, W_g, None, W1, b1, W2, b2, k=1, capacity_factor=0.0, shared=shared,
                          tokens=[0, 4, 8])
    np.testing.assert_allclose(res_t["y"], ref[[0, 4, 8]], rtol=1e-12, atol=1e-13)


PINS = [pin_worked_example, pin_router_logits_linear, pin_capacity_formula, pin_gelu_textbook,
        pin_topk_then_softmax_router, pin_topk_ties_lower_expert, pin_k1_gates_exactly_one, pin_dense_mixture_k_equals_n,
        pin_single_expert_is_mlp, pin_brute_force, pin_linear_experts_closed_form,
        pin_dispatch_invariants, pin_capacity_ties_lower_token, pin_routing_stats_uniform,
        pin_routing_stats_collapse, pin_routing_stats_code_form, pin_first_come_worked_example,
        pin_renorm_worked_example, pin_identity_fallback, pin_brute_force_policies,
        pin_expert_choice_dense, pin_expert_choice_balance_and_brute, pin_shared_expert]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ------------------------------------------------------------- mutants ----
_orig = {n: getattr(M, n) for n in ("router_logits", "gelu", "route_topk", "capacity", "capacity_dispatch",
                                    "expert_ffn_rows", "combine", "routing_stats",
                                    "renormalise_survivors", "expert_choice_dispatch",
                                    "shared_expert_out")}


def _mut_logit_bias_ignored(x, W_g, logit_bias=None):
    return _orig["router_logits"](x, W_g, None)


def _mut_logit_bias_negated(x, W_g, logit_bias=None):
    return _orig["router_logits"](x, W_g, None if logit_bias is None else -M.to_f64(logit_bias))


def _mut_gelu_tanh(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))


def _mut_no_renorm(L, k):
    r = _orig["route_topk"](L, k)
    r.w = np.exp(r.key)
    return r


def _mut_ties_high(L, k):
    L = np.asarray(L, dtype=np.float64)
    r = _orig["route_topk"](L, k)
    order = np.argsort(-L[:, ::-1], axis=1, kind="stable")
    r.idx = (L.shape[1] - 1 - order[:, :k]).astype(np.int32)
    rows = np.arange(L.shape[0])[:, None]
    p = r.probs[rows, r.idx]
    r.w = p / p.sum(1, keepdims=True)
    r.key = L[rows, r.idx] - r.lse[:, None]
    return r


def _mut_key_sign(L, k):
    r = _orig["route_topk"](L, k)
    r.key = r.key + 2 * r.lse[:, None]
    return r


def _mut_key_from_w(L, k):
    r = _orig["route_topk"](L, k)
    r.key = np.log(r.w)
    return r


def _mut_capacity_no_k(T, N, k, cf):
    return _orig["capacity"](T, N, 1, cf)


def _mut_drop_highest(idx, key, w, N, C, first_come=False):
    return _orig["capacity_dispatch"](idx, -np.asarray(key), w, N, C, first_come=first_come)


def _mut_slot_order_by_key(idx, key, w, N, C, first_come=False):
    disp = _orig["capacity_dispatch"](idx, key, w, N, C, first_come=first_come)
    key = np.asarray(key).reshape(-1)
    for e in range(N):
        seg = slice(disp.offsets[e], disp.offsets[e + 1])
        p = disp.perm[seg]
        disp.perm[seg] = p[np.argsort(-key[p], kind="stable")]
    disp.inv[:] = -1
    disp.inv[disp.perm] = np.arange(len(disp.perm))
    disp.slot_gate = np.asarray(w).reshape(-1)[disp.perm]
    return disp


def _mut_w1_untransposed(X_rows, W1_e, b1_e, W2_e, b2_e, return_hidden=False):
    return _orig["expert_ffn_rows"](X_rows, M.to_f64(W1_e).T, b1_e, W2_e, b2_e, return_hidden)


def _mut_drop_b2(X_rows, W1_e, b1_e, W2_e, b2_e, return_hidden=False):
    return _orig["expert_ffn_rows"](X_rows, W1_e, b1_e, W2_e, None, return_hidden)


def _mut_combine_no_gate(slot_out, disp, T, k, d, tokens=None, x_fallback=None):
    import copy
    d2 = copy.copy(disp)
    d2.slot_gate = np.ones_like(disp.slot_gate)
    return _orig["combine"](slot_out, d2, T, k, d, tokens, x_fallback)


def _mut_combine_first_only(slot_out, disp, T, k, d, tokens=None, x_fallback=None):
    import copy
    d2 = copy.copy(disp)
    d2.inv = disp.inv.copy()
    d2.inv.reshape(-1, k)[:, 1:] = -1
    return _orig["combine"](slot_out, d2, T, k, d, tokens, x_fallback)


def _mut_stats_f_over_tokens(L, idx):
    st = _orig["routing_stats"](L, idx)
    k = np.asarray(idx).shape[1]
    st.f = st.f * k
    st.aux = st.aux * k
    return st


def _mut_stats_P_from_topk(L, idx):
    st = _orig["routing_stats"](L, idx)
    L = np.asarray(L, dtype=np.float64)
    idx = np.asarray(idx)
    T, N = L.shape
    Pk = np.zeros(N)
    for t in range(T):
        v = np.exp(L[t, idx[t]] - L[t, idx[t]].max())
        Pk[idx[t]] += v / v.sum()
    st.P = Pk / T
    st.aux = float(N * np.dot(st.f, st.P))
    return st


def _mut_stats_z_unsquared(L, idx):
    st = _orig["routing_stats"](L, idx)
    L = np.asarray(L, dtype=np.float64)
    m = L.max(axis=1)
    st.z = float(np.mean(m + np.log(np.exp(L - m[:, None]).sum(axis=1))))
    return st


def _mut_first_come_ignored(idx, key, w, N, C, first_come=False):
    return _orig["capacity_dispatch"](idx, key, w, N, C)


def _mut_renorm_over_all_picks(disp, w, k):
    return disp


def _mut_fallback_ignored(slot_out, disp, T, k, d, tokens=None, x_fallback=None):
    return _orig["combine"](slot_out, disp, T, k, d, tokens)


def _mut_ec_first_tokens(L, C):
    # every expert takes the first C tokens (arrival order) instead of its top C
    disp = _orig["expert_choice_dispatch"](L, C)
    L = np.asarray(L, dtype=np.float64)
    T, N = L.shape
    Cc = min(C, T)
    perm = np.concatenate([np.arange(Cc) * N + e for e in range(N)]).astype(np.int32)
    inv = np.full(T * N, -1, dtype=np.int32)
    inv[perm] = np.arange(len(perm), dtype=np.int32)
    p = np.exp(L - (L.max(1) + np.log(np.exp(L - L.max(1)[:, None]).sum(1)))[:, None])
    disp.perm, disp.inv = perm, inv
    disp.slot_gate = p.reshape(-1)[perm]
    return disp


def _mut_ec_gate_renormalised(L, C):
    disp = _orig["expert_choice_dispatch"](L, C)
    N = np.asarray(L).shape[1]
    g = disp.slot_gate.copy()
    tok = disp.perm // N
    for t in np.unique(tok):
        sel = tok == t
        g[sel] = g[sel] / g[sel].sum()
    disp.slot_gate = g
    return disp


def _mut_shared_no_b2(x, shared, tokens=None):
    W1s, b1s, W2s, b2s = shared
    return _orig["shared_expert_out"](x, (W1s, b1s, W2s, None), tokens)


MUTANTS = {
    "logit_bias_ignored": ("router_logits", _mut_logit_bias_ignored),
    "logit_bias_negated": ("router_logits", _mut_logit_bias_negated),
    "gelu_tanh_approx": ("gelu", _mut_gelu_tanh),
    "no_renormalisation": ("route_topk", _mut_no_renorm),
    "ties_to_higher_expert": ("route_topk", _mut_ties_high),
    "key_sign_of_lse": ("route_topk", _mut_key_sign),
    "rank_by_renormalised_weight": ("route_topk", _mut_key_from_w),
    "capacity_without_k": ("capacity", _mut_capacity_no_k),
    "drop_highest_scoring": ("capacity_dispatch", _mut_drop_highest),
    "slot_order_by_score": ("capacity_dispatch", _mut_slot_order_by_key),
    "w1_not_transposed": ("expert_ffn_rows", _mut_w1_untransposed),
    "second_bias_dropped": ("expert_ffn_rows", _mut_drop_b2),
    "combine_without_gate": ("combine", _mut_combine_no_gate),
    "combine_first_pick_only": ("combine", _mut_combine_first_only),
    "stats_f_over_tokens": ("routing_stats", _mut_stats_f_over_tokens),
    "stats_P_from_topk_weights": ("routing_stats", _mut_stats_P_from_topk),
    "stats_z_unsquared": ("routing_stats", _mut_stats_z_unsquared),
    "first_come_ignored": ("capacity_dispatch", _mut_first_come_ignored),
    "renorm_not_applied": ("renormalise_survivors", _mut_renorm_over_all_picks),
    "identity_fallback_ignored": ("combine", _mut_fallback_ignored),
    "expert_choice_by_token_order": ("expert_choice_dispatch", _mut_ec_first_tokens),
    "expert_choice_gate_renormalised": ("expert_choice_dispatch", _mut_ec_gate_renormalised),
    "shared_expert_second_bias_dropped": ("shared_expert_out", _mut_shared_no_b2),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(M, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except TypeError:
            raise  # a mutant with the wrong signature proves nothing
        except Exception as exc:  # noqa: BLE001 - a wrong value or shape counts as a catch
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"mutant {name} passed every pin"
