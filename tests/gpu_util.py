"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding and compare with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np
import torch

import oracle.moe_ref as M
from moe_inputs import Workload, make_inputs

EPS32 = 2.0 ** -24  # unit roundoff of fp32
U_BF16 = 2.0 ** -8  # unit roundoff of bf16 (8 significant bits)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_logit_err(L_gpu: np.ndarray, L_ref: np.ndarray) -> float:
    """max |dL| / max(|L_ref|, rms(L_ref)), elementwise denominator."""
    rms = float(np.sqrt(np.mean(L_ref ** 2))) if L_ref.size else 1.0
    den = np.maximum(np.abs(L_ref), rms)
    return float(np.max(np.abs(L_gpu - L_ref) / den)) if L_ref.size else 0.0


def to_dev(inp: dict, dev="cuda"):
    return {k: (None if v is None else v.to(dev).contiguous()) for k, v in inp.items()}


def capacity_cut_gap(idx, key, N, C):
    """Smallest |key(C-th) - key(C+1-th)| over over-capacity experts (inf if none)."""
    gap = np.inf
    flat_i = idx.reshape(-1)
    flat_k = key.reshape(-1)
    for e in range(N):
        ks = np.sort(flat_k[flat_i == e])[::-1]
        if len(ks) > C:
            gap = min(gap, abs(ks[C - 1] - ks[C]))
    return gap


def check_dispatch_valid(idx, key_ref, key_gpu, N, C, perm, inv, offsets, k):
    """Validity of a dispatch result when keys tie within rounding at a cut.

    The GPU's selection must be exactly consistent with the GPU's own fp64 keys
    (every kept key >= every dropped key of the same expert, and among keys
    equal to the cut the lower tokens are kept), and consistent with the
    oracle's keys within the key tolerance (1e-12)."""
    T = idx.shape[0]
    P = T * k
    S = int(offsets[-1])
    assert np.array_equal(inv[perm[:S]], np.arange(S))
    assert np.sum(inv[:P] >= 0) == S
    flat_i = idx.reshape(-1)
    kr = np.asarray(key_ref, dtype=np.float64).reshape(-1)
    kg = np.asarray(key_gpu, dtype=np.float64).reshape(-1)
    kept = inv[:P] >= 0
    for e in range(N):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat_i[seg] == e)
        assert np.all(np.diff(seg // k) > 0)
        pairs = np.nonzero(flat_i == e)[0]
        assert len(seg) == min(C, len(pairs))
        kk = kept[pairs]
        if kk.all():
            continue
        pk, pd = pairs[kk], pairs[~kk]
        if len(pk) == 0:
            continue
        # exact order on the GPU's own keys, ties to the lower token
        gk, gd = kg[pk], kg[pd]
        cut = gk.min()
        assert cut >= gd.max(), f"expert {e}: a dropped key exceeds a kept key"
        tk, td = pk[gk == cut] // k, pd[gd == cut] // k
        if len(tk) and len(td):
            assert tk.max() < td.min(), f"expert {e}: equal keys not kept by lower token"
        # the oracle's keys within the key tolerance
        assert kr[pk].min() >= kr[pd].max() - 1e-12, f"expert {e}: order differs beyond 1e-12"


def output_error_bound(inp, od, k, toks, u_h, gelu_abs=0.0):
    """Elementwise a-priori bound on |y_gpu - y_exact| for the fp32-output path.

    Derived from the arithmetic of the HIP path (not from the oracle's code):
      GEMM1 : bf16 x bf16 products are exact in fp32; fp32 accumulation over d
              terms errs by at most (d+4) eps32 sum|x||W1| (fp32 inputs: the
              products' own rounding is inside the same bound);
      GELU  : |GELU'| <= 1.13 carries that error; the fp32 erf-based GELU adds
              a few ulp, taken as 8 eps32 |h|; the bf16 kernels' GELU (erfc from
              Abramowitz-Stegun 7.1.26, |error| <= 1.5e-7, in fp32) adds at most
              gelu_abs |z| (0.75e-7 from the approximation, the rest from about
              12 fp32 roundings of erfc <= 1);
      hidden: rounded to bf16 (u_h = 2^-8), carried as a bf16 hi + lo pair
              (u_h = 2^-16) or kept fp32 (u_h = eps32);
      GEMM2 : fp32 accumulation over d_ff terms, (d_ff+4) eps32 sum|h||W2|;
      gate, combine over k picks in fp32: (k+5) eps32 sum g|o| (this also
              covers the fp32 gates' <= 2 eps32 relative difference).
    """
    X = M.to_f64(inp["x"])
    d = X.shape[1]
    N = len(od.counts)
    W1, W2, b1, b2 = inp["W1"], inp["W2"], inp["b1"], inp["b2"]
    d_ff = W1.shape[1]
    toks = np.asarray(toks, dtype=np.int64)
    pairs = (toks[:, None] * k + np.arange(k)[None, :])  # [len(toks), k]
    slots = od.inv[pairs]
    want = np.unique(slots[slots >= 0]).astype(np.int64)
    exp_of = od.slot_expert()
    tok_of = od.slot_token(k)
    # per wanted slot: the bound of its gate-free output row, and |o|
    pos = np.full(max(od.S, 1), -1, dtype=np.int64)
    pos[want] = np.arange(len(want))
    Bo_all = np.zeros((len(want), d))
    Oabs_all = np.zeros((len(want), d))
    for e in range(N):
        sel = want[exp_of[want] == e] if len(want) else want
        if len(sel) == 0:
            continue
        rows = X[tok_of[sel]]
        W1e, W2e = M.to_f64(W1[e]), M.to_f64(W2[e])
        b1e = None if b1 is None else M.to_f64(b1[e])
        b2e = None if b2 is None else M.to_f64(b2[e])
        Z = rows @ W1e.T + (0 if b1e is None else b1e)
        A1 = np.abs(rows) @ np.abs(W1e).T + (0 if b1e is None else np.abs(b1e))
        H = M.gelu(Z)
        E = (u_h * np.abs(H) + 1.13 * (d + 4) * EPS32 * A1 + (d_ff + 12) * EPS32 * np.abs(H)
             + gelu_abs * np.abs(Z))
        Bo_all[pos[sel]] = E @ np.abs(W2e).T + (0 if b2e is None else (d_ff + 4) * EPS32 * np.abs(b2e))
        Oabs_all[pos[sel]] = np.abs(H @ W2e.T + (0 if b2e is None else b2e))
    B = np.zeros((len(toks), d))
    for j in range(k):
        s = slots[:, j]
        m = s >= 0
        if not m.any():
            continue
        q = pos[s[m]]
        g = np.asarray(od.slot_gate, dtype=np.float64)[s[m]][:, None]
        B[m] += g * (Bo_all[q] + (k + 5) * EPS32 * Oabs_all[q])
    return B


def record(kind: str, name: str, res: dict):
    """Append one measured result as a JSON line to $MOE_PARITY_RECORD (if set)."""
    path = os.environ.get("MOE_PARITY_RECORD")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps({"kind": kind, "case": name,
                            **{k: (float(v) if isinstance(v, (np.floating, float)) else v)
                               for k, v in res.items()}}) + "\n")


def heavy_drop_plain(dtype: str, split: bool, dropped_share: float, identity: bool) -> bool:
    """The one class of cases not held to 2e-2 x RMS(y): the plain bf16 hidden
    layer when more than three quarters of the picks are dropped and dropped
    tokens output zero. The hidden layer's bf16 rounding (relative 2^-9 per
    element) sets the largest row errors, while RMS(y) falls with the share of
    rows that are zero or keep a small gate, so the ratio can exceed the bar
    (measured up to 4.6e-2 on such cases) with every element still inside the
    arithmetic error bound. The same shapes are held to the bar with the hi+lo
    hidden layer (MOE_FLAG_HIDDEN_SPLIT)."""
    return dtype == "bf16" and not split and not identity and dropped_share > 0.75


def run_and_compare(w: Workload, lib, check_compose=True, seed=None, inputs=None, flags=0,
                    strict=None):
    """Run moe_forward (+ sub-calls) on the GPU and compare with the oracle on
    every token: logits on every row, every output element.

    flags: MOE_FLAG_HIDDEN_SPLIT and the drop-policy flags (FIRST_COME,
    RENORM_SURVIVORS, IDENTITY_FALLBACK); the fp32-output variant is always run.
    strict: also hold y to max|dy| <= 2e-2 (bf16) / 1e-4 (fp32) x RMS(y_ref).
    None (default): every case except heavy_drop_plain ones; a caller that
    passes False states why.
    Returns a dict of measured errors.
    """
    t0 = time.time()
    split = bool(flags & lib.MOE_FLAG_HIDDEN_SPLIT)
    first_come = bool(flags & lib.MOE_FLAG_FIRST_COME)
    renorm = bool(flags & lib.MOE_FLAG_RENORM_SURVIVORS)
    identity = bool(flags & lib.MOE_FLAG_IDENTITY_FALLBACK)
    dflags = flags & (lib.MOE_FLAG_FIRST_COME | lib.MOE_FLAG_RENORM_SURVIVORS)
    say(f"[case] {w.name} T={w.T} d={w.d} d_ff={w.d_ff} N={w.N} k={w.k} cf={w.capacity_factor} "
        f"dtype={w.dtype} skew={w.skew} seed={w.seed if seed is None else seed} flags={flags}")
    inp = make_inputs(w, seed=seed) if inputs is None else inputs
    dv = to_dev(inp)
    k, N, T = w.k, w.N, w.T
    say(f"[step] moe_forward {w.name}")
    y32, ex = lib.moe_forward(dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"], dv["W2"],
                              dv["b2"], k, w.capacity_factor, want_routing=True,
                              flags=flags | lib.MOE_FLAG_Y_F32)
    y_act = lib.moe_forward(dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"], dv["W2"],
                            dv["b2"], k, w.capacity_factor, flags=flags)
    torch.cuda.synchronize()
    say(f"[step] moe_route/moe_dispatch {w.name}")
    logits, idx, gw, gkey = lib.moe_route(dv["x"], dv["W_g"], dv["logit_bias"], k)
    disp = lib.moe_dispatch(idx, gw, gkey, N, w.capacity_factor, flags=dflags)
    torch.cuda.synchronize()
    L_gpu = logits.cpu().double().numpy()
    res = {}

    # the activation-dtype output is the fp32 output rounded once (RNE)
    if not torch.equal(y_act.view(torch.uint8), y32.to(y_act.dtype).view(torch.uint8)):
        bad = (y_act.view(torch.uint8) != y32.to(y_act.dtype).view(torch.uint8)).view(T, -1)
        rows = bad.any(1).nonzero().flatten()
        r0 = int(rows[0])
        raise AssertionError(
            f"activation-dtype output is not the rounded fp32 output: {int(rows.numel())} rows "
            f"differ, first row {r0} (inv {ex['inv'][r0].tolist()}): fp32 "
            f"{y32[r0, :4].tolist()} vs {y_act[r0, :4].float().tolist()}")

    # logits: bit-identical between forward and route, within 1e-5 of the oracle
    assert torch.equal(ex["logits"], logits), "forward and moe_route logits differ"
    L_ref = M.router_logits(inp["x"], inp["W_g"], inp["logit_bias"])
    res["logit_rel_err"] = rel_logit_err(L_gpu, L_ref)
    assert res["logit_rel_err"] <= 1e-5, res

    # routing from the GPU's own fp32 logits: indices bit-exact
    r = M.route_topk(L_gpu, k)
    assert np.array_equal(idx.cpu().numpy(), r.idx), "top-k indices differ"
    assert np.array_equal(ex["topk_idx"].cpu().numpy(), r.idx)
    np.testing.assert_allclose(gw.cpu().double().numpy(), r.w, rtol=2e-7, atol=1e-7)
    res["key_abs_err"] = float(np.max(np.abs(gkey.cpu().numpy() - r.key))) if T else 0.0
    assert res["key_abs_err"] <= 1e-12 * max(1.0, float(np.max(np.abs(r.key)))), res

    C = M.capacity(T, N, k, w.capacity_factor)
    assert C == lib.moe_capacity(T, N, k, w.capacity_factor)
    od = M.capacity_dispatch(r.idx, r.key, r.w, N, C, first_come=first_come)
    S = od.S
    g_off = disp["offsets"].cpu().numpy()
    g_perm = disp["perm"].cpu().numpy()[:S]
    g_inv = disp["inv"].cpu().numpy()[:T * k]
    assert np.array_equal(disp["req_counts"].cpu().numpy(), od.req_counts)
    assert np.array_equal(disp["counts"].cpu().numpy(), od.counts)
    assert np.array_equal(g_off, od.offsets)
    assert int(disp["n_dropped"].item()) == od.n_dropped
    res["S"], res["n_dropped"], res["C"] = S, od.n_dropped, C
    exact = np.array_equal(g_perm, od.perm) and np.array_equal(g_inv, od.inv)
    if not exact and not first_come:
        gap = capacity_cut_gap(r.idx, r.key, N, C)
        assert gap < 1e-12, f"perm/inv differ and no near-tie at a capacity cut (gap {gap})"
        check_dispatch_valid(r.idx, r.key, gkey.cpu().numpy(), N, C, g_perm, g_inv, g_off, k)
        say(f"[note] near-tie at a capacity cut (gap {gap}); validity checked")
        od = M.Dispatch(C=C, req_counts=od.req_counts, counts=od.counts, offsets=od.offsets,
                        perm=g_perm.astype(np.int32), inv=g_inv.astype(np.int32),
                        slot_gate=r.w.reshape(-1)[g_perm], n_dropped=od.n_dropped)
    else:
        assert exact, "first-come perm/inv differ (no ties are possible)"
    if renorm:
        od = M.renormalise_survivors(od, r.w, k)
        # fp32 w / fp32 sum of the kept w against the fp64 quotient
        np.testing.assert_allclose(disp["slot_gate"].cpu().double().numpy()[:S], od.slot_gate,
                                   rtol=4 * (k + 2) * EPS32, atol=0)
    elif exact:
        np.testing.assert_array_equal(disp["slot_gate"].cpu().numpy()[:S],
                                      gw.cpu().numpy().reshape(-1)[od.perm])
    assert np.array_equal(ex["inv"].cpu().numpy()[:T * k], g_inv)
    assert np.array_equal(ex["counts"].cpu().numpy(), od.counts)
    assert np.array_equal(ex["req_counts"].cpu().numpy(), od.req_counts)
    assert int(ex["n_dropped"].item()) == od.n_dropped

    # layer output
    say(f"[step] oracle output {w.name}")
    O = M.expert_slots_out(inp["x"], od, k, inp["W1"], inp["b1"], inp["W2"], inp["b2"])
    y_ref = M.combine(O, od, T, k, w.d, x_fallback=inp["x"] if identity else None)
    del O
    toks = np.arange(T)
    y_gpu = y32.cpu().double().numpy()[toks]
    diff = np.abs(y_gpu - y_ref)
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    err = float(np.max(diff)) if y_ref.size else 0.0
    res["y_rms"], res["y_max_abs_err"], res["y_err_over_rms"] = rms, err, err / rms if rms else 0.0

    say(f"[step] error bound {w.name}")
    u_h = EPS32 if w.dtype == "f32" else (2.0 ** -16 + EPS32 if split else U_BF16)
    bound = output_error_bound(inp, od, k, toks, u_h, gelu_abs=0.0 if w.dtype == "f32" else 5e-7)
    over = diff > bound
    res["worst_err_over_bound"] = float(np.max(diff / np.maximum(bound, 1e-300))) if diff.size else 0.0
    assert not over.any(), f"{int(over.sum())} outputs exceed the arithmetic error bound {res}"
    tol = 1e-4 if w.dtype == "f32" else 2e-2
    res["strict_tol"] = tol
    if strict is None:
        strict = not heavy_drop_plain(w.dtype, split, od.n_dropped / max(1, T * k), identity)
    res["strict"] = bool(strict)
    record("layer", w.name + (f"_f{flags}" if flags else ""), res)
    if strict:
        assert err <= tol * rms, res
    # fully dropped tokens are exactly zero, or exactly their input row with
    # the identity fallback
    dropped_all = np.all(od.inv.reshape(T, k) < 0, axis=1)
    res["fully_dropped"] = int(dropped_all.sum())
    if dropped_all.any():
        sel = torch.as_tensor(np.nonzero(dropped_all)[0], device=y32.device)
        if identity:
            assert torch.equal(y32[sel], dv["x"][sel].float())
            assert torch.equal(y_act[sel].view(torch.uint8), dv["x"][sel].view(torch.uint8))
        else:
            assert torch.count_nonzero(y32[sel]) == 0 and torch.count_nonzero(y_act[sel]) == 0

    if check_compose:
        say(f"[step] sub-call composition + determinism {w.name}")
        so = lib.moe_expert_ffn(dv["x"], disp["perm"], disp["offsets"], disp["slot_gate"], dv["W1"],
                                dv["b1"], dv["W2"], dv["b2"], k, w.capacity_factor,
                                flags=flags & lib.MOE_FLAG_HIDDEN_SPLIT)
        y2 = lib.moe_combine(so, disp["inv"], T, k, dtype=y_act.dtype,
                             x=dv["x"] if identity else None,
                             flags=lib.MOE_FLAG_IDENTITY_FALLBACK if identity else 0)
        y3 = lib.moe_forward(dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"], dv["W2"],
                             dv["b2"], k, w.capacity_factor, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.uint8), y_act.view(torch.uint8)), \
            "sub-calls do not compose to the forward's bits"
        assert torch.equal(y3.view(torch.uint8), y_act.view(torch.uint8)), "forward not deterministic"
    say(f"[ok] {w.name} {res} ({time.time() - t0:.1f}s)")
    return res
