"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case, the five full-size workloads included (in the launch
configuration the benchmark times), is compared element by element on every
token: every logit, every routing decision, every output element.
Bars:
  * logits within 1e-5 relative (max |dL| / max(|L|, rms L));
  * top-k indices, request/kept counts, offsets, permutation, inverse map and
    drop set bit-exact against the oracle fed the GPU's fp32 logits;
  * every output element within the a-priori error bound of the path's
    arithmetic (tests/gpu_util.py, output_error_bound);
  * max |dy| <= 2e-2 x RMS(y) (bf16) or 1e-4 x RMS(y) (fp32) on the fp32
    output, for every case but the plain bf16 hidden layer with more than half
    of the picks dropped (tests/gpu_util.py, heavy_drop_plain: those shapes
    are repeated with the hi+lo hidden layer, which is held to it);
  * the activation-dtype output equals the fp32 output rounded once;
  * sub-calls compose to the forward's bits; repeated runs are bit-identical.
"""
from __future__ import annotations

import pytest
import torch

from moe_inputs import WORKLOADS, Workload

pytestmark = pytest.mark.gpu

SPLIT = 1  # MOE_FLAG_HIDDEN_SPLIT

CASES = [
    # name, T, d, d_ff, N, k, cf, dtype, bias, skew, flags
    ("f32_drops", 300, 64, 96, 6, 3, 0.5, "f32", True, "none", 0),
    ("f32_ktail_N5", 77, 40, 24, 5, 2, 1.0, "f32", True, "normal0.5", 0),
    ("decode_small", 32, 256, 384, 8, 2, 0.0, "bf16", False, "none", 0),
    ("decode_bias_ktail", 40, 200, 136, 8, 2, 0.0, "bf16", True, "none", 0),
    ("decode_split", 40, 200, 136, 8, 2, 0.0, "bf16", True, "none", SPLIT),
    ("decode_splitk", 24, 512, 4096, 4, 2, 0.0, "bf16", True, "none", 0),
    ("decode_splitk_hilo", 24, 512, 4096, 4, 2, 0.0, "bf16", True, "none", SPLIT),
    ("decode_splitk_tail", 24, 2048, 6400, 6, 2, 0.0, "bf16", True, "normal0.5", 0),
    ("decode_splitk_tail_hilo", 20, 2048, 6400, 6, 2, 0.0, "bf16", False, "none", SPLIT),
    ("decode_64_slots", 64, 256, 512, 2, 2, 0.0, "bf16", False, "none", 0),
    ("decode_64_slots_hilo", 64, 256, 512, 2, 2, 0.0, "bf16", True, "normal0.5", SPLIT),
    ("tiledM_ragged", 600, 256, 320, 4, 2, 1.0, "bf16", False, "none", 0),
    ("tiledM_bias_ktail", 500, 200, 136, 3, 1, 0.0, "bf16", True, "none", 0),
    ("tiledM_split", 600, 256, 320, 4, 2, 1.0, "bf16", True, "none", SPLIT),
    ("tiledL_ragged", 2048, 512, 768, 2, 1, 0.0, "bf16", False, "none", 0),
    ("switch_small", 1024, 128, 256, 16, 1, 1.0, "bf16", False, "normal0.5", 0),
    ("switch_small_split", 1024, 128, 256, 16, 1, 1.0, "bf16", False, "normal0.5", SPLIT),
    ("fine_small_zipf", 2048, 128, 64, 64, 8, 1.25, "bf16", False, "zipf1.1", 0),
    ("router_N13", 256, 64, 64, 13, 3, 1.0, "bf16", False, "normal0.5", 0),
    # N*d too large to stage W_g^T in LDS: the transposed-copy router path
    ("router_transposed_N64", 256, 768, 64, 64, 2, 1.0, "bf16", False, "normal0.5", 0),
    # 64 < N <= 256: top-k rows in 16-lane groups (8 and 16 experts per lane)
    ("router_N100_groups", 300, 64, 64, 100, 4, 1.0, "bf16", False, "zipf1.1", 0),
    ("router_N256_groups", 333, 128, 64, 256, 8, 1.25, "bf16", False, "zipf1.1", 0),
    # the heavy-drop shapes with the hi+lo hidden layer, held to 2e-2 x RMS(y)
    ("fine_small_zipf_split", 2048, 128, 64, 64, 8, 1.25, "bf16", False, "zipf1.1", SPLIT),
    ("router_N100_groups_split", 300, 64, 64, 100, 4, 1.0, "bf16", False, "zipf1.1", SPLIT),
    ("router_N256_groups_split", 333, 128, 64, 256, 8, 1.25, "bf16", False, "zipf1.1", SPLIT),
    ("capacity_one_split", 64, 64, 64, 8, 2, 0.01, "bf16", False, "zipf1.1", SPLIT),
    # the documented maxima: N = 1024 experts with k = 16 (the widest top-k
    # rows), d = 65536 (router and first GEMM over the longest K), d_ff = 65536
    ("max_N_k", 256, 64, 64, 1024, 16, 1.0, "bf16", False, "normal0.5", 0),
    # top-12 with drops on rows wide enough for the combine's ballot path (and
    # single-pick tokens written by the second GEMM)
    ("topk12_wide_rows", 512, 512, 256, 16, 12, 0.2, "bf16", False, "zipf1.1", 0),
    ("max_d", 8, 65536, 64, 4, 2, 0.0, "bf16", False, "none", 0),
    ("max_dff", 8, 64, 65536, 4, 2, 0.0, "bf16", True, "none", 0),
    ("dense_k_eq_N", 128, 64, 128, 4, 4, 0.0, "bf16", False, "none", 0),
    # small batches without capacity limit, 3 and 4 column tiles of 16 experts
    # in the skinny router, 1024 pairs
    ("small_route_N40", 48, 256, 128, 40, 4, 0.0, "bf16", True, "normal0.5", 0),
    ("small_route_N64_k16", 64, 128, 64, 64, 16, 0.0, "bf16", False, "zipf1.1", 0),
    ("small_route_T17_split", 17, 512, 256, 8, 2, 0.0, "bf16", True, "none", SPLIT),
    # few tokens with d % 128 == 0: the split-K router, whose partial logits
    # the dispatch block adds before its top-k (forward) or a top-k kernel
    # adds (moe_route); with capacity drops (the selection after it), a ragged
    # 37 tokens over 2 column tiles, one token with one partial, and d = 16384
    # (two K steps per wave, 64 partials)
    ("few_tokens_drops", 64, 256, 128, 8, 2, 0.5, "bf16", True, "zipf1.1", 0),
    ("few_tokens_N24_ragged", 37, 384, 128, 24, 3, 0.75, "bf16", False, "normal0.5", 0),
    ("few_tokens_single", 1, 128, 64, 8, 2, 0.0, "bf16", False, "none", 0),
    ("few_tokens_long_d", 5, 16384, 64, 16, 4, 0.0, "bf16", True, "none", 0),
    ("single_token", 1, 64, 64, 8, 2, 0.0, "bf16", False, "none", 0),
    ("capacity_one", 64, 64, 64, 8, 2, 0.01, "bf16", False, "zipf1.1", 0),
    ("many_experts_N1000", 512, 64, 64, 1000, 16, 1.0, "bf16", False, "none", 0),
    # the one-kernel wide router with fewer than 64 experts (columns padded to
    # 128; W_g too large to stage in LDS) and a ragged last block of 64 tokens
    ("wide_router_N40", 4100, 1408, 64, 40, 3, 1.0, "bf16", False, "normal0.5", 0),
]

# Named workloads in the configuration the benchmark times: the hi+lo hidden
# layer where the plain bf16 one misses 2e-2 x RMS(y) (the fine-grained layer,
# 82% of picks dropped), plain bf16 elsewhere.
FULL = {"switch_top1": 0, "decode": 0, "fine_grained": SPLIT, "mixtral_prefill": 0}


def _wl(c) -> Workload:
    name, T, d, d_ff, N, k, cf, dt, bias, skew, _ = c
    return Workload(name, T=T, d=d, d_ff=d_ff, N=N, k=k, capacity_factor=cf, dtype=dt,
                    ffn_bias=bias, skew=skew, seed=0)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mixture_experts_43_amd as m
    return m


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_parity_small(lib, case):
    from gpu_util import run_and_compare
    run_and_compare(_wl(case), lib, flags=case[-1])


def test_parity_tiny_f32_full(lib):
    from gpu_util import run_and_compare
    run_and_compare(WORKLOADS["tiny_f32"], lib, strict=True)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_empty_batch(lib, dt):
    """T = 0 is a successful no-op through every entry point of the binding."""
    from gpu_util import to_dev
    from moe_inputs import make_inputs
    w = Workload("empty", T=0, d=64, d_ff=128, N=8, k=2, capacity_factor=1.0, dtype=dt,
                 ffn_bias=True, skew="none")
    dv = to_dev(make_inputs(w))
    args = (dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"], dv["W2"], dv["b2"], 2, 1.0)
    y = lib.moe_forward(*args)
    y32, ex = lib.moe_forward(*args, flags=lib.MOE_FLAG_Y_F32, want_routing=True)
    yec = lib.moe_forward(*args, flags=lib.MOE_FLAG_EXPERT_CHOICE | lib.MOE_FLAG_IDENTITY_FALLBACK)
    ysh = lib.moe_forward(*args, shared_out=torch.empty((0, 64), dtype=torch.float32, device="cuda"))
    logits, idx, gw, gkey = lib.moe_route(dv["x"], dv["W_g"], dv["logit_bias"], 2)
    disp = lib.moe_dispatch(idx, gw, gkey, 8, 1.0)
    stats = lib.moe_routing_stats(logits, idx)
    torch.cuda.synchronize()
    for t in (y, y32, yec, ysh):
        assert t.shape == (0, 64)
    assert logits.shape == (0, 8) and idx.shape == (0, 2)
    assert disp["perm"].numel() >= 0 and stats.shape == (18,)


def test_parity_prefill_work_queue(lib):
    """Enough 256x256 tiles in the first GEMM (at least four per resident
    workgroup) for the per-XCD work queue."""
    from gpu_util import run_and_compare
    w = Workload("prefill_queue", T=4096, d=256, d_ff=16384, N=2, k=2, capacity_factor=0.0,
                 dtype="bf16", ffn_bias=True, skew="none", seed=0)
    run_and_compare(w, lib)


def test_parity_tiled128_work_queue(lib):
    """Capacity-limited layer whose 128x128 GEMMs both have enough tiles for
    the per-XCD work queues (with the split hidden layer)."""
    from gpu_util import run_and_compare
    w = Workload("tiled128_queue", T=4096, d=2048, d_ff=4096, N=16, k=2, capacity_factor=1.0,
                 dtype="bf16", ffn_bias=True, skew="normal0.5", seed=0)
    run_and_compare(w, lib, flags=1)


def test_identical_tokens_tie_break(lib):
    """Every token identical: equal keys at the cut keep the lowest tokens."""
    from gpu_util import run_and_compare
    from moe_inputs import make_inputs
    w = Workload("identical_tokens", T=96, d=64, d_ff=64, N=8, k=2, capacity_factor=0.5,
                 dtype="bf16", ffn_bias=False, skew="none")
    inp = make_inputs(w)
    inp["x"] = inp["x"][:1].repeat(w.T, 1).contiguous()
    res = run_and_compare(w, lib, inputs=inp)
    assert res["n_dropped"] > 0


def test_few_distinct_tokens_select(lib):
    """40960 pairs from three distinct token rows: an over-full expert's keys
    take three values, so the threshold bin of the capacity selection holds
    thousands of equal keys (the selection falls back from its short candidate
    list to passes over all keys); equal keys keep the lowest tokens."""
    from gpu_util import run_and_compare
    from moe_inputs import make_inputs
    w = Workload("three_token_rows", T=20480, d=64, d_ff=64, N=4, k=2, capacity_factor=0.7,
                 dtype="bf16", ffn_bias=False, skew="none")
    inp = make_inputs(w)
    rows = inp["x"][:3]
    inp["x"] = rows[torch.arange(w.T) % 3].contiguous()
    res = run_and_compare(w, lib, inputs=inp)
    assert res["n_dropped"] > 0


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(FULL))
def test_parity_full_size(lib, name):
    """Every token of the full-size workload, with the sub-call composition."""
    from gpu_util import run_and_compare
    run_and_compare(WORKLOADS[name], lib, flags=FULL[name])


@pytest.mark.slow
@pytest.mark.parametrize("name", ["switch_top1", "fine_grained"])
def test_other_hidden_full_size(lib, name):
    """The other hidden-layer form at the two capacity-limited workloads: the
    hi+lo pair at the Switch-style layer (held to 2e-2 x RMS(y)), the plain
    bf16 layer at the fine-grained one (routing bit-exact, every element within
    the arithmetic error bound, not held to 2e-2 x RMS(y): with 82% of the
    picks dropped, RMS(y) is small against the rows that keep a large gate, and
    the hidden layer's bf16 rounding alone reaches that bar; the measured ratio
    is recorded)."""
    from gpu_util import record, run_and_compare, say
    plain = FULL[name] == SPLIT
    res = run_and_compare(WORKLOADS[name], lib, flags=0 if plain else SPLIT,
                          strict=None if plain else True, check_compose=False)
    say(f"[{'plain-bf16' if plain else 'hi+lo'}] {name} max|dy|/rms(y) = "
        f"{res['y_err_over_rms']:.4e} (bar {res['strict_tol']:.0e})")
    record("plain_bf16_full" if plain else "split_full", name, res)


MISMATCH = [
    # name, T, d, d_ff, N, k, capacity factor of the dispatch, of the FFN call
    ("decode_path", 96, 256, 384, 8, 2, 0.0, 1.0),
    ("tiled_path", 600, 256, 320, 4, 2, 0.0, 0.5),
]


@pytest.mark.parametrize("case", MISMATCH, ids=[c[0] for c in MISMATCH])
def test_ffn_offsets_from_larger_capacity(lib, case):
    """moe_expert_ffn given the dispatch of a larger capacity factor than its
    own (an API misuse): the kernels clamp each expert's rows to the call's
    capacity C and all rows to min(T*k, N*C), so every access stays inside the
    buffers planned for the call. The rows inside those bounds equal the
    consistent call's (up to fp32 summation order); every other slot_out row
    keeps the value it held before the call."""
    import numpy as np
    from gpu_util import say, to_dev
    from moe_inputs import make_inputs
    name, T, d, d_ff, N, k, cf_disp, cf_ffn = case
    w = Workload(name, T=T, d=d, d_ff=d_ff, N=N, k=k, capacity_factor=cf_disp, dtype="bf16",
                 ffn_bias=True, skew="normal0.5", seed=2)
    say(f"[case] mismatched capacity {name} T={T} d={d} d_ff={d_ff} N={N} k={k} "
        f"dispatch cf={cf_disp} ffn cf={cf_ffn}")
    dv = to_dev(make_inputs(w))
    _, idx, gw, gkey = lib.moe_route(dv["x"], dv["W_g"], dv["logit_bias"], k)
    disp = lib.moe_dispatch(idx, gw, gkey, N, cf_disp)
    args = (dv["x"], disp["perm"], disp["offsets"], disp["slot_gate"], dv["W1"], dv["b1"],
            dv["W2"], dv["b2"], k)
    good = lib.moe_expert_ffn(*args, cf_disp)
    sentinel = torch.full((T * k, d), float("nan"), dtype=torch.float32, device="cuda")
    so = lib.moe_expert_ffn(*args, cf_ffn, slot_out=sentinel.clone())
    torch.cuda.synchronize()
    off = disp["offsets"].cpu().numpy().astype(np.int64)
    C = lib.moe_capacity(T, N, k, cf_ffn)
    S_max = min(T * k, N * C)
    computed = np.zeros(T * k, dtype=bool)
    for e in range(N):
        a = min(off[e], S_max)
        b = min(off[e + 1], S_max)
        computed[a:a + min(b - a, C)] = True
    assert off[-1] > S_max or np.any(np.diff(off) > C), "the case must need the clamp"
    got = so.cpu().numpy()
    ref = good.cpu().numpy()
    assert np.all(np.isnan(got[~computed])), "a row outside the call's bounds was written"
    assert np.all(np.isfinite(got[computed]))
    np.testing.assert_allclose(got[computed], ref[computed], rtol=1e-4,
                               atol=1e-4 * float(np.abs(ref[computed]).max()))
    say(f"[ok] {name}: {int(computed.sum())} of {int(off[-1])} rows computed")
