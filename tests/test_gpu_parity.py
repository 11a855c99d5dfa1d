"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small and medium cases get a full element-by-element comparison; the five
full-size workloads run in the launch configuration the benchmark times and
are checked on every routing decision and on sampled output rows.
Bars:
  * logits within 1e-5 relative (max |dL| / max(|L|, rms L));
  * top-k indices, request/kept counts, offsets, permutation, inverse map and
    drop set bit-exact against the oracle fed the GPU's fp32 logits;
  * every output element within the a-priori error bound of the path's
    arithmetic (tests/gpu_util.py, output_error_bound);
  * for the named workloads, max |dy| <= 2e-2 x RMS(y) (bf16) or
    1e-4 x RMS(y) (fp32) on the fp32 output;
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
    # the documented maxima: N = 1024 experts with k = 16 (the widest top-k
    # rows), d = 65536 (router and first GEMM over the longest K), d_ff = 65536
    ("max_N_k", 256, 64, 64, 1024, 16, 1.0, "bf16", False, "normal0.5", 0),
    ("max_d", 8, 65536, 64, 4, 2, 0.0, "bf16", False, "none", 0),
    ("max_dff", 8, 64, 65536, 4, 2, 0.0, "bf16", True, "none", 0),
    ("dense_k_eq_N", 128, 64, 128, 4, 4, 0.0, "bf16", False, "none", 0),
    ("single_token", 1, 64, 64, 8, 2, 0.0, "bf16", False, "none", 0),
    ("capacity_one", 64, 64, 64, 8, 2, 0.01, "bf16", False, "zipf1.1", 0),
    ("many_experts_N1000", 512, 64, 64, 1000, 16, 1.0, "bf16", False, "none", 0),
]

# Named workloads: hidden-split where the weight stream bounds the time and the
# plain bf16 hidden layer cannot meet 2e-2 x RMS (heavy drops skew y).
FULL = {"switch_top1": SPLIT, "decode": 0, "fine_grained": SPLIT, "mixtral_prefill": 0}


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
    workgroup) for the per-XCD work queue; checked on sampled tokens."""
    from gpu_util import run_and_compare
    w = Workload("prefill_queue", T=4096, d=256, d_ff=16384, N=2, k=2, capacity_factor=0.0,
                 dtype="bf16", ffn_bias=True, skew="none", seed=0)
    run_and_compare(w, lib, sample_tokens=32)


def test_parity_tiled128_work_queue(lib):
    """Capacity-limited layer whose 128x128 GEMMs both have enough tiles for
    the per-XCD work queues (with the split hidden layer); sampled tokens."""
    from gpu_util import run_and_compare
    w = Workload("tiled128_queue", T=4096, d=2048, d_ff=4096, N=16, k=2, capacity_factor=1.0,
                 dtype="bf16", ffn_bias=True, skew="normal0.5", seed=0)
    run_and_compare(w, lib, sample_tokens=32, flags=1)


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
    res = run_and_compare(w, lib, inputs=inp, sample_tokens=64)
    assert res["n_dropped"] > 0


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(FULL))
def test_parity_full_size(lib, name):
    from gpu_util import run_and_compare
    run_and_compare(WORKLOADS[name], lib, sample_tokens=24, flags=FULL[name], strict=True,
                    check_compose=(name != "mixtral_prefill"))
