"""Benchmark of the sparse MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--configs all]

A step is one moe_forward call (router, dispatch, both expert GEMMs, combine)
on one batch of seeded synthetic inputs already resident in HBM. W untimed
warm-up steps, an untimed pass with a HIP event between every stage (the
per-stage breakdown, which also names the dominant expert GEMM), then exactly
K timed steps between two device synchronisations with nothing else on the
stream (value, ms_per_step), then K more steps each carrying the events the
library records around the dominant GEMM on its stream (the roofline's launch
duration). Prints ONE JSON line (metric, value in tokens/s, roofline of the
dominant kernel from those events, and the CPU oracle timed on a bounded
sample on the host). The other workloads are then timed the same way and
reported under "configs".
Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec + % of bf16 MFMA peak (or % HBM BW at small T)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
# Oracle sample (tokens whose outputs the CPU oracle computes) per workload,
# sized for roughly 10-30 s of host work; routing always covers every token.
CPU_SAMPLE = {"tiny_f32": 256, "switch_top1": 8192, "mixtral_prefill": 4096, "decode": 32,
              "fine_grained": 16384}
# Hidden layer per workload: the hi+lo pair where the plain bf16 hidden layer
# misses 2e-2 x RMS(y) at full size (the fine-grained layer), plain bf16 elsewhere.
DEFAULT_FLAGS = {"fine_grained": "split"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles from the process's HIP runtime (the one torch loaded).

    Created with hipEventDisableSystemFence: they only time work, and are read
    (hipEventElapsedTime) after a full device synchronisation, so they need no
    system-scope fence. With the default flags every record between two
    kernels writes back and invalidates the caches, which held the GPU idle for
    about 6 us per event in kernel traces of this benchmark."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.made = []

    def create(self):
        h = ctypes.c_void_p()
        if self.rt.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.made.append(h.value)
        return h.value

    def ms(self, a, b):
        out = ctypes.c_float()
        self.rt.hipEventSynchronize(ctypes.c_void_p(b))
        if self.rt.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def record(self, h, stream):
        if self.rt.hipEventRecord(ctypes.c_void_p(h), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def close(self):
        for h in self.made:
            self.rt.hipEventDestroy(ctypes.c_void_p(h))
        self.made = []


def source_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "sparse_mixture_experts_43_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel):
    """HBM bytes per call of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a copy probe), if its counters were taken on
    the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    try:
        text = open(p).read()
    except OSError:
        return None
    m = re.search(r"^source_hash: (\w+)", text, re.M)
    if m is None or m.group(1) != source_hash():
        return None
    m = re.search(r"^traffic\[" + re.escape(kernel) + r"\] = ([0-9.eE+-]+)", text, re.M)
    return None if m is None else float(m.group(1))


def cpu_baseline(w, inp, sample, budget_s=10.0):
    import numpy as np
    import oracle

    toks = np.unique(np.linspace(0, w.T - 1, min(sample, w.T)).astype(np.int64))
    # repeat the same sample until about budget_s of host work (at most 8 passes)
    reps = 0
    t0 = time.perf_counter()
    while reps < 8 and (reps == 0 or time.perf_counter() - t0 < budget_s):
        oracle.moe_forward(inp["x"], inp["W_g"], inp["logit_bias"], inp["W1"], inp["b1"], inp["W2"],
                           inp["b2"], w.k, w.capacity_factor, tokens=toks)
        reps += 1
    dt = time.perf_counter() - t0
    threads = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 0) for i in info), default=None)
    except Exception:  # noqa: BLE001
        pass
    if not threads:
        threads = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    what = (f"all {w.T} tokens" if len(toks) == w.T else
            f"{len(toks)} evenly spaced tokens (routing and capacity still over all {w.T})")
    return {
        "value": reps * len(toks) / dt,
        "unit": "tokens/s",
        "cores": int(threads),
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"fp64 numpy oracle, one layer forward over {what}, {reps} pass(es); "
                  f"{dt:.1f} s wall",
    }


def measure_extras(moe, torch, w, dv, ws, y, flags):
    """After the timed region: moe_routing_stats on this input's logits and
    top-k ids (20 calls), the layer with every drop-policy flag, with
    expert-choice routing, and with a shared expert (20 steps each)."""
    _, rx = moe.moe_forward(dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"], dv["W2"],
                            dv["b2"], w.k, w.capacity_factor, workspace=ws, want_routing=True,
                            flags=flags)
    nx = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stats = moe.moe_routing_stats(rx["logits"], rx["topk_idx"], workspace=ws)
    e0.record()
    for _ in range(nx):
        moe.moe_routing_stats(rx["logits"], rx["topk_idx"], workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    stats_us = e0.elapsed_time(e1) * 1e3 / nx
    st_h = stats.cpu()
    pol = (flags | moe.MOE_FLAG_FIRST_COME | moe.MOE_FLAG_RENORM_SURVIVORS
           | moe.MOE_FLAG_IDENTITY_FALLBACK)

    def pstep():
        moe.moe_forward(dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"], dv["W2"],
                        dv["b2"], w.k, w.capacity_factor, workspace=ws, y=y, flags=pol)

    for _ in range(3):
        pstep()
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    for _ in range(nx):
        pstep()
    torch.cuda.synchronize()
    pol_ms = (time.perf_counter() - tp0) * 1e3 / nx
    ecf = flags | moe.MOE_FLAG_EXPERT_CHOICE

    def estep():
        moe.moe_forward(dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"], dv["W2"],
                        dv["b2"], w.k, w.capacity_factor, workspace=ws, y=y, flags=ecf)

    for _ in range(3):
        estep()
    torch.cuda.synchronize()
    te0 = time.perf_counter()
    for _ in range(nx):
        estep()
    torch.cuda.synchronize()
    ec_ms = (time.perf_counter() - te0) * 1e3 / nx
    # a shared expert of the routed experts' width on every token
    from moe_inputs import make_shared_expert
    sh = {k_: (None if v is None else v.to(dv["x"].device)) for k_, v in
          make_shared_expert(w).items()}
    sflags = flags & moe.MOE_FLAG_HIDDEN_SPLIT
    sws = moe.alloc_workspace(moe.moe_shared_workspace_bytes(w.T, w.d, w.d_ff, dv["x"].dtype),
                              dv["x"].device)
    sout = torch.empty((w.T, w.d), dtype=torch.float32, device=dv["x"].device)

    def shstep():
        moe.moe_shared_expert(dv["x"], sh["W1s"], sh["b1s"], sh["W2s"], sh["b2s"], workspace=sws,
                              flags=sflags, out=sout)

    def sstep():
        shstep()
        moe.moe_forward(dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"], dv["W2"],
                        dv["b2"], w.k, w.capacity_factor, workspace=ws, y=y, flags=flags,
                        shared_out=sout)

    for _ in range(3):
        sstep()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(nx):
        shstep()
    e1.record()
    torch.cuda.synchronize()
    sh_ms = e0.elapsed_time(e1) / nx
    ts0 = time.perf_counter()
    for _ in range(nx):
        sstep()
    torch.cuda.synchronize()
    ss_ms = (time.perf_counter() - ts0) * 1e3 / nx
    sh_tflops = 4.0 * w.T * w.d * w.d_ff / (sh_ms * 1e-3) / 1e12  # algorithmic flops
    # the same step captured once in a HIP graph and replayed (the library
    # enqueues kernels only, so the forward is capturable as it is)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"], dv["W2"],
                        dv["b2"], w.k, w.capacity_factor, workspace=ws, y=y, flags=flags)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    # eager and graph blocks alternate (two of each): the clock drifts over a
    # run by a few percent, which a single graph block timed after the others
    # would read as a graph cost
    blk = {"eager": [], "graph": []}
    for _ in range(2):
        for mode in ("eager", "graph"):
            tg0 = time.perf_counter()
            for _ in range(nx):
                if mode == "graph":
                    g.replay()
                else:
                    moe.moe_forward(dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"],
                                    dv["W2"], dv["b2"], w.k, w.capacity_factor, workspace=ws, y=y,
                                    flags=flags)
            torch.cuda.synchronize()
            blk[mode].append((time.perf_counter() - tg0) * 1e3 / nx)
    graph_ms = sum(blk["graph"]) / 2
    eager_alt_ms = sum(blk["eager"]) / 2
    del g
    C = moe.moe_capacity(w.T, w.N, w.k, w.capacity_factor)
    extras = {"routing_stats_us": stats_us, "aux_balance": float(st_h[2 * w.N]),
              "z_mean_lse_sq": float(st_h[2 * w.N + 1]),
              "all_drop_policies_ms_per_step": pol_ms,
              "expert_choice_ms_per_step": ec_ms,
              "expert_choice_slots": w.N * min(C, w.T),
              "shared_expert_ms": sh_ms,
              "shared_expert_tflops": sh_tflops,
              "with_shared_expert_ms_per_step": ss_ms,
              "graph_replay_ms_per_step": graph_ms,
              "eager_ms_per_step_beside_graph": eager_alt_ms,
              "note": "after the timed steps; moe_routing_stats averaged over 20 calls, the layer "
                      "with first-come capacity + survivor renormalisation + identity fallback "
                      "over 20 steps, with expert-choice routing (every expert takes "
                      "min(C, T) tokens) over 20 steps, a shared expert of width d_ff on every "
                      "token alone (HIP events, 20 calls; TFLOP/s = 4 T d d_ff / time) and "
                      "added to the layer (20 steps), and the plain step captured in a HIP "
                      "graph and replayed, in two blocks of 20 replays alternating with two blocks of "
                      "20 eager steps (both averaged: the same clock conditions)"}
    log(f"extras: routing stats {stats_us:.1f}us, aux {extras['aux_balance']:.4f}, "
        f"all drop policies {pol_ms:.3f} ms/step, expert choice {ec_ms:.3f} ms/step "
        f"({extras['expert_choice_slots']} slots), shared expert {sh_ms:.3f} ms "
        f"({sh_tflops:.0f} TFLOP/s), layer + shared expert {ss_ms:.3f} ms/step, "
        f"graph replay {graph_ms:.3f} ms/step (eager beside it {eager_alt_ms:.3f})")
    return extras


def run_workload(moe, torch, w, fl, steps, warmup, want_extras, cpu_budget_s, copy_probe_mib=0,
                 pack=True):
    """Times one workload: W warm-up steps, an untimed pass with stage events,
    then exactly K timed steps. Returns the workload's record (value, roofline
    of the dominant expert GEMM, layer figures, CPU oracle baseline)."""
    from moe_inputs import make_inputs

    flags = moe.MOE_FLAG_Y_F32 | (moe.MOE_FLAG_HIDDEN_SPLIT if fl == "split" else 0)
    log(f"workload {w.name}: T={w.T} d={w.d} d_ff={w.d_ff} N={w.N} k={w.k} cf={w.capacity_factor} "
        f"dtype={w.dtype} flags={fl}+y_f32")
    t0 = time.time()
    inp = make_inputs(w)
    log(f"inputs drawn on the host in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    dv = {k: (None if v is None else v.to(dev).contiguous()) for k, v in inp.items()}
    # The expert weights in the library's packed layout, written once as a
    # model would at load time (a reordering of the same values; no step
    # includes it): bf16 layers with d and d_ff multiples of 128.
    packed = pack and w.dtype == "bf16" and w.d % 128 == 0 and w.d_ff % 128 == 0
    if packed:
        dv["W1"] = moe.moe_pack_weights(dv["W1"])
        dv["W2"] = moe.moe_pack_weights(dv["W2"])
        flags |= moe.MOE_FLAG_PACKED_WEIGHTS
        torch.cuda.synchronize()
        log("expert weights packed (moe_pack_weights, once, outside every timed region)")
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(w.T, w.d, w.d_ff, w.N, w.k, w.capacity_factor,
                                                     dv["x"].dtype), dev)
    y = torch.empty((w.T, w.d), dtype=torch.float32, device=dev)

    def step():
        moe.moe_forward(dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"], dv["W2"], dv["b2"],
                        w.k, w.capacity_factor, workspace=ws, y=y, flags=flags)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"warm-up done ({warmup} steps)")

    names = ["router", "dispatch", "schedule", "expert_gemm1", "expert_gemm2", "combine"]
    ev = HipEvents()
    # Per-stage breakdown from an untimed pass: an event between every stage
    # adds a few microseconds per event, so the timed steps below carry only
    # the two events around the dominant expert GEMM.
    nprof = max(3, min(steps, 10))
    pmarks = [[ev.create() for _ in range(7)] for _ in range(nprof)]
    for i in range(nprof):
        moe.moe_set_profile_events(pmarks[i])
        step()
    torch.cuda.synchronize()
    moe.moe_set_profile_events([])
    per = {n: 0.0 for n in names}
    for m in pmarks:
        for j, n in enumerate(names):
            per[n] += ev.ms(m[j], m[j + 1])
    per = {n: v / nprof for n, v in per.items()}
    dom = "expert_gemm1" if per["expert_gemm1"] >= per["expert_gemm2"] else "expert_gemm2"
    dslot = 3 if dom == "expert_gemm1" else 4  # event slots before / after that GEMM

    # Timed region: exactly K steps between two device synchronisations, with
    # nothing else on the stream. (An event recorded between two kernels held
    # the GPU idle about 4.5 us in kernel traces even without a system fence,
    # so no event is recorded here.)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_step = (t_end - t_start) * 1e3 / steps

    # Second region, the same K steps, each carrying the two events the library
    # records around the dominant expert GEMM on its stream, and one before its
    # router: the GEMM's average launch duration (the roofline) and each step's
    # GPU time.
    marks = [(ev.create(), ev.create()) for _ in range(steps)]
    starts = [ev.create() for _ in range(steps + 1)]
    torch.cuda.synchronize()
    for i in range(steps):
        slots = [None] * 7
        slots[0] = starts[i]
        slots[dslot], slots[dslot + 1] = marks[i]
        moe.moe_set_profile_events(slots)
        step()
    moe.moe_set_profile_events([])
    ev.record(starts[-1], torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    dom_ms = sum(ev.ms(a, b) for a, b in marks) / steps
    step_ms = sorted(ev.ms(starts[i], starts[i + 1]) for i in range(steps))
    step_med = (step_ms[(steps - 1) // 2] + step_ms[steps // 2]) / 2
    ev.close()
    log(f"timed {steps} steps: {ms_step:.3f} ms/step; event region: {dom} {dom_ms * 1e3:.1f}us, "
        f"steps median {step_med:.3f} ms (min {step_ms[0]:.3f}, with 3 events each); "
        f"stage breakdown (untimed pass with stage events): "
        + ", ".join(f"{n} {v * 1e3:.1f}us" for n, v in per.items()))

    # extras, after the timed region: the routing statistics pass (from this
    # input's logits and top-k ids) and the layer with every drop-policy flag
    extras = measure_extras(moe, torch, w, dv, ws, y, flags) if want_extras else None

    if copy_probe_mib > 0:
        n = copy_probe_mib << 18  # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {copy_probe_mib} MiB read + {copy_probe_mib} MiB written")
        del src, dst

    # routing statistics of the timed input (read back after timing)
    _, ex = moe.moe_forward(dv["x"], dv["W_g"], dv["logit_bias"], dv["W1"], dv["b1"], dv["W2"],
                            dv["b2"], w.k, w.capacity_factor, workspace=ws, want_routing=True,
                            flags=flags)
    torch.cuda.synchronize()
    counts = ex["counts"].cpu()
    S = int(counts.sum())
    touched = int((counts > 0).sum())
    dropped = int(ex["n_dropped"].item())

    es = 4 if w.dtype == "f32" else 2
    gemm_flops = 2.0 * S * w.d * w.d_ff  # per expert GEMM
    layer_flops = 2.0 * w.T * w.d * w.N + 2 * gemm_flops
    w_bytes = touched * w.d * w.d_ff * es  # one expert matrix set (W1 or W2) of touched experts
    layer_bytes = (w.T * w.d * es + w.d * w.N * es + 2 * w_bytes + w.T * w.d * 4
                   + (0 if inp["b1"] is None else touched * (w.d + w.d_ff) * es))
    # kernel-level algorithmic bytes: its weights + its unique activation inputs + its outputs
    g1_bytes = w_bytes + w.T * w.d * es + S * w.d_ff * es
    g2_bytes = w_bytes + S * w.d_ff * es + S * w.d * 4
    peak_f = PEAK_F32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
    intensity = layer_flops / layer_bytes
    bound = "mfma" if intensity > peak_f * 1e12 / (PEAK_HBM_GBPS * 1e9) else "hbm"
    traffic = load_traffic(w.name, dom)
    if bound == "mfma":
        achieved = gemm_flops / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak_f, "unit": "TFLOP/s",
                "frac": achieved / peak_f, "traffic": traffic, "kernel": dom,
                "launch_us": dom_ms * 1e3,
                "per_launch": f"{gemm_flops:.4g} flop (2*S*d*d_ff, S={S})"}
    else:
        kb = g1_bytes if dom == "expert_gemm1" else g2_bytes
        achieved = kb / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic, "kernel": dom,
                "launch_us": dom_ms * 1e3,
                "per_launch": f"{kb:.4g} B (touched-expert weights + activations in/out)"}
    layer_tflops = layer_flops / (ms_step * 1e-3) / 1e12
    layer_gbps = layer_bytes / (ms_step * 1e-3) / 1e9
    rec = {
        "value": w.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "ms_per_step": ms_step,
        "step_ms_gpu": {"median": step_med, "min": step_ms[0], "max": step_ms[-1],
                        "note": "per step of the event region (K more steps after the timed "
                                "region, each with an event before its router and two around "
                                "the dominant GEMM; the events add a few us per step)"},
        "dtype": "f32" if w.dtype == "f32" else "bf16",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "d_ff": w.d_ff, "N": w.N, "k": w.k,
                   "capacity_factor": w.capacity_factor, "hidden": fl, "y_dtype": "f32",
                   "expert_weights": "packed at load" if packed else "row-major",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer": {"tflops": layer_tflops, "frac_bf16_peak": layer_tflops / peak_f,
                  "alg_gbps": layer_gbps, "frac_hbm_peak": layer_gbps / PEAK_HBM_GBPS,
                  "bound": bound,
                  "frac_of_bound": (layer_tflops / peak_f if bound == "mfma"
                                    else layer_gbps / PEAK_HBM_GBPS),
                  "flop_per_byte": intensity, "S": S, "dropped_pairs": dropped,
                  "drop_rate": dropped / max(1, w.T * w.k), "touched_experts": touched,
                  "kept_per_expert": [int(c) for c in counts.tolist()],
                  "requests_per_expert": [int(c) for c in ex["req_counts"].cpu().tolist()]},
        "kernels_us": {n: v * 1e3 for n, v in per.items()},
        "kernels_us_note": "stage times from an untimed pass with an event between stages",
        "extras": extras,
    }
    log(f"{w.name}: {ms_step:.3f} ms/step, {rec['value']:.4g} tokens/s, {dom} "
        f"{roof['frac']:.3f} of {roof['bound']} peak; layer {rec['layer']['frac_of_bound']:.3f} "
        f"of {bound} peak")
    del dv, ws, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu_budget_s > 0:
        log(f"timing the CPU oracle on a {CPU_SAMPLE.get(w.name, 32)}-token sample")
        rec["cpu_baseline"] = cpu_baseline(w, inp, CPU_SAMPLE.get(w.name, 32), cpu_budget_s)
    else:
        rec["cpu_baseline"] = None
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_prefill",
                    help="the headline workload (value, roofline, cpu_baseline of the line)")
    ap.add_argument("--configs", default="all",
                    help="other workloads timed after the headline, under 'configs': 'all' "
                         "(every other workload), 'none', or a comma-separated list")
    ap.add_argument("--flags", default=None,
                    help="'split' for the bf16 hi+lo hidden layer, 'plain' for bf16 (headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the routing-statistics and drop-policy measurements after timing")
    ap.add_argument("--unpacked", action="store_true",
                    help="pass the expert weights row-major instead of packed once at load")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (the "
                         "reference dispatch that scales rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(expert parallelism is a design note only); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_mixture_experts_43_amd as moe
    from moe_inputs import WORKLOADS, get_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = get_workload(args.workload)
    fl = args.flags or DEFAULT_FLAGS.get(w.name, "plain")
    head = run_workload(moe, torch, w, fl, args.steps, args.warmup, not args.no_extras,
                        0 if args.no_cpu_baseline else 10.0, args.copy_probe_mib,
                        not args.unpacked)
    if args.configs == "all":
        others = [n for n in WORKLOADS if n != w.name]
    elif args.configs in ("", "none"):
        others = []
    else:
        others = [n for n in args.configs.split(",") if n and n != w.name]
    configs = {}
    for name in others:
        wo = get_workload(name)
        configs[name] = run_workload(moe, torch, wo, DEFAULT_FLAGS.get(name, "plain"), args.steps,
                                     args.warmup, False, 0 if args.no_cpu_baseline else 5.0,
                                     pack=not args.unpacked)
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "step_ms_gpu": head["step_ms_gpu"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded normal draws of the workload's shapes and distributions)",
        "config": head["config"],
        "roofline": head["roofline"],
        "layer": head["layer"],
        "kernels_us": head["kernels_us"],
        "kernels_us_note": head["kernels_us_note"],
        "extras": head["extras"],
        "source_hash": source_hash(),
        "cpu_baseline": head["cpu_baseline"],
        "configs": configs,
        "configs_note": "each other workload timed the same way after the headline (same steps "
                        "and warm-up; value, roofline of its dominant expert GEMM, the layer's "
                        "fraction of its bound, CPU oracle on a bounded sample)",
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
