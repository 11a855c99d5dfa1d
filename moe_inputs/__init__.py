"""Seeded synthetic inputs for the sparse MoE layer forward.

This module is shared by the CPU oracle and the GPU path. It holds the
workload table and the random-number recipe only: no routing, capacity,
expert or combine arithmetic lives here.

Recipe (one ``torch.Generator`` on the CPU, seeded per workload, drawing
fp32 standard normals in this fixed order):

    x      [T, d]        ~ N(0, 1)
    W_g    [d, N]        ~ N(0, 0.02^2)       router weight, x @ W_g (router
                                               init range on the "Mixture of
                                               Experts (MoE): Architecture,
                                               Routing, and Scaling" page,
                                               section "Initialization
                                               Strategies")
    bias   [N]  (fp32)   per-workload logit skew (see ``logit_bias``)
    W1     [N, d_ff, d]  ~ N(0, 1/d)           nn.Linear(d, d_ff) layout [out, in]
    b1     [N, d_ff]     ~ N(0, 0.01^2)        only where the workload has biases
    W2     [N, d, d_ff]  ~ N(0, 1/d_ff)        nn.Linear(d_ff, d) layout [out, in]
    b2     [N, d]        ~ N(0, 0.01^2)        only where the workload has biases

A shared expert (``make_shared_expert``) has a generator of its own, seeded
with the workload seed + 7919, drawing in this order:

    W1s    [d_fs, d]     ~ N(0, 1/d)
    b1s    [d_fs]        ~ N(0, 0.01^2)        only where the workload has biases
    W2s    [d, d_fs]     ~ N(0, 1/d_fs)
    b2s    [d]           ~ N(0, 0.01^2)        only where the workload has biases

Each tensor is drawn in fp32, scaled, then rounded once (round-to-nearest-
even) to the workload's activation dtype. Both sides consume exactly these
rounded values; the logit bias stays fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "get_workload", "make_inputs", "make_shared_expert",
           "scaled"]


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    d_ff: int
    N: int
    k: int
    capacity_factor: float  # <= 0 means "no capacity limit"
    dtype: str  # "f32" or "bf16"
    ffn_bias: bool
    skew: str  # "none" | "normal0.5" | "zipf1.1"
    seed: int = 0
    note: str = field(default="", compare=False)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads of the layer as measured here. Seeds are 0 throughout.
WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", T=256, d=128, d_ff=512, N=8, k=2, capacity_factor=1.25,
        dtype="f32", ffn_bias=True, skew="none",
        note="tiny fp32 layer with FFN biases, capacity factor 1.25"),
    "switch_top1": Workload(
        "switch_top1", T=8192, d=1024, d_ff=4096, N=64, k=1, capacity_factor=1.0,
        dtype="bf16", ffn_bias=False, skew="normal0.5",
        note="Switch-style top-1, capacity factor 1.0, per-expert logit bias N(0,0.5^2)"),
    "mixtral_prefill": Workload(
        "mixtral_prefill", T=4096, d=4096, d_ff=14336, N=8, k=2, capacity_factor=0.0,
        dtype="bf16", ffn_bias=False, skew="none",
        note="Mixtral-shaped prefill, batch 2 x seq 2048, no capacity limit"),
    "decode": Workload(
        "decode", T=32, d=4096, d_ff=14336, N=8, k=2, capacity_factor=0.0,
        dtype="bf16", ffn_bias=False, skew="none",
        note="decode-shaped small batch, Mixtral dims, no capacity limit"),
    "fine_grained": Workload(
        "fine_grained", T=16384, d=2048, d_ff=512, N=256, k=8, capacity_factor=1.25,
        dtype="bf16", ffn_bias=False, skew="zipf1.1",
        note="256 fine-grained experts, top-8, capacity factor 1.25, Zipf(1.1) logit skew"),
}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None


def _torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "f32":
        return torch.float32
    if dtype == "bf16":
        return torch.bfloat16
    raise ValueError(f"unsupported dtype {dtype!r}")


def scaled(g: torch.Generator, shape, std: float, dtype: torch.dtype) -> torch.Tensor:
    """One fp32 standard-normal draw of ``shape``, times ``std``, rounded once to ``dtype``."""
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def logit_bias(w: Workload, g: torch.Generator) -> Optional[torch.Tensor]:
    """Per-expert fp32 logit skew of a workload, or None.

    ``normal0.5``: b_e ~ N(0, 0.5^2), drawn from the workload's generator.
    ``zipf1.1``:   b_e = -1.1 * ln(e + 1), so the prior routing odds of expert e
                   are proportional to (e + 1)^-1.1 (expert 0 most popular); no draw.
    """
    if w.skew == "none":
        return None
    if w.skew == "normal0.5":
        return torch.randn(w.N, generator=g, dtype=torch.float32).mul_(0.5)
    if w.skew == "zipf1.1":
        e = torch.arange(w.N, dtype=torch.float64)
        return (-1.1 * torch.log(e + 1.0)).to(torch.float32)
    raise ValueError(f"unknown skew {w.skew!r}")


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw the inputs of workload ``w`` on the CPU. Returns a dict of CPU tensors.

    Keys: x, W_g, logit_bias (or None), W1, b1 (or None), W2, b2 (or None).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    dt = _torch_dtype(w.dtype)
    x = scaled(g, (w.T, w.d), 1.0, dt)
    W_g = scaled(g, (w.d, w.N), 0.02, dt)
    bias = logit_bias(w, g)
    W1 = scaled(g, (w.N, w.d_ff, w.d), 1.0 / math.sqrt(w.d), dt)
    b1 = scaled(g, (w.N, w.d_ff), 0.01, dt) if w.ffn_bias else None
    W2 = scaled(g, (w.N, w.d, w.d_ff), 1.0 / math.sqrt(w.d_ff), dt)
    b2 = scaled(g, (w.N, w.d), 0.01, dt) if w.ffn_bias else None
    return {"x": x, "W_g": W_g, "logit_bias": bias, "W1": W1, "b1": b1, "W2": W2, "b2": b2}


def make_shared_expert(w: Workload, d_fs: Optional[int] = None,
                       seed: Optional[int] = None) -> dict:
    """Draw a shared expert's weights for workload ``w`` (hidden width ``d_fs``,
    default the workload's d_ff). Keys: W1s, b1s (or None), W2s, b2s (or None)."""
    d_fs = w.d_ff if d_fs is None else d_fs
    g = torch.Generator(device="cpu")
    g.manual_seed((w.seed if seed is None else seed) + 7919)
    dt = _torch_dtype(w.dtype)
    W1s = scaled(g, (d_fs, w.d), 1.0 / math.sqrt(w.d), dt)
    b1s = scaled(g, (d_fs,), 0.01, dt) if w.ffn_bias else None
    W2s = scaled(g, (w.d, d_fs), 1.0 / math.sqrt(d_fs), dt)
    b2s = scaled(g, (w.d,), 0.01, dt) if w.ffn_bias else None
    return {"W1s": W1s, "b1s": b1s, "W2s": W2s, "b2s": b2s}
