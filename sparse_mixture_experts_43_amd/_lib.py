"""Python binding of libmoe (ctypes): argument marshalling only.

Each function has the name of the C entry point it calls (include/moe.h).
PyTorch supplies device memory and the current HIP stream; every step of the
layer runs in the library's HIP kernels. There is no fallback: if libmoe.so is
missing or fails to load, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_F32 = 0
MOE_BF16 = 1
MOE_FLAG_HIDDEN_SPLIT = 1
MOE_FLAG_Y_F32 = 2
MOE_FLAG_FIRST_COME = 4
MOE_FLAG_RENORM_SURVIVORS = 8
MOE_FLAG_IDENTITY_FALLBACK = 16
MOE_FLAG_EXPERT_CHOICE = 32
MOE_FLAG_PACKED_WEIGHTS = 64

_c_int, _c_size, _c_double, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_double, ctypes.c_void_p


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.moe_strerror(status).decode()
        if status == -4:
            msg += f" (hip error {_lib.moe_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmoe.so not found at {LIB_PATH}; build it first "
            "(python -c 'import __graft_entry__ as g; g.build()' or "
            "python sparse_mixture_experts_43_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "moe_version": (_c_int, []),
        "moe_strerror": (ctypes.c_char_p, [_c_int]),
        "moe_last_hip_error": (_c_int, []),
        "moe_capacity": (_c_int, [_c_int, _c_int, _c_int, _c_double]),
        "moe_workspace_bytes": (_c_size, [_c_int] * 5 + [_c_double, _c_int]),
        "moe_route": (_c_int, [_vp, _vp, _vp] + [_c_int] * 5 + [_vp] * 4 + [_vp, _c_size, _vp]),
        "moe_routing_stats": (_c_int, [_vp, _vp] + [_c_int] * 3 + [_vp] + [_vp, _c_size, _vp]),
        "moe_dispatch": (_c_int, [_vp] * 3 + [_c_int] * 3 + [_c_double, _c_int] + [_vp] * 7
                         + [_vp, _c_size, _vp]),
        "moe_expert_ffn": (_c_int, [_vp] * 8 + [_c_int] * 5 + [_c_double, _c_int, _c_int]
                           + [_vp, _vp, _c_size, _vp]),
        "moe_combine": (_c_int, [_vp] * 4 + [_c_int] * 5 + [_vp, _vp]),
        "moe_forward": (_c_int, [_vp] * 7 + [_c_int] * 5 + [_c_double, _c_int, _c_int]
                        + [_vp] * 8 + [_vp, _c_size, _vp]),
        "moe_forward_noalloc": (_c_int, [_vp] * 7 + [_c_int] * 5 + [_c_double, _c_int, _c_int]
                                + [_vp] * 8 + [_vp]),
        "moe_shared_workspace_bytes": (_c_size, [_c_int] * 4),
        "moe_shared_expert": (_c_int, [_vp] * 5 + [_c_int] * 5 + [_vp] + [_vp, _c_size, _vp]),
        "moe_set_profile_events": (_c_int, [ctypes.POINTER(_vp), _c_int]),
        "moe_pack_weights": (_c_int, [_vp] + [_c_int] * 4 + [_vp, _vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()

EXPORTED = ("moe_version", "moe_strerror", "moe_last_hip_error", "moe_capacity",
            "moe_workspace_bytes", "moe_route", "moe_routing_stats", "moe_dispatch",
            "moe_expert_ffn", "moe_combine", "moe_forward", "moe_forward_noalloc",
            "moe_set_profile_events",
            "moe_shared_workspace_bytes", "moe_shared_expert", "moe_pack_weights")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return MOE_F32
    if dt == torch.bfloat16:
        return MOE_BF16
    raise ValueError(f"unsupported activation dtype {dt}; use float32 or bfloat16")


def _check(t: Optional[torch.Tensor], name: str, dev, dtype=None, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _raise(st: int, where: str):
    if st != MOE_OK:
        raise MoeError(st, where)


def moe_version() -> int:
    return _lib.moe_version()


def moe_capacity(T: int, N: int, k: int, capacity_factor: float) -> int:
    c = _lib.moe_capacity(T, N, k, float(capacity_factor))
    _raise(min(c, 0), "moe_capacity")
    return c


def moe_workspace_bytes(T: int, d: int, d_ff: int, N: int, k: int, capacity_factor: float,
                        dtype: torch.dtype) -> int:
    n = _lib.moe_workspace_bytes(T, d, d_ff, N, k, float(capacity_factor), _dtype_code(dtype))
    if n == 0:
        raise ValueError("moe_workspace_bytes: invalid arguments")
    return n


def moe_shared_workspace_bytes(T: int, d: int, d_fs: int, dtype: torch.dtype) -> int:
    n = _lib.moe_shared_workspace_bytes(T, d, d_fs, _dtype_code(dtype))
    if n == 0:
        raise ValueError("moe_shared_workspace_bytes: invalid arguments")
    return n


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("workspace allocation is not 256-byte aligned")
    return ws


def moe_route(x: torch.Tensor, W_g: torch.Tensor, logit_bias: Optional[torch.Tensor], k: int,
              workspace: Optional[torch.Tensor] = None):
    """Steps 1-3. Returns (logits fp32 [T,N], topk_idx int32 [T,k], topk_w fp32 [T,k], topk_key fp64 [T,k])."""
    dev = x.device
    T, d = x.shape
    N = W_g.shape[1]
    _check(x, "x", dev)
    _check(W_g, "W_g", dev, x.dtype, (d, N))
    _check(logit_bias, "logit_bias", dev, torch.float32, (N,))
    logits = torch.empty((T, N), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    key = torch.empty((T, k), dtype=torch.float64, device=dev)
    if workspace is None:
        workspace = alloc_workspace(moe_workspace_bytes(T, d, 8, N, k, 0.0, x.dtype), dev)
    st = _lib.moe_route(_ptr(x), _ptr(W_g), _ptr(logit_bias), T, d, N, k, _dtype_code(x.dtype),
                        _ptr(logits), _ptr(idx), _ptr(w), _ptr(key), _ptr(workspace),
                        workspace.numel(), _stream(dev))
    _raise(st, "moe_route")
    return logits, idx, w, key


def moe_pack_weights(W: torch.Tensor) -> torch.Tensor:
    """Expert weights W [N, rows, K] (bf16) in the packed layout that the FFN
    entry points read with MOE_FLAG_PACKED_WEIGHTS: a new tensor of the same
    shape and dtype whose bytes are reordered (see include/moe.h)."""
    dev = W.device
    if W.dim() != 3:
        raise ValueError(f"W must be [N, rows, K], got shape {tuple(W.shape)}")
    _check(W, "W", dev, torch.bfloat16)
    N, rows, K = W.shape
    out = torch.empty_like(W)
    st = _lib.moe_pack_weights(_ptr(W), N, rows, K, MOE_BF16, _ptr(out), _stream(dev))
    _raise(st, "moe_pack_weights")
    return out


def moe_routing_stats(logits: torch.Tensor, topk_idx: torch.Tensor,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Routing statistics from moe_route's outputs: fp32 [2N + 2] device tensor
    holding f (share of the top-k picks per expert), P (mean router probability
    per expert), N * sum f P, and the mean squared log-sum-exp."""
    dev = logits.device
    T, N = logits.shape
    k = topk_idx.shape[1]
    _check(logits, "logits", dev, torch.float32)
    _check(topk_idx, "topk_idx", dev, torch.int32, (T, k))
    stats = torch.empty(2 * N + 2, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(moe_workspace_bytes(T, 8, 8, N, k, 0.0, torch.float32), dev)
    st = _lib.moe_routing_stats(_ptr(logits), _ptr(topk_idx), T, N, k, _ptr(stats),
                                _ptr(workspace), workspace.numel(), _stream(dev))
    _raise(st, "moe_routing_stats")
    return stats


def moe_dispatch(topk_idx: torch.Tensor, topk_w: torch.Tensor, topk_key: Optional[torch.Tensor],
                 N: int, capacity_factor: float, workspace: Optional[torch.Tensor] = None,
                 flags: int = 0) -> dict:
    """Steps 4-5. Returns dict of device tensors req_counts, counts, offsets, perm, inv, slot_gate, n_dropped.
    flags: MOE_FLAG_FIRST_COME (topk_key may then be None), MOE_FLAG_RENORM_SURVIVORS."""
    dev = topk_idx.device
    T, k = topk_idx.shape
    _check(topk_idx, "topk_idx", dev, torch.int32)
    _check(topk_w, "topk_w", dev, torch.float32, (T, k))
    if topk_key is not None:
        _check(topk_key, "topk_key", dev, torch.float64, (T, k))
    out = {
        "req_counts": torch.empty(N, dtype=torch.int32, device=dev),
        "counts": torch.empty(N, dtype=torch.int32, device=dev),
        "offsets": torch.empty(N + 1, dtype=torch.int32, device=dev),
        "perm": torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
        "inv": torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
        "slot_gate": torch.empty(max(T * k, 1), dtype=torch.float32, device=dev),
        "n_dropped": torch.empty(1, dtype=torch.int32, device=dev),
    }
    if workspace is None:
        workspace = alloc_workspace(moe_workspace_bytes(T, 8, 8, N, k, capacity_factor,
                                                        torch.float32), dev)
    st = _lib.moe_dispatch(_ptr(topk_idx), _ptr(topk_w), _ptr(topk_key), T, N, k,
                           float(capacity_factor), int(flags), _ptr(out["req_counts"]),
                           _ptr(out["counts"]),
                           _ptr(out["offsets"]), _ptr(out["perm"]), _ptr(out["inv"]),
                           _ptr(out["slot_gate"]), _ptr(out["n_dropped"]), _ptr(workspace),
                           workspace.numel(), _stream(dev))
    _raise(st, "moe_dispatch")
    return out


def moe_expert_ffn(x, perm, offsets, slot_gate, W1, b1, W2, b2, k: int, capacity_factor: float,
                   workspace: Optional[torch.Tensor] = None, flags: int = 0,
                   slot_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Step 6 with the gate folded in. Returns fp32 slot_out [T*k, d] (rows past S
    unspecified; a given slot_out keeps the rows the call does not write)."""
    dev = x.device
    T, d = x.shape
    N, d_ff, _ = W1.shape
    _check(x, "x", dev)
    for name, t in (("perm", perm), ("offsets", offsets)):
        _check(t, name, dev, torch.int32)
    _check(slot_gate, "slot_gate", dev, torch.float32)
    _check(W1, "W1", dev, x.dtype, (N, d_ff, d))
    _check(W2, "W2", dev, x.dtype, (N, d, d_ff))
    _check(b1, "b1", dev, x.dtype, (N, d_ff))
    _check(b2, "b2", dev, x.dtype, (N, d))
    if slot_out is None:
        slot_out = torch.empty((max(T * k, 1), d), dtype=torch.float32, device=dev)
    _check(slot_out, "slot_out", dev, torch.float32, (max(T * k, 1), d))
    if workspace is None:
        workspace = alloc_workspace(moe_workspace_bytes(T, d, d_ff, N, k, capacity_factor, x.dtype), dev)
    st = _lib.moe_expert_ffn(_ptr(x), _ptr(perm), _ptr(offsets), _ptr(slot_gate), _ptr(W1), _ptr(b1),
                             _ptr(W2), _ptr(b2), T, d, d_ff, N, k, float(capacity_factor),
                             _dtype_code(x.dtype), int(flags), _ptr(slot_out), _ptr(workspace),
                             workspace.numel(), _stream(dev))
    _raise(st, "moe_expert_ffn")
    return slot_out


def moe_shared_expert(x, W1s, b1s, W2s, b2s, workspace: Optional[torch.Tensor] = None,
                      flags: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Shared expert on every token: fp32 [T, d] = W2s GELU(W1s x + b1s) + b2s,
    for the shared_out argument of moe_combine / moe_forward.
    flags: MOE_FLAG_HIDDEN_SPLIT."""
    dev = x.device
    T, d = x.shape
    d_fs = W1s.shape[0]
    _check(x, "x", dev)
    _check(W1s, "W1s", dev, x.dtype, (d_fs, d))
    _check(W2s, "W2s", dev, x.dtype, (d, d_fs))
    _check(b1s, "b1s", dev, x.dtype, (d_fs,))
    _check(b2s, "b2s", dev, x.dtype, (d,))
    if out is None:
        out = torch.empty((T, d), dtype=torch.float32, device=dev)
    _check(out, "out", dev, torch.float32, (T, d))
    if workspace is None:
        workspace = alloc_workspace(moe_shared_workspace_bytes(T, d, d_fs, x.dtype), dev)
    st = _lib.moe_shared_expert(_ptr(x), _ptr(W1s), _ptr(b1s), _ptr(W2s), _ptr(b2s), T, d, d_fs,
                                _dtype_code(x.dtype), int(flags), _ptr(out), _ptr(workspace),
                                workspace.numel(), _stream(dev))
    _raise(st, "moe_shared_expert")
    return out


def moe_combine(slot_out: torch.Tensor, inv: torch.Tensor, T: int, k: int,
                dtype: torch.dtype = torch.bfloat16, x: Optional[torch.Tensor] = None,
                flags: int = 0, shared_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Step 7. slot_out is fp32 [T*k, d]; returns y [T, d] in ``dtype`` (the
    activation dtype; float32 with MOE_FLAG_Y_F32). With
    MOE_FLAG_IDENTITY_FALLBACK, x [T, d] in ``dtype`` fills fully dropped tokens;
    shared_out (fp32 [T, d], moe_shared_expert's output) is added to every token."""
    dev = slot_out.device
    d = slot_out.shape[1]
    _check(slot_out, "slot_out", dev, torch.float32)
    _check(inv, "inv", dev, torch.int32)
    _check(x, "x", dev, dtype, (T, d))
    _check(shared_out, "shared_out", dev, torch.float32, (T, d))
    y = torch.empty((T, d), dtype=torch.float32 if (flags & MOE_FLAG_Y_F32) else dtype, device=dev)
    st = _lib.moe_combine(_ptr(slot_out), _ptr(inv), _ptr(x), _ptr(shared_out), T, d, k,
                          _dtype_code(dtype), int(flags), _ptr(y), _stream(dev))
    _raise(st, "moe_combine")
    return y


def moe_forward(x, W_g, logit_bias, W1, b1, W2, b2, k: int, capacity_factor: float,
                workspace: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                want_routing: bool = False, flags: int = 0,
                shared_out: Optional[torch.Tensor] = None):
    """Steps 1-7 in one enqueue. Returns y, or (y, extras) when want_routing is set;
    extras holds logits, topk_idx, inv, req_counts, counts, n_dropped (device tensors).
    flags: any MOE_FLAG_* (MOE_FLAG_Y_F32 makes y float32). shared_out: fp32
    [T, d] from moe_shared_expert, added to every token before y's rounding."""
    dev = x.device
    T, d = x.shape
    N, d_ff, _ = W1.shape
    _check(x, "x", dev)
    _check(W_g, "W_g", dev, x.dtype, (d, N))
    _check(logit_bias, "logit_bias", dev, torch.float32, (N,))
    _check(W1, "W1", dev, x.dtype, (N, d_ff, d))
    _check(W2, "W2", dev, x.dtype, (N, d, d_ff))
    _check(b1, "b1", dev, x.dtype, (N, d_ff))
    _check(b2, "b2", dev, x.dtype, (N, d))
    _check(shared_out, "shared_out", dev, torch.float32, (T, d))
    y_dtype = torch.float32 if (flags & MOE_FLAG_Y_F32) else x.dtype
    if y is None:
        y = torch.empty((T, d), dtype=y_dtype, device=dev)
    _check(y, "y", dev, y_dtype, (T, d))
    if workspace is None:
        workspace = alloc_workspace(moe_workspace_bytes(T, d, d_ff, N, k, capacity_factor, x.dtype), dev)
    ex = {}
    ec = bool(flags & MOE_FLAG_EXPERT_CHOICE)
    kp = N if ec else k  # pairs per token (expert choice: every expert)
    if want_routing:
        ex = {
            "logits": torch.empty((T, N), dtype=torch.float32, device=dev),
            "topk_idx": None if ec else torch.empty((T, k), dtype=torch.int32, device=dev),
            "inv": torch.empty(max(T * kp, 1), dtype=torch.int32, device=dev),
            "req_counts": torch.empty(N, dtype=torch.int32, device=dev),
            "counts": torch.empty(N, dtype=torch.int32, device=dev),
            "n_dropped": torch.empty(1, dtype=torch.int32, device=dev),
        }
    st = _lib.moe_forward(_ptr(x), _ptr(W_g), _ptr(logit_bias), _ptr(W1), _ptr(b1), _ptr(W2),
                          _ptr(b2), T, d, d_ff, N, k, float(capacity_factor), _dtype_code(x.dtype),
                          int(flags), _ptr(shared_out), _ptr(y), _ptr(ex.get("logits")),
                          _ptr(ex.get("topk_idx")), _ptr(ex.get("inv")),
                          _ptr(ex.get("req_counts")), _ptr(ex.get("counts")), _ptr(ex.get("n_dropped")),
                          _ptr(workspace), workspace.numel(), _stream(dev))
    _raise(st, "moe_forward")
    return (y, ex) if want_routing else y


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(x, W_g, logit_bias, W1, b1, W2, b2, k: int, capacity_factor: float,
                        y: Optional[torch.Tensor] = None, want_routing: bool = False,
                        flags: int = 0, shared_out: Optional[torch.Tensor] = None):
    """moe_forward without a workspace: the library's static per-GPU scratch
    array (MOE_NOALLOC_SCRATCH_BYTES) holds the intermediates. Pass y (and
    shared_out) preallocated to keep the call free of allocation; the routing
    extras, when asked for, are allocated here as for moe_forward."""
    dev = x.device
    T, d = x.shape
    N, d_ff, _ = W1.shape
    _check(x, "x", dev)
    _check(W_g, "W_g", dev, x.dtype, (d, N))
    _check(logit_bias, "logit_bias", dev, torch.float32, (N,))
    _check(W1, "W1", dev, x.dtype, (N, d_ff, d))
    _check(W2, "W2", dev, x.dtype, (N, d, d_ff))
    _check(b1, "b1", dev, x.dtype, (N, d_ff))
    _check(b2, "b2", dev, x.dtype, (N, d))
    _check(shared_out, "shared_out", dev, torch.float32, (T, d))
    y_dtype = torch.float32 if (flags & MOE_FLAG_Y_F32) else x.dtype
    if y is None:
        y = torch.empty((T, d), dtype=y_dtype, device=dev)
    _check(y, "y", dev, y_dtype, (T, d))
    ex = {}
    ec = bool(flags & MOE_FLAG_EXPERT_CHOICE)
    kp = N if ec else k
    if want_routing:
        ex = {
            "logits": torch.empty((T, N), dtype=torch.float32, device=dev),
            "topk_idx": None if ec else torch.empty((T, k), dtype=torch.int32, device=dev),
            "inv": torch.empty(max(T * kp, 1), dtype=torch.int32, device=dev),
            "req_counts": torch.empty(N, dtype=torch.int32, device=dev),
            "counts": torch.empty(N, dtype=torch.int32, device=dev),
            "n_dropped": torch.empty(1, dtype=torch.int32, device=dev),
        }
    st = _lib.moe_forward_noalloc(_ptr(x), _ptr(W_g), _ptr(logit_bias), _ptr(W1), _ptr(b1),
                                  _ptr(W2), _ptr(b2), T, d, d_ff, N, k, float(capacity_factor),
                                  _dtype_code(x.dtype), int(flags), _ptr(shared_out), _ptr(y),
                                  _ptr(ex.get("logits")), _ptr(ex.get("topk_idx")),
                                  _ptr(ex.get("inv")), _ptr(ex.get("req_counts")),
                                  _ptr(ex.get("counts")), _ptr(ex.get("n_dropped")), _stream(dev))
    _raise(st, "moe_forward_noalloc")
    return (y, ex) if want_routing else y


def moe_set_profile_events(events) -> None:
    """Register raw hipEvent_t handles (ints or None, at most 7) for this thread; [] clears."""
    n = len(events)
    arr = (_vp * max(n, 1))(*[None if e is None else _vp(e) for e in events])
    _raise(_lib.moe_set_profile_events(arr, n), "moe_set_profile_events")
