"""ctypes binding of libmoe_hip.so (C ABI in include/moe.h).

Argument marshalling only: tensors are passed by ``data_ptr()`` and the
current torch stream is passed as the hipStream_t.  Every step of the layer
runs in the library's HIP kernels; nothing here computes.  A missing or
unloadable library raises MoEError -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_HIP_LIB names another build of the same library (the sanitized host
# build that the CPU tests load); default: the in-tree libmoe_hip.so
LIB_PATH = os.environ.get("MOE_HIP_LIB") or os.path.join(PKG, "libmoe_hip.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
GATING = {"topk_softmax": 0, "softmax_topk": 1, "switch": 2, "expert_choice": 3}
ACT = {"relu": 0, "gelu": 1, "swiglu": 2}
DTYPE = {"f32": 0, "bf16": 1}
STAGE_FORWARD, STAGE_PERMUTE, STAGE_FFN, STAGE_LOSSES = 0, 1, 2, 3

EXPORTS = ["moe_capacity", "moe_workspace_size", "moe_route", "moe_route_noisy", "moe_route_from_logits",
           "moe_router_losses", "moe_permute", "moe_permute_noalloc",
           "moe_expert_ffn", "moe_combine", "moe_forward", "moe_last_error", "moe_timing_enable",
           "moe_timing_reset", "moe_timing_read", "moe_kernel_name"]


class MoEError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"moe status {status}: {message}")
        self.status = status


class moe_config(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("d_model", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
                ("gating", ctypes.c_int32), ("act", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("capacity_group", ctypes.c_int32), ("capacity_factor", ctypes.c_float),
                ("min_capacity", ctypes.c_int32), ("num_shared", ctypes.c_int32)]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "b_router", "w1", "w3", "w2", "b1", "b2", "ws1", "ws3", "ws2")]


class moe_routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("logits", "topk_idx", "topk_w", "counts", "offsets", "row_token", "slot_row")]


_lib = None


def load():
    """Load the in-tree library (built by ``python -m sparse_mixture_experts_gating_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoEError(-1, f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_mixture_experts_gating_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(moe_config)
    sig = {
        "moe_capacity": [cfgp, ctypes.POINTER(I32)],
        "moe_workspace_size": [cfgp, I32, ctypes.POINTER(SZ)],
        "moe_route": [cfgp, P, ctypes.POINTER(moe_weights), ctypes.POINTER(moe_routing), P],
        "moe_route_from_logits": [cfgp, P, ctypes.POINTER(moe_routing), P],
        "moe_route_noisy": [cfgp, P, ctypes.POINTER(moe_weights), P, P, ctypes.POINTER(moe_routing), P],
        "moe_router_losses": [cfgp, P, P, P, P, SZ, P],
        "moe_permute": [cfgp, P, ctypes.POINTER(moe_routing), P, P, SZ, P],
        "moe_permute_noalloc": [cfgp, P, ctypes.POINTER(moe_routing), P, P],
        "moe_expert_ffn": [cfgp, P, P, ctypes.POINTER(moe_routing), ctypes.POINTER(moe_weights), P, P, P, SZ, P],
        "moe_combine": [cfgp, P, P, ctypes.POINTER(moe_routing), P, P],
        "moe_forward": [cfgp, P, ctypes.POINTER(moe_weights), P, ctypes.POINTER(moe_routing), P, SZ, P],
        "moe_timing_enable": [I32],
        "moe_timing_reset": [],
        "moe_timing_read": [I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_kernel_name.argtypes = [I32]
    lib.moe_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status):
    if status != MOE_OK:
        raise MoEError(status, load().moe_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---------------------------------------------------------------------------
# structures
# ---------------------------------------------------------------------------

def make_config(T, d, E, k, F, gating, act, dtype, F_shared=0, capacity_factor=0.0, capacity_group=0,
                min_capacity=0, num_shared=1):
    return moe_config(T, d, E, k, F, F_shared, GATING[gating], ACT[act], DTYPE[dtype], capacity_group,
                      float(capacity_factor), int(min_capacity), int(num_shared) if F_shared else 0)


def config_from_spec(spec) -> moe_config:
    """moe_config of a layer description with attributes T, d, E, k, F, gating, act, dtype,
    F_shared, capacity_factor, capacity_group (and optionally min_capacity, num_shared)."""
    return make_config(spec.T, spec.d, spec.E, spec.k, spec.F, spec.gating, spec.act, spec.dtype,
                       spec.F_shared, spec.capacity_factor, spec.capacity_group, getattr(spec, "min_capacity", 0),
                       getattr(spec, "num_shared", 1))


def make_weights(t: dict) -> moe_weights:
    """moe_weights of a dict of device tensors (keys wg, bg, w1, w3, w2, b1, b2, ws1, ws3, ws2).
    The returned structure keeps no reference to the tensors; the caller must."""
    g = lambda key: None if t.get(key) is None else t[key].data_ptr()
    return moe_weights(g("wg"), g("bg"), g("w1"), g("w3"), g("w2"), g("b1"), g("b2"), g("ws1"), g("ws3"), g("ws2"))


def make_routing(r: dict) -> moe_routing:
    g = lambda key: None if r.get(key) is None else r[key].data_ptr()
    return moe_routing(g("logits"), g("topk_idx"), g("topk_w"), g("counts"), g("offsets"), g("row_token"),
                       g("slot_row"))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def moe_capacity(cfg: moe_config) -> int:
    out = ctypes.c_int32()
    _check(load().moe_capacity(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def moe_workspace_size(cfg: moe_config, stage: int = STAGE_FORWARD) -> int:
    out = ctypes.c_size_t()
    _check(load().moe_workspace_size(ctypes.byref(cfg), stage, ctypes.byref(out)))
    return out.value


def moe_route(cfg, x, weights: moe_weights, routing: moe_routing, stream=None):
    _check(load().moe_route(ctypes.byref(cfg), _p(x), ctypes.byref(weights), ctypes.byref(routing),
                            _stream(stream)))


def moe_route_from_logits(cfg, logits, routing: moe_routing, stream=None):
    _check(load().moe_route_from_logits(ctypes.byref(cfg), _p(logits), ctypes.byref(routing), _stream(stream)))


def moe_route_noisy(cfg, x, weights: moe_weights, w_noise, noise, routing: moe_routing, stream=None):
    _check(load().moe_route_noisy(ctypes.byref(cfg), _p(x), ctypes.byref(weights), _p(w_noise), _p(noise),
                                  ctypes.byref(routing), _stream(stream)))


def moe_router_losses(cfg, logits, topk_idx, out, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().moe_router_losses(ctypes.byref(cfg), _p(logits), _p(topk_idx), _p(out), _p(ws), nbytes,
                                    _stream(stream)))


def moe_permute(cfg, x, routing: moe_routing, x_perm, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().moe_permute(ctypes.byref(cfg), _p(x), ctypes.byref(routing), _p(x_perm), _p(ws), nbytes,
                              _stream(stream)))


def moe_permute_noalloc(cfg, x, routing: moe_routing, x_perm, stream=None):
    _check(load().moe_permute_noalloc(ctypes.byref(cfg), _p(x), ctypes.byref(routing), _p(x_perm),
                                      _stream(stream)))


def moe_expert_ffn(cfg, x_perm, x, routing: moe_routing, weights: moe_weights, y_perm, y_shared, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().moe_expert_ffn(ctypes.byref(cfg), _p(x_perm), _p(x), ctypes.byref(routing),
                                 ctypes.byref(weights), _p(y_perm), _p(y_shared), _p(ws), nbytes,
                                 _stream(stream)))


def moe_combine(cfg, y_perm, y_shared, routing: moe_routing, y, stream=None):
    _check(load().moe_combine(ctypes.byref(cfg), _p(y_perm), _p(y_shared), ctypes.byref(routing), _p(y),
                              _stream(stream)))


def moe_forward(cfg, x, weights: moe_weights, y, routing, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    rp = None if routing is None else ctypes.byref(routing)
    _check(load().moe_forward(ctypes.byref(cfg), _p(x), ctypes.byref(weights), _p(y), rp, _p(ws), nbytes,
                              _stream(stream)))


def moe_last_error() -> str:
    return load().moe_last_error().decode()


def moe_timing_enable(on: bool):
    _check(load().moe_timing_enable(1 if on else 0))


def moe_timing_reset():
    _check(load().moe_timing_reset())


def moe_timing_read(kind: int):
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(load().moe_timing_read(kind, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def moe_kernel_names() -> list:
    out, i = [], 0
    while True:
        n = load().moe_kernel_name(i)
        if n is None:
            return out
        out.append(n.decode())
        i += 1


# ---------------------------------------------------------------------------
# buffer plumbing (allocation with torch; no computation)
# ---------------------------------------------------------------------------

def alloc_routing(cfg: moe_config, device) -> dict:
    """Routing buffers of moe.h's moe_routing for a configuration, on ``device``."""
    import torch
    T, E = cfg.num_tokens, cfg.num_experts
    if cfg.gating == GATING["expert_choice"]:
        C = moe_capacity(cfg)
        slots, S = E * C, E
    else:
        slots, S = T * cfg.top_k, cfg.top_k
    i32 = dict(dtype=torch.int32, device=device)
    return dict(logits=torch.empty((T, E), dtype=torch.float32, device=device),
                topk_idx=torch.empty(slots, **i32), topk_w=torch.empty(slots, dtype=torch.float32, device=device),
                counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                row_token=torch.empty(max(slots, 1), **i32), slot_row=torch.empty(max(T * S, 1), **i32))


def alloc_workspace(cfg: moe_config, stage: int, device):
    import torch
    n = moe_workspace_size(cfg, stage)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)
