"""Python binding of libmoe_hip.so, the MI355X (gfx950) MoE-layer hot path.

Thin ctypes marshalling over the C ABI in include/moe.h: every function below
has the C entry point's name and argument order, turns torch tensors (device
memory), ints and None into pointers and sizes, and raises MoeError on a
non-zero status. All computation happens in the HIP library; torch provides
device memory and streams only. There is no fallback: if the library is not
built, loading fails with an error that says so.

`forward()` is a convenience on top: it allocates outputs and the workspace
with torch and calls moe_layer_forward once.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_hip.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
TOTALS = ("dropped", "fully_dropped_tokens", "padded_rows", "offrank_bytes")

EXPORTS = ("moe_capacity", "moe_workspace_size", "moe_layer_forward", "moe_backward_workspace_size",
           "moe_layer_backward", "moe_layer_backward_saved", "moe_replica_plan", "moe_replicated_workspace_size", "moe_layer_forward_replicated", "moe_router_workspace_size", "moe_router", "moe_route",
           "moe_permute_workspace_size", "moe_permute", "moe_permute_static", "moe_grouped_gemm_workspace_size",
           "moe_grouped_gemm", "moe_combine", "moe_set_stage_events", "moe_stage_ran", "moe_status_string", "moe_last_error")
STAGES = ("router", "route", "slots", "scatter", "gate_up", "down", "combine")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({detail})")


class moe_stats_t(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("slot", ctypes.c_void_p),
                ("src", ctypes.c_void_p), ("routed_count", ctypes.c_void_p),
                ("kept_count", ctypes.c_void_p), ("send_count", ctypes.c_void_p),
                ("totals", ctypes.c_void_p), ("buckets", ctypes.c_void_p), ("instance", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("u", ctypes.c_void_p), ("h", ctypes.c_void_p)]


_lib = None
_P, _I32, _I64, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "moe_capacity": [_I64, _I32, _I32, _F32, _P],
    "moe_workspace_size": [_I64, _I64, _I64, _I32, _I32, _F32, _I32, ctypes.c_int, _P],
    "moe_layer_forward": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _F32, _I32, _I32, ctypes.c_int,
                          _P, ctypes.POINTER(moe_stats_t), _P, _SZ, _P],
    "moe_backward_workspace_size": [_I64, _I64, _I64, _I32, _I32, _F32, _I32, ctypes.c_int, _P],
    "moe_layer_backward": [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _F32, _I32, _I32, ctypes.c_int,
                           _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "moe_layer_backward_saved": [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _F32, _I32, _I32,
                                 ctypes.c_int, ctypes.POINTER(moe_stats_t), _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "moe_replica_plan": [_P, _I32, _I32, _P],
    "moe_replicated_workspace_size": [_I64, _I64, _I64, _I32, _I32, _F32, _I32, _I32, ctypes.c_int, _P],
    "moe_layer_forward_replicated": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _F32, _I32, _I32, _P,
                                     _I32, ctypes.c_int, _P, ctypes.POINTER(moe_stats_t), _P, _SZ, _P],
    "moe_router_workspace_size": [_I64, _I64, _I32, ctypes.c_int, _P],
    "moe_router": [_P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, ctypes.c_int, _P, _P, _P, _P, _SZ, _P],
    "moe_route": [_P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P],
    "moe_permute_workspace_size": [_I64, _I32, _P],
    "moe_permute": [_P, _P, _I64, _I64, _I32, _I32, _I64, _I32, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P,
                    _P, _SZ, _P],
    "moe_permute_static": [_P, _P, _I64, _I64, _I32, _I32, _I64, _I32, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P,
                           _P],
    "moe_grouped_gemm_workspace_size": [_I32, _I64, _P],
    "moe_grouped_gemm": [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, ctypes.c_int, _P, _P, _P, _SZ, _P],
    "moe_combine": [_P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I64, ctypes.c_int, _P, _P],
    "moe_set_stage_events": [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int],
    "moe_stage_ran": [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)],
}


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m routing_dispatch_expert_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_status_string(status: int) -> str:
    return status_string(status)


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where, moe_last_error())


def _ptr(a):
    """Device pointer of a torch tensor, an int address, or None (NULL)."""
    if a is None:
        return None
    if isinstance(a, int):
        return a or None
    return a.data_ptr() or None


def _dtype(dt) -> int:
    if isinstance(dt, int):
        return dt
    s = str(dt)
    if s in ("bf16", "torch.bfloat16"):
        return MOE_DTYPE_BF16
    if s in ("f32", "fp32", "torch.float32"):
        return MOE_DTYPE_F32
    raise ValueError(f"unsupported dtype {dt!r}")


def _stream(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


# ----------------------------------------------------------------- C entry points

def moe_capacity(T: int, E: int, k: int, cf: float) -> int:
    C = ctypes.c_int64(0)
    _check(lib().moe_capacity(T, E, k, cf, ctypes.byref(C)), "moe_capacity")
    return C.value


def moe_workspace_size(T, d, d_ff, E, k, cf, P, dtype) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(T, d, d_ff, E, k, cf, P, _dtype(dtype), ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def _stats(stats) -> "ctypes.POINTER(moe_stats_t) | None":
    if stats is None:
        return None
    s = moe_stats_t()
    for name, _ in moe_stats_t._fields_:
        setattr(s, name, _ptr(stats.get(name)))
    return ctypes.pointer(s)


def moe_layer_forward(x, W_router, router_bias, W_gate, W_up, W_down, T, d, d_ff, E, k, cf, P, max_ranks,
                      dtype, out, stats, workspace, workspace_bytes, stream=None):
    """stats: None or a dict of moe_stats_t field name -> tensor (or None)."""
    _check(lib().moe_layer_forward(_ptr(x), _ptr(W_router), _ptr(router_bias), _ptr(W_gate), _ptr(W_up),
                                   _ptr(W_down), T, d, d_ff, E, k, cf, P, max_ranks, _dtype(dtype), _ptr(out),
                                   _stats(stats), _ptr(workspace), workspace_bytes, _stream(stream)),
           "moe_layer_forward")


def moe_backward_workspace_size(T, d, d_ff, E, k, cf, P, dtype) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_backward_workspace_size(T, d, d_ff, E, k, cf, P, _dtype(dtype), ctypes.byref(n)),
           "moe_backward_workspace_size")
    return n.value


def moe_layer_backward(x, W_router, router_bias, W_gate, W_up, W_down, dout, T, d, d_ff, E, k, cf, P, max_ranks,
                       dtype, dx, dW_router, d_bias, dW_gate, dW_up, dW_down, workspace, workspace_bytes,
                       stream=None):
    _check(lib().moe_layer_backward(_ptr(x), _ptr(W_router), _ptr(router_bias), _ptr(W_gate), _ptr(W_up),
                                    _ptr(W_down), _ptr(dout), T, d, d_ff, E, k, cf, P, max_ranks, _dtype(dtype),
                                    _ptr(dx), _ptr(dW_router), _ptr(d_bias), _ptr(dW_gate), _ptr(dW_up),
                                    _ptr(dW_down), _ptr(workspace), workspace_bytes, _stream(stream)),
           "moe_layer_backward")


def moe_layer_backward_saved(x, W_router, router_bias, W_gate, W_up, W_down, dout, T, d, d_ff, E, k, cf, P,
                             max_ranks, dtype, saved, dx, dW_router, d_bias, dW_gate, dW_up, dW_down, workspace,
                             workspace_bytes, stream=None):
    """saved: the stats dict of a moe_layer_forward call that kept g, u and h."""
    _check(lib().moe_layer_backward_saved(_ptr(x), _ptr(W_router), _ptr(router_bias), _ptr(W_gate), _ptr(W_up),
                                          _ptr(W_down), _ptr(dout), T, d, d_ff, E, k, cf, P, max_ranks,
                                          _dtype(dtype), _stats(saved), _ptr(dx), _ptr(dW_router), _ptr(d_bias),
                                          _ptr(dW_gate), _ptr(dW_up), _ptr(dW_down), _ptr(workspace),
                                          workspace_bytes, _stream(stream)),
           "moe_layer_backward_saved")


def moe_replica_plan(routed_count, extra):
    """Host-side replica counts (numpy int32 array of length E) from routed counts."""
    import numpy as np
    routed = np.ascontiguousarray(routed_count, dtype=np.int32)
    out = np.empty_like(routed)
    _check(lib().moe_replica_plan(routed.ctypes.data, routed.size, int(extra), out.ctypes.data), "moe_replica_plan")
    return out


def moe_replicated_workspace_size(T, d, d_ff, E, k, cf, P, R, dtype) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_replicated_workspace_size(T, d, d_ff, E, k, cf, P, R, _dtype(dtype), ctypes.byref(n)),
           "moe_replicated_workspace_size")
    return n.value


def moe_layer_forward_replicated(x, W_router, router_bias, W_gate, W_up, W_down, T, d, d_ff, E, k, cf, P, max_ranks,
                                 replicas, R, dtype, out, stats, workspace, workspace_bytes, stream=None):
    _check(lib().moe_layer_forward_replicated(_ptr(x), _ptr(W_router), _ptr(router_bias), _ptr(W_gate), _ptr(W_up),
                                              _ptr(W_down), T, d, d_ff, E, k, cf, P, max_ranks, _ptr(replicas), R,
                                              _dtype(dtype), _ptr(out), _stats(stats), _ptr(workspace),
                                              workspace_bytes, _stream(stream)),
           "moe_layer_forward_replicated")


def moe_router_workspace_size(T, d, E, dtype) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_router_workspace_size(T, d, E, _dtype(dtype), ctypes.byref(n)), "moe_router_workspace_size")
    return n.value


def moe_router(x, W_router, router_bias, T, d, E, k, P, max_ranks, dtype, topk_idx, topk_w, logits_out,
               workspace, workspace_bytes, stream=None):
    _check(lib().moe_router(_ptr(x), _ptr(W_router), _ptr(router_bias), T, d, E, k, P, max_ranks, _dtype(dtype),
                            _ptr(topk_idx), _ptr(topk_w), _ptr(logits_out), _ptr(workspace),
                            workspace_bytes, _stream(stream)), "moe_router")


def moe_route(logits, T, E, k, P, max_ranks, topk_idx, topk_w, stream=None):
    _check(lib().moe_route(_ptr(logits), T, E, k, P, max_ranks, _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
           "moe_route")


def moe_permute_workspace_size(T, E) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_permute_workspace_size(T, E, ctypes.byref(n)), "moe_permute_workspace_size")
    return n.value


def moe_permute(x, topk_idx, T, d, E, k, C, P, dtype, buckets, slot, src, routed_count, kept_count,
                send_count, totals, workspace, workspace_bytes, stream=None):
    _check(lib().moe_permute(_ptr(x), _ptr(topk_idx), T, d, E, k, C, P, _dtype(dtype), _ptr(buckets),
                             _ptr(slot), _ptr(src), _ptr(routed_count), _ptr(kept_count),
                             _ptr(send_count), _ptr(totals), _ptr(workspace), workspace_bytes,
                             _stream(stream)), "moe_permute")


def moe_permute_static(x, topk_idx, T, d, E, k, C, P, dtype, buckets, slot, src, routed_count, kept_count,
                       send_count, totals, stream=None):
    _check(lib().moe_permute_static(_ptr(x), _ptr(topk_idx), T, d, E, k, C, P, _dtype(dtype), _ptr(buckets),
                                    _ptr(slot), _ptr(src), _ptr(routed_count), _ptr(kept_count),
                                    _ptr(send_count), _ptr(totals), _stream(stream)), "moe_permute_static")


def moe_grouped_gemm_workspace_size(E, C) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_grouped_gemm_workspace_size(E, C, ctypes.byref(n)), "moe_grouped_gemm_workspace_size")
    return n.value


def moe_grouped_gemm(buckets, kept_count, W_gate, W_up, W_down, E, C, d, d_ff, dtype, h, y, workspace,
                     workspace_bytes, stream=None):
    _check(lib().moe_grouped_gemm(_ptr(buckets), _ptr(kept_count), _ptr(W_gate), _ptr(W_up), _ptr(W_down),
                                  E, C, d, d_ff, _dtype(dtype), _ptr(h), _ptr(y), _ptr(workspace),
                                  workspace_bytes, _stream(stream)), "moe_grouped_gemm")


def moe_combine(x, y, topk_idx, topk_w, slot, T, d, E, k, C, dtype, out, stream=None):
    _check(lib().moe_combine(_ptr(x), _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(slot), T, d, E, k, C,
                             _dtype(dtype), _ptr(out), _stream(stream)), "moe_combine")


def moe_set_stage_events(events):
    """events: None (off) or 2 * len(STAGES) raw hipEvent_t handles (ints)."""
    if events is None:
        _check(lib().moe_set_stage_events(None, 0), "moe_set_stage_events")
        return
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(lib().moe_set_stage_events(arr, len(events)), "moe_set_stage_events")


def moe_stage_ran(stage: int) -> bool:
    """Whether the last layer call with stage events recorded this stage's events."""
    ran = ctypes.c_int32(0)
    _check(lib().moe_stage_ran(stage, ctypes.byref(ran)), "moe_stage_ran")
    return bool(ran.value)


# ----------------------------------------------------------------- convenience

def _require(t, name, torch_dtype, shape):
    if t.device.type != "cuda" or not t.is_contiguous() or t.dtype != torch_dtype or tuple(t.shape) != shape:
        raise ValueError(f"{name}: need a contiguous {torch_dtype} cuda tensor of shape {shape}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def forward(x, W_router, W_gate, W_up, W_down, k, cf, P=1, router_bias=None, stream=None,
            want_buckets=False, want_src=False, workspace=None, max_ranks=0, keep_activations=False):
    """Run the layer once on torch device tensors; returns a dict of outputs.

    x [T, d]; W_router [E, d]; W_gate, W_up [E, d_ff, d]; W_down [E, d, d_ff]
    (bf16 or fp32, all the same dtype); router_bias [E] fp32 or None;
    max_ranks > 0 limits each token's experts to that many of the P ranks.
    keep_activations: also return the buckets and g, u, h [E, C, d_ff], the
    state backward(..., saved=result) takes instead of recomputing it.
    """
    import torch
    T, d = x.shape
    E = W_router.shape[0]
    d_ff = W_gate.shape[1]
    dt = x.dtype
    for t, n, s in ((x, "x", (T, d)), (W_router, "W_router", (E, d)), (W_gate, "W_gate", (E, d_ff, d)),
                    (W_up, "W_up", (E, d_ff, d)), (W_down, "W_down", (E, d, d_ff))):
        _require(t, n, dt, s)
    if router_bias is not None:
        _require(router_bias, "router_bias", torch.float32, (E,))
    C = moe_capacity(T, E, k, cf)
    dev = x.device
    i32 = dict(dtype=torch.int32, device=dev)
    res = {
        "C": C,
        "out": torch.empty_like(x),
        "topk_idx": torch.empty((T, k), **i32),
        "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev),
        "slot": torch.empty((T, k), **i32),
        "routed_count": torch.empty(E, **i32),
        "kept_count": torch.empty(E, **i32),
        "send_count": torch.empty(P, **i32),
        "totals": torch.empty(4, dtype=torch.int64, device=dev),
    }
    if want_buckets or keep_activations:
        res["buckets"] = torch.empty((E, C, d), dtype=dt, device=dev)
    if want_src:
        res["src"] = torch.empty((E, C), **i32)
    if keep_activations:
        for name in ("g", "u", "h"):
            res[name] = torch.empty((E, C, d_ff), dtype=dt, device=dev)
    nbytes = moe_workspace_size(T, d, d_ff, E, k, cf, P, dt)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    moe_layer_forward(x, W_router, router_bias, W_gate, W_up, W_down, T, d, d_ff, E, k, cf, P, max_ranks, dt,
                      res["out"], res, workspace, nbytes, stream)
    res["workspace"] = workspace
    return res


def backward(x, W_router, W_gate, W_up, W_down, dout, k, cf, P=1, router_bias=None, stream=None, max_ranks=0,
             workspace=None, want_d_bias=False, saved=None):
    """Gradients of the layer for dout on torch device tensors; returns a dict
    dx, dW_router, d_bias (fp32, when router_bias is given or want_d_bias),
    dW_gate, dW_up, dW_down, workspace. saved: the result of
    forward(..., keep_activations=True) on the same inputs, whose routing,
    buckets and activations are then used instead of being recomputed."""
    import torch
    T, d = x.shape
    E = W_router.shape[0]
    d_ff = W_gate.shape[1]
    dt = x.dtype
    for t, n, s in ((x, "x", (T, d)), (dout, "dout", (T, d)), (W_router, "W_router", (E, d)),
                    (W_gate, "W_gate", (E, d_ff, d)), (W_up, "W_up", (E, d_ff, d)), (W_down, "W_down", (E, d, d_ff))):
        _require(t, n, dt, s)
    if router_bias is not None:
        _require(router_bias, "router_bias", torch.float32, (E,))
    res = {"dx": torch.empty_like(x), "dW_router": torch.empty_like(W_router), "dW_gate": torch.empty_like(W_gate),
           "dW_up": torch.empty_like(W_up), "dW_down": torch.empty_like(W_down),
           "d_bias": (torch.empty(E, dtype=torch.float32, device=x.device)
                      if router_bias is not None or want_d_bias else None)}
    nbytes = moe_backward_workspace_size(T, d, d_ff, E, k, cf, P, dt)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    if saved is None:
        moe_layer_backward(x, W_router, router_bias, W_gate, W_up, W_down, dout, T, d, d_ff, E, k, cf, P, max_ranks,
                           dt, res["dx"], res["dW_router"], res["d_bias"], res["dW_gate"], res["dW_up"],
                           res["dW_down"], workspace, nbytes, stream)
    else:
        moe_layer_backward_saved(x, W_router, router_bias, W_gate, W_up, W_down, dout, T, d, d_ff, E, k, cf, P,
                                 max_ranks, dt, saved, res["dx"], res["dW_router"], res["d_bias"], res["dW_gate"],
                                 res["dW_up"], res["dW_down"], workspace, nbytes, stream)
    res["workspace"] = workspace
    return res


def forward_replicated(x, W_router, W_gate, W_up, W_down, k, cf, replicas, P=1, router_bias=None, stream=None,
                       want_buckets=False, want_src=False, workspace=None, max_ranks=0):
    """The layer with replicated experts; replicas is an int32 cuda tensor [E]
    (each >= 1). Returns a dict like forward(), with per-instance kept_count,
    src and buckets, and the instance of each copy."""
    import torch
    T, d = x.shape
    E = W_router.shape[0]
    d_ff = W_gate.shape[1]
    dt = x.dtype
    _require(replicas, "replicas", torch.int32, (E,))
    R = int(replicas.sum().item())
    C = moe_capacity(T, E, k, cf)
    dev = x.device
    i32 = dict(dtype=torch.int32, device=dev)
    res = {"C": C, "R": R, "out": torch.empty_like(x), "topk_idx": torch.empty((T, k), **i32),
           "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev), "slot": torch.empty((T, k), **i32),
           "instance": torch.empty((T, k), **i32), "routed_count": torch.empty(E, **i32),
           "kept_count": torch.empty(R, **i32), "send_count": torch.empty(P, **i32),
           "totals": torch.empty(4, dtype=torch.int64, device=dev)}
    if want_buckets:
        res["buckets"] = torch.empty((R, C, d), dtype=dt, device=dev)
    if want_src:
        res["src"] = torch.empty((R, C), **i32)
    nbytes = moe_replicated_workspace_size(T, d, d_ff, E, k, cf, P, R, dt)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    moe_layer_forward_replicated(x, W_router, router_bias, W_gate, W_up, W_down, T, d, d_ff, E, k, cf, P, max_ranks,
                                 replicas, R, dt, res["out"], res, workspace, nbytes, stream)
    res["workspace"] = workspace
    return res
