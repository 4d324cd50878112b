"""Python binding of libmoe, the MI355X (gfx950) MoE FFN layer library.

Argument marshalling only: every step of the layer runs in the HIP kernels
of libmoe.so (C ABI in include/moe.h).  PyTorch supplies device memory and
the stream.  The binding checks that every tensor lives on the GPU and has
the size the shape implies, so the library never sees a host pointer or a
short buffer; it then calls the entry point of the same name and raises
MoeError on any status other than MOE_OK.

There is no fallback: if libmoe.so is missing the import of this module
fails loudly (build it with `python mixture_experts_sparse_router_amd/build.py`).
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

MOE_DT_F32 = 0
MOE_DT_BF16 = 1

WS_NAMES = ("topk_idx", "topk_w", "counts", "offsets", "sorted_slot", "slot_pos",
            "act", "expert_out")

ENTRY_POINTS = ("moe_status_string", "moe_version", "moe_last_hip_error", "moe_route", "moe_permute",
                "moe_grouped_gemm_gate_up", "moe_grouped_gemm_down", "moe_grouped_gemm",
                "moe_combine", "moe_workspace_size", "moe_workspace_offsets",
                "moe_layer_forward", "moe_layer_forward_static",
                "moe_route_balance_workspace_size", "moe_route_balance",
                "moe_permute_capacity", "moe_expert_capacity",
                "moe_layer_forward_capacity", "moe_grouped_gemm_gate_up_mxfp4",
                "moe_grouped_gemm_down_mxfp4", "moe_layer_forward_mxfp4",
                "moe_backward_workspace_size", "moe_layer_backward",
                "moe_route_workspace_size", "moe_route_ws")

# size of the library's static intermediate array (include/moe.h)
STATIC_SCRATCH_BYTES = 32 << 20


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = f"{fn} returned {status_string(status)} ({status})"
        if status == MOE_ERR_HIP:
            msg += f": {last_hip_error()}"
        super().__init__(msg)


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("f", ctypes.c_int64),
                ("E", ctypes.c_int64), ("k", ctypes.c_int64), ("n_shared", ctypes.c_int64),
                ("dt", ctypes.c_int32)]

    @property
    def R(self):
        return self.T * self.k + self.n_shared * self.T

    @property
    def G(self):
        return self.E + self.n_shared


def _load():
    # torch first: its bundled HIP runtime (soname libamdhip64.so.7) then
    # serves libmoe's dependency too, so torch's allocations and streams and
    # libmoe's launches share one runtime in the process
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python mixture_experts_sparse_router_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sp = ctypes.c_void_p, ctypes.POINTER(moe_shape)
    i = ctypes.c_int
    L.moe_status_string.argtypes = [i]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_version.argtypes = []
    L.moe_version.restype = ctypes.c_char_p
    L.moe_last_hip_error.argtypes = []
    L.moe_last_hip_error.restype = ctypes.c_char_p
    L.moe_workspace_size.argtypes = [sp]
    L.moe_workspace_size.restype = ctypes.c_size_t
    L.moe_workspace_offsets.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_route_balance_workspace_size.argtypes = [sp]
    L.moe_route_balance_workspace_size.restype = ctypes.c_size_t
    L.moe_route_workspace_size.argtypes = [sp]
    L.moe_route_workspace_size.restype = ctypes.c_size_t
    i64 = ctypes.c_int64
    L.moe_expert_capacity.argtypes = [i64, i64, i64, ctypes.c_double]
    L.moe_expert_capacity.restype = i64
    L.moe_backward_workspace_size.argtypes = [sp]
    L.moe_backward_workspace_size.restype = ctypes.c_size_t
    sigs = {
        "moe_route": [sp, vp, vp, vp, vp, vp, vp],
        "moe_route_ws": [sp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "moe_permute": [sp, vp, vp, vp, vp, vp, vp],
        "moe_grouped_gemm_gate_up": [sp, vp, vp, vp, vp, vp, vp],
        "moe_grouped_gemm_down": [sp, vp, vp, vp, vp, vp],
        "moe_grouped_gemm": [sp, vp, vp, vp, vp, vp, vp, vp, vp],
        "moe_combine": [sp, vp, vp, vp, vp, vp],
        "moe_layer_forward": [sp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "moe_layer_forward_static": [sp, vp, vp, vp, vp, vp, vp, vp],
        "moe_route_balance": [sp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "moe_permute_capacity": [sp, vp, i64, vp, vp, vp, vp, vp],
        "moe_layer_forward_capacity": [sp, vp, vp, vp, vp, vp, i64, vp, vp, ctypes.c_size_t,
                                       vp],
        "moe_grouped_gemm_gate_up_mxfp4": [sp, vp, vp, vp, vp, vp, vp, vp],
        "moe_grouped_gemm_down_mxfp4": [sp, vp, vp, vp, vp, vp, vp],
        "moe_layer_forward_mxfp4": [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                    vp],
        "moe_layer_backward": [sp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp, vp, vp, vp,
                               vp, vp, ctypes.c_size_t, vp],
    }
    for name, argtypes in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = argtypes
        fn.restype = i
    L.moe_workspace_offsets.restype = i
    return L


_lib = _load()


def lib():
    return _lib


def status_string(status: int) -> str:
    return _lib.moe_status_string(int(status)).decode()


def version() -> str:
    return _lib.moe_version().decode()


def last_hip_error() -> str:
    return _lib.moe_last_hip_error().decode()


def shape(T, d, f, E, k, n_shared=0, dt=MOE_DT_BF16) -> moe_shape:
    return moe_shape(int(T), int(d), int(f), int(E), int(k), int(n_shared), int(dt))


def workspace_size(s: moe_shape) -> int:
    return int(_lib.moe_workspace_size(ctypes.byref(s)))


def route_workspace_size(s: moe_shape) -> int:
    return int(_lib.moe_route_workspace_size(ctypes.byref(s)))


def route_balance_workspace_size(s: moe_shape) -> int:
    return int(_lib.moe_route_balance_workspace_size(ctypes.byref(s)))


def backward_workspace_size(s: moe_shape) -> int:
    return int(_lib.moe_backward_workspace_size(ctypes.byref(s)))


def expert_capacity(T, k, E, capacity_factor) -> int:
    """ceil(capacity_factor * T*k / E) (moe_expert_capacity); -1 if invalid."""
    return int(_lib.moe_expert_capacity(int(T), int(k), int(E), float(capacity_factor)))


def workspace_offsets(s: moe_shape) -> dict:
    out = (ctypes.c_size_t * len(WS_NAMES))()
    rc = _lib.moe_workspace_offsets(ctypes.byref(s), out)
    if rc != MOE_OK:
        raise MoeError("moe_workspace_offsets", rc)
    return dict(zip(WS_NAMES, (int(v) for v in out)))


# ------------------------------------------------------------ marshalling

def _torch():
    import torch
    return torch


def _float_dtype(s: moe_shape):
    torch = _torch()
    return torch.bfloat16 if s.dt == MOE_DT_BF16 else torch.float32


def _ptr(t, numel, dtype, name, optional=False):
    """Device pointer of tensor t after checking device, dtype, size, layout."""
    if t is None:
        if optional or numel == 0:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, the shape needs {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if numel else None


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _call(name, *args):
    rc = getattr(_lib, name)(*args)
    if rc != MOE_OK:
        raise MoeError(name, rc)


def moe_route(s: moe_shape, x, W_router, bias, topk_idx, topk_w, stream=None):
    torch = _torch()
    fd = _float_dtype(s)
    _call("moe_route", ctypes.byref(s),
          _ptr(x, s.T * s.d, fd, "x"),
          _ptr(W_router, s.E * s.d, fd, "W_router"),
          _ptr(bias, s.E, torch.float32, "bias", optional=True),
          _ptr(topk_idx, s.T * s.k, torch.int32, "topk_idx"),
          _ptr(topk_w, s.T * s.k, torch.float32, "topk_w"),
          _stream(stream))


def moe_route_ws(s: moe_shape, x, W_router, bias, topk_idx, topk_w, workspace, stream=None):
    """moe_route with a workspace of route_workspace_size(s) bytes (uint8 GPU
    tensor, or None when that size is 0)."""
    torch = _torch()
    fd = _float_dtype(s)
    ws_ptr, ws_bytes = _workspace(workspace)
    _call("moe_route_ws", ctypes.byref(s),
          _ptr(x, s.T * s.d, fd, "x"),
          _ptr(W_router, s.E * s.d, fd, "W_router"),
          _ptr(bias, s.E, torch.float32, "bias", optional=True),
          _ptr(topk_idx, s.T * s.k, torch.int32, "topk_idx"),
          _ptr(topk_w, s.T * s.k, torch.float32, "topk_w"),
          ws_ptr, ws_bytes, _stream(stream))


def moe_route_balance(s: moe_shape, x, W_router, bias, topk_idx, topk_w, importance, loss,
                      workspace, stream=None):
    """moe_route plus importance[E] (float64) and the balance loss ([1] float64)."""
    torch = _torch()
    fd = _float_dtype(s)
    ws_ptr, ws_bytes = _workspace(workspace)
    _call("moe_route_balance", ctypes.byref(s),
          _ptr(x, s.T * s.d, fd, "x"),
          _ptr(W_router, s.E * s.d, fd, "W_router"),
          _ptr(bias, s.E, torch.float32, "bias", optional=True),
          _ptr(topk_idx, s.T * s.k, torch.int32, "topk_idx"),
          _ptr(topk_w, s.T * s.k, torch.float32, "topk_w"),
          _ptr(importance, s.E, torch.float64, "importance"),
          _ptr(loss, 1, torch.float64, "loss"),
          ws_ptr, ws_bytes, _stream(stream))


def moe_permute_capacity(s: moe_shape, topk_idx, capacity, counts, offsets, sorted_slot,
                         slot_pos, stream=None):
    i32 = _torch().int32
    _call("moe_permute_capacity", ctypes.byref(s),
          _ptr(topk_idx, s.T * s.k, i32, "topk_idx"),
          int(capacity),
          _ptr(counts, s.G, i32, "counts"),
          _ptr(offsets, s.G + 1, i32, "offsets"),
          _ptr(sorted_slot, s.T * s.k, i32, "sorted_slot"),
          _ptr(slot_pos, s.T * s.k, i32, "slot_pos"),
          _stream(stream))


def moe_permute(s: moe_shape, topk_idx, counts, offsets, sorted_slot, slot_pos,
                stream=None):
    i32 = _torch().int32
    _call("moe_permute", ctypes.byref(s),
          _ptr(topk_idx, s.T * s.k, i32, "topk_idx"),
          _ptr(counts, s.G, i32, "counts"),
          _ptr(offsets, s.G + 1, i32, "offsets"),
          _ptr(sorted_slot, s.T * s.k, i32, "sorted_slot"),
          _ptr(slot_pos, s.T * s.k, i32, "slot_pos"),
          _stream(stream))


def moe_grouped_gemm_gate_up(s: moe_shape, x, sorted_slot, offsets, W_gate_up, act,
                             stream=None):
    i32, fd = _torch().int32, _float_dtype(s)
    _call("moe_grouped_gemm_gate_up", ctypes.byref(s),
          _ptr(x, s.T * s.d, fd, "x"),
          _ptr(sorted_slot, s.T * s.k, i32, "sorted_slot"),
          _ptr(offsets, s.G + 1, i32, "offsets"),
          _ptr(W_gate_up, s.G * 2 * s.f * s.d, fd, "W_gate_up"),
          _ptr(act, s.R * s.f, fd, "act"),
          _stream(stream))


def moe_grouped_gemm_down(s: moe_shape, act, offsets, W_down, expert_out, stream=None):
    i32, fd = _torch().int32, _float_dtype(s)
    _call("moe_grouped_gemm_down", ctypes.byref(s),
          _ptr(act, s.R * s.f, fd, "act"),
          _ptr(offsets, s.G + 1, i32, "offsets"),
          _ptr(W_down, s.G * s.d * s.f, fd, "W_down"),
          _ptr(expert_out, s.R * s.d, fd, "expert_out"),
          _stream(stream))


def moe_grouped_gemm(s: moe_shape, x, sorted_slot, offsets, W_gate_up, W_down, act,
                     expert_out, stream=None):
    i32, fd = _torch().int32, _float_dtype(s)
    _call("moe_grouped_gemm", ctypes.byref(s),
          _ptr(x, s.T * s.d, fd, "x"),
          _ptr(sorted_slot, s.T * s.k, i32, "sorted_slot"),
          _ptr(offsets, s.G + 1, i32, "offsets"),
          _ptr(W_gate_up, s.G * 2 * s.f * s.d, fd, "W_gate_up"),
          _ptr(W_down, s.G * s.d * s.f, fd, "W_down"),
          _ptr(act, s.R * s.f, fd, "act"),
          _ptr(expert_out, s.R * s.d, fd, "expert_out"),
          _stream(stream))


def moe_combine(s: moe_shape, expert_out, slot_pos, topk_w, y, stream=None):
    torch = _torch()
    fd = _float_dtype(s)
    _call("moe_combine", ctypes.byref(s),
          _ptr(expert_out, s.R * s.d, fd, "expert_out"),
          _ptr(slot_pos, s.T * s.k, torch.int32, "slot_pos"),
          _ptr(topk_w, s.T * s.k, torch.float32, "topk_w"),
          _ptr(y, s.T * s.d, fd, "y"),
          _stream(stream))


def _workspace(workspace):
    """(pointer, bytes) of a uint8 GPU workspace tensor (None: no workspace)."""
    torch = _torch()
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 GPU tensor")
    if workspace.data_ptr() % 256:
        raise ValueError("workspace must be 256-byte aligned")
    return workspace.data_ptr(), workspace.numel()


def moe_layer_forward(s: moe_shape, x, W_router, bias, W_gate_up, W_down, y, workspace,
                      stream=None):
    torch = _torch()
    fd = _float_dtype(s)
    if workspace is None:
        raise ValueError("workspace must be a uint8 GPU tensor")
    ws_ptr, ws_bytes = _workspace(workspace)
    _call("moe_layer_forward", ctypes.byref(s),
          _ptr(x, s.T * s.d, fd, "x"),
          _ptr(W_router, s.E * s.d, fd, "W_router"),
          _ptr(bias, s.E, torch.float32, "bias", optional=True),
          _ptr(W_gate_up, s.G * 2 * s.f * s.d, fd, "W_gate_up"),
          _ptr(W_down, s.G * s.d * s.f, fd, "W_down"),
          _ptr(y, s.T * s.d, fd, "y"),
          ws_ptr, ws_bytes,
          _stream(stream))


def moe_layer_forward_capacity(s: moe_shape, x, W_router, bias, W_gate_up, W_down, capacity,
                               y, workspace, stream=None):
    """The layer with an expert capacity (moe_layer_forward's workspace)."""
    torch = _torch()
    fd = _float_dtype(s)
    if workspace is None:
        raise ValueError("workspace must be a uint8 GPU tensor")
    ws_ptr, ws_bytes = _workspace(workspace)
    _call("moe_layer_forward_capacity", ctypes.byref(s),
          _ptr(x, s.T * s.d, fd, "x"),
          _ptr(W_router, s.E * s.d, fd, "W_router"),
          _ptr(bias, s.E, torch.float32, "bias", optional=True),
          _ptr(W_gate_up, s.G * 2 * s.f * s.d, fd, "W_gate_up"),
          _ptr(W_down, s.G * s.d * s.f, fd, "W_down"),
          int(capacity),
          _ptr(y, s.T * s.d, fd, "y"),
          ws_ptr, ws_bytes,
          _stream(stream))


def moe_layer_forward_static(s: moe_shape, x, W_router, bias, W_gate_up, W_down, y,
                             stream=None):
    """moe_layer_forward with the library's static intermediate array (no
    workspace, no allocation; shapes up to STATIC_SCRATCH_BYTES of
    intermediates; calls on one GPU must not overlap)."""
    torch = _torch()
    fd = _float_dtype(s)
    _call("moe_layer_forward_static", ctypes.byref(s),
          _ptr(x, s.T * s.d, fd, "x"),
          _ptr(W_router, s.E * s.d, fd, "W_router"),
          _ptr(bias, s.E, torch.float32, "bias", optional=True),
          _ptr(W_gate_up, s.G * 2 * s.f * s.d, fd, "W_gate_up"),
          _ptr(W_down, s.G * s.d * s.f, fd, "W_down"),
          _ptr(y, s.T * s.d, fd, "y"),
          _stream(stream))


def moe_grouped_gemm_gate_up_mxfp4(s: moe_shape, x, sorted_slot, offsets, Wq_gate_up,
                                   Ws_gate_up, act, stream=None):
    torch = _torch()
    i32, u8, fd = torch.int32, torch.uint8, _float_dtype(s)
    _call("moe_grouped_gemm_gate_up_mxfp4", ctypes.byref(s),
          _ptr(x, s.T * s.d, fd, "x"),
          _ptr(sorted_slot, s.T * s.k, i32, "sorted_slot"),
          _ptr(offsets, s.G + 1, i32, "offsets"),
          _ptr(Wq_gate_up, s.G * 2 * s.f * (s.d // 2), u8, "Wq_gate_up"),
          _ptr(Ws_gate_up, s.G * 2 * s.f * (s.d // 32), u8, "Ws_gate_up"),
          _ptr(act, s.R * s.f, fd, "act"),
          _stream(stream))


def moe_grouped_gemm_down_mxfp4(s: moe_shape, act, offsets, Wq_down, Ws_down, expert_out,
                                stream=None):
    torch = _torch()
    i32, u8, fd = torch.int32, torch.uint8, _float_dtype(s)
    _call("moe_grouped_gemm_down_mxfp4", ctypes.byref(s),
          _ptr(act, s.R * s.f, fd, "act"),
          _ptr(offsets, s.G + 1, i32, "offsets"),
          _ptr(Wq_down, s.G * s.d * (s.f // 2), u8, "Wq_down"),
          _ptr(Ws_down, s.G * s.d * (s.f // 32), u8, "Ws_down"),
          _ptr(expert_out, s.R * s.d, fd, "expert_out"),
          _stream(stream))


def moe_layer_forward_mxfp4(s: moe_shape, x, W_router, bias, Wq_gate_up, Ws_gate_up, Wq_down,
                            Ws_down, y, workspace, stream=None):
    """The layer with MXFP4 expert weights (moe_layer_forward's workspace)."""
    torch = _torch()
    u8, fd = torch.uint8, _float_dtype(s)
    if workspace is None:
        raise ValueError("workspace must be a uint8 GPU tensor")
    ws_ptr, ws_bytes = _workspace(workspace)
    _call("moe_layer_forward_mxfp4", ctypes.byref(s),
          _ptr(x, s.T * s.d, fd, "x"),
          _ptr(W_router, s.E * s.d, fd, "W_router"),
          _ptr(bias, s.E, torch.float32, "bias", optional=True),
          _ptr(Wq_gate_up, s.G * 2 * s.f * (s.d // 2), u8, "Wq_gate_up"),
          _ptr(Ws_gate_up, s.G * 2 * s.f * (s.d // 32), u8, "Ws_gate_up"),
          _ptr(Wq_down, s.G * s.d * (s.f // 2), u8, "Wq_down"),
          _ptr(Ws_down, s.G * s.d * (s.f // 32), u8, "Ws_down"),
          _ptr(y, s.T * s.d, fd, "y"),
          ws_ptr, ws_bytes, _stream(stream))


def moe_layer_backward(s: moe_shape, x, W_router, W_gate_up, W_down, dy, fwd_workspace, dx,
                       dW_router, db, dW_gate_up, dW_down, dw, workspace, stream=None):
    """Gradients (float32) of the layer given dy, using the forward call's
    workspace (routing, permutation, act, expert_out); dw may be None."""
    torch = _torch()
    fd, f32 = _float_dtype(s), torch.float32
    fw_ptr, fw_bytes = _workspace(fwd_workspace)
    ws_ptr, ws_bytes = _workspace(workspace)
    _call("moe_layer_backward", ctypes.byref(s),
          _ptr(x, s.T * s.d, fd, "x"),
          _ptr(W_router, s.E * s.d, fd, "W_router"),
          _ptr(W_gate_up, s.G * 2 * s.f * s.d, fd, "W_gate_up"),
          _ptr(W_down, s.G * s.d * s.f, fd, "W_down"),
          _ptr(dy, s.T * s.d, fd, "dy"),
          fw_ptr, fw_bytes,
          _ptr(dx, s.T * s.d, f32, "dx"),
          _ptr(dW_router, s.E * s.d, f32, "dW_router"),
          _ptr(db, s.E, f32, "db"),
          _ptr(dW_gate_up, s.G * 2 * s.f * s.d, f32, "dW_gate_up"),
          _ptr(dW_down, s.G * s.d * s.f, f32, "dW_down"),
          _ptr(dw, s.T * s.k, f32, "dw", optional=True),
          ws_ptr, ws_bytes, _stream(stream))


def workspace_views(s: moe_shape, workspace) -> dict:
    """Typed views of the intermediates inside a layer workspace (for tests
    and inspection; the layout is the one moe_workspace_offsets reports)."""
    torch = _torch()
    off = workspace_offsets(s)
    fd = _float_dtype(s)
    es = 2 if s.dt == MOE_DT_BF16 else 4
    spec = {
        "topk_idx": (torch.int32, 4, (s.T, s.k)),
        "topk_w": (torch.float32, 4, (s.T, s.k)),
        "counts": (torch.int32, 4, (s.G,)),
        "offsets": (torch.int32, 4, (s.G + 1,)),
        "sorted_slot": (torch.int32, 4, (s.T * s.k,)),
        "slot_pos": (torch.int32, 4, (s.T * s.k,)),
        "act": (fd, es, (s.R, s.f)),
        "expert_out": (fd, es, (s.R, s.d)),
    }
    views = {}
    for name, (dt, size, shp) in spec.items():
        n = 1
        for v in shp:
            n *= v
        views[name] = workspace[off[name]: off[name] + n * size].view(dt).view(*shp)
    return views
