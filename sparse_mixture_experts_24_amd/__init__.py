"""MI355X (gfx950) sparse mixture-of-experts FFN forward pass.

Thin ctypes binding over libmoe.so (C ABI in include/moe.h).  PyTorch supplies device
memory and the current HIP stream; every step of the layer runs in the library's HIP
kernels.  The functions mirror the C entry points:

    forward(x, W_router, router_bias, W_gate, W_up, W_down, k, capacity_factor, ...)
    route(...), dispatch(...), experts(...), combine(...)
    forward_fp8(...) and the *_fp8 stages (8-bit expert weights)
    forward_expert_choice(...), route_expert_choice(...), combine_expert_choice(...)
    forward_next_best(...), route_next_best(...), dispatch_next_best(...) (capacity
    overflow handed to the next-best expert)

There is no fallback: without the built library (python -m
sparse_mixture_experts_24_amd.build) every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
STATUS = {0: "MOE_OK", 1: "MOE_E_NULL", 2: "MOE_E_SHAPE", 3: "MOE_E_UNSUPPORTED",
          4: "MOE_E_WORKSPACE", 5: "MOE_E_HIP", 6: "MOE_E_SCRATCH"}
EXPORTS = ("moe_status_str", "moe_validate", "moe_workspace_bytes", "moe_capacity",
           "moe_forward", "moe_route", "moe_dispatch", "moe_experts", "moe_experts_gate_up",
           "moe_experts_down", "moe_combine", "moe_forward_fp8", "moe_experts_fp8",
           "moe_experts_gate_up_fp8", "moe_experts_down_fp8",
           "moe_workspace_bytes_expert_choice", "moe_capacity_expert_choice",
           "moe_route_expert_choice", "moe_combine_expert_choice", "moe_forward_expert_choice",
           "moe_forward_next_best", "moe_route_next_best", "moe_dispatch_next_best",
           "moe_forward_noalloc")
# Bytes of the library's static device scratch that moe_forward_noalloc uses (moe.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeDesc(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("d_model", ctypes.c_int64), ("n_experts", ctypes.c_int64),
        ("d_ff", ctypes.c_int64), ("top_k", ctypes.c_int64), ("n_shared", ctypes.c_int64),
        ("capacity_factor", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: "
                         f"{lib().moe_status_str(status).decode()}")
        self.status = status


_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m sparse_mixture_experts_24_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        D = ctypes.POINTER(MoeDesc)
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [I]
        L.moe_validate.restype = I
        L.moe_validate.argtypes = [D]
        L.moe_workspace_bytes.restype = S
        L.moe_workspace_bytes.argtypes = [D]
        L.moe_capacity.restype = ctypes.c_int64
        L.moe_capacity.argtypes = [D]
        L.moe_forward.restype = I
        L.moe_forward.argtypes = [D, P, P, P, P, P, P, P, P, P, P, S, P]
        L.moe_route.restype = I
        L.moe_route.argtypes = [D, P, P, P, P, P, P, P, P, P, S, P]
        L.moe_dispatch.restype = I
        L.moe_dispatch.argtypes = [D, P, P, P, P, P, P, S, P]
        L.moe_experts.restype = I
        L.moe_experts.argtypes = [D, P, P, P, P, P, P, P, P, P, S, P]
        L.moe_experts_gate_up.restype = I
        L.moe_experts_gate_up.argtypes = [D, P, P, P, P, P, P, P, S, P]
        L.moe_experts_down.restype = I
        L.moe_experts_down.argtypes = [D, P, P, P, P, P, S, P]
        L.moe_combine.restype = I
        L.moe_combine.argtypes = [D, P, P, P, P, P]
        L.moe_forward_fp8.restype = I
        L.moe_forward_fp8.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
        L.moe_experts_fp8.restype = I
        L.moe_experts_fp8.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
        L.moe_experts_gate_up_fp8.restype = I
        L.moe_experts_gate_up_fp8.argtypes = [D, P, P, P, P, P, P, P, P, P, S, P]
        L.moe_experts_down_fp8.restype = I
        L.moe_experts_down_fp8.argtypes = [D, P, P, P, P, P, P, S, P]
        L.moe_workspace_bytes_expert_choice.restype = S
        L.moe_workspace_bytes_expert_choice.argtypes = [D]
        L.moe_capacity_expert_choice.restype = ctypes.c_int64
        L.moe_capacity_expert_choice.argtypes = [D]
        L.moe_route_expert_choice.restype = I
        L.moe_route_expert_choice.argtypes = [D, P, P, P, P, P, P, P, P, P, S, P]
        L.moe_combine_expert_choice.restype = I
        L.moe_combine_expert_choice.argtypes = [D, P, P, P, P, P]
        L.moe_forward_expert_choice.restype = I
        L.moe_forward_expert_choice.argtypes = [D, P, P, P, P, P, P, P, P, P, S, P]
        L.moe_forward_next_best.restype = I
        L.moe_forward_next_best.argtypes = [D, P, P, P, P, P, P, P, P, P, P, S, P]
        L.moe_route_next_best.restype = I
        L.moe_route_next_best.argtypes = [D, P, P, P, P, P, P, P, P, P, S, P]
        L.moe_dispatch_next_best.restype = I
        L.moe_dispatch_next_best.argtypes = [D, P, P, P, P, P, P, P, S, P]
        L.moe_forward_noalloc.restype = I
        L.moe_forward_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
        _lib = L
    return _lib


def _dt(t: torch.dtype) -> int:
    if t == torch.float32:
        return MOE_DTYPE_F32
    if t == torch.bfloat16:
        return MOE_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")


def make_desc(T, d_model, n_experts, d_ff, top_k, n_shared=0, capacity_factor=0.0,
              dtype=torch.bfloat16, out_dtype=None) -> MoeDesc:
    return MoeDesc(int(T), int(d_model), int(n_experts), int(d_ff), int(top_k), int(n_shared),
                   float(capacity_factor), _dt(dtype), _dt(out_dtype or dtype))


def desc_for(x, W_router, W_gate, k, capacity_factor=0.0, out_dtype=None) -> MoeDesc:
    T, d = x.shape
    E = W_router.shape[0]
    G, F, _ = W_gate.shape
    return make_desc(T, d, E, F, k, G - E, capacity_factor, x.dtype, out_dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn, status):
    if status != 0:
        raise MoeError(fn, status)


def _require(t, name, device, dtype=None, shape=None):
    if t is None:
        return
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def workspace_bytes(desc: MoeDesc) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(desc)))


def capacity(desc: MoeDesc):
    c = int(lib().moe_capacity(ctypes.byref(desc)))
    return None if c < 0 else c


def validate(desc: MoeDesc) -> int:
    return int(lib().moe_validate(ctypes.byref(desc)))


def alloc_workspace(desc: MoeDesc, device) -> torch.Tensor:
    n = workspace_bytes(desc)
    if n == 0:
        _check("moe_workspace_bytes", validate(desc) or 2)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _ws(desc, device, workspace):
    if workspace is None:
        workspace = alloc_workspace(desc, device)
    return workspace


def forward(x, W_router, router_bias, W_gate, W_up, W_down, k, capacity_factor=0.0,
            out=None, f=None, p=None, out_dtype=None, workspace=None, want_stats=True):
    """The whole MoE layer on the GPU.  Returns (y, f, p)."""
    dev = x.device
    desc = desc_for(x, W_router, W_gate, k, capacity_factor, out_dtype)
    T, d = x.shape
    E = W_router.shape[0]
    G, F, _ = W_gate.shape
    for t, n, shp in ((x, "x", (T, d)), (W_router, "W_router", (E, d)),
                      (W_gate, "W_gate", (G, F, d)), (W_up, "W_up", (G, F, d)),
                      (W_down, "W_down", (G, d, F))):
        _require(t, n, dev, x.dtype, shp)
    _require(router_bias, "router_bias", dev, torch.float32, (E,))
    odt = out_dtype or x.dtype
    if out is None:
        out = torch.empty(T, d, dtype=odt, device=dev)
    if want_stats:
        f = torch.empty(E, dtype=torch.float32, device=dev) if f is None else f
        p = torch.empty(E, dtype=torch.float32, device=dev) if p is None else p
    _require(out, "out", dev, odt, (T, d))
    ws = _ws(desc, dev, workspace)
    st = lib().moe_forward(ctypes.byref(desc), _ptr(x), _ptr(W_router), _ptr(router_bias),
                           _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(out), _ptr(f), _ptr(p),
                           _ptr(ws), ws.numel(), _stream(dev))
    _check("moe_forward", st)
    return out, f, p


def forward_noalloc(x, W_router, router_bias, W_gate, W_up, W_down, k, capacity_factor=0.0, *,
                    out, f=None, p=None, out_dtype=None):
    """The whole layer through moe_forward_noalloc: no workspace, the library's static
    device scratch instead (NOALLOC_SCRATCH_BYTES per GPU; larger layers raise with
    MOE_E_SCRATCH).  `out` (and f, p, if wanted) must be given, so that nothing is
    allocated here either.  Calls that overlap on one GPU race on that scratch."""
    dev = x.device
    desc = desc_for(x, W_router, W_gate, k, capacity_factor, out_dtype)
    T, d = x.shape
    E = W_router.shape[0]
    G, F, _ = W_gate.shape
    for t, n, shp in ((x, "x", (T, d)), (W_router, "W_router", (E, d)),
                      (W_gate, "W_gate", (G, F, d)), (W_up, "W_up", (G, F, d)),
                      (W_down, "W_down", (G, d, F))):
        _require(t, n, dev, x.dtype, shp)
    _require(router_bias, "router_bias", dev, torch.float32, (E,))
    if out is None:
        raise ValueError("forward_noalloc needs the output tensor `out`")
    _require(out, "out", dev, out_dtype or x.dtype, (T, d))
    _require(f, "f", dev, torch.float32, (E,))
    _require(p, "p", dev, torch.float32, (E,))
    st = lib().moe_forward_noalloc(ctypes.byref(desc), _ptr(x), _ptr(W_router),
                                   _ptr(router_bias), _ptr(W_gate), _ptr(W_up), _ptr(W_down),
                                   _ptr(out), _ptr(f), _ptr(p), _stream(dev))
    _check("moe_forward_noalloc", st)
    return out, f, p


def _require_fp8(q, s, name, dev, shape):
    _require(q, "Wq_" + name, dev, torch.uint8, shape)
    _require(s, "s_" + name, dev, torch.float32, shape[:2])


def forward_fp8(x, W_router, router_bias, Wq_gate, Wq_up, Wq_down, s_gate, s_up, s_down, k,
                capacity_factor=0.0, out=None, f=None, p=None, out_dtype=None, workspace=None,
                want_stats=True):
    """The whole layer with 8-bit (e4m3, per-row scale) expert weights: uint8 codes
    Wq_* shaped like the bf16 weights, float32 scales s_gate/s_up [E+S, F], s_down
    [E+S, d].  x and W_router bf16.  Returns (y, f, p)."""
    dev = x.device
    T, d = x.shape
    E = W_router.shape[0]
    G, F, _ = Wq_gate.shape
    desc = make_desc(T, d, E, F, k, G - E, capacity_factor, x.dtype, out_dtype or x.dtype)
    _require(x, "x", dev, x.dtype, (T, d))
    _require(W_router, "W_router", dev, x.dtype, (E, d))
    _require_fp8(Wq_gate, s_gate, "gate", dev, (G, F, d))
    _require_fp8(Wq_up, s_up, "up", dev, (G, F, d))
    _require_fp8(Wq_down, s_down, "down", dev, (G, d, F))
    _require(router_bias, "router_bias", dev, torch.float32, (E,))
    odt = out_dtype or x.dtype
    if out is None:
        out = torch.empty(T, d, dtype=odt, device=dev)
    if want_stats:
        f = torch.empty(E, dtype=torch.float32, device=dev) if f is None else f
        p = torch.empty(E, dtype=torch.float32, device=dev) if p is None else p
    _require(out, "out", dev, odt, (T, d))
    ws = _ws(desc, dev, workspace)
    st = lib().moe_forward_fp8(ctypes.byref(desc), _ptr(x), _ptr(W_router), _ptr(router_bias),
                               _ptr(Wq_gate), _ptr(Wq_up), _ptr(Wq_down), _ptr(s_gate),
                               _ptr(s_up), _ptr(s_down), _ptr(out), _ptr(f), _ptr(p), _ptr(ws),
                               ws.numel(), _stream(dev))
    _check("moe_forward_fp8", st)
    return out, f, p


def experts_gate_up_fp8(x, perm_src, offsets, Wq_gate, Wq_up, s_gate, s_up, k, n_experts,
                        H=None, workspace=None):
    """Gate/up grouped GEMM on 8-bit weights.  Returns H (x.dtype)."""
    dev = x.device
    T, d = x.shape
    G, F, _ = Wq_gate.shape
    desc = make_desc(T, d, n_experts, F, k, G - n_experts, 0.0, x.dtype)
    rows = T * k + (G - n_experts) * T
    if H is None:
        H = torch.empty(rows, F, dtype=x.dtype, device=dev)
    _require(H, "H", dev, x.dtype, (rows, F))
    _require_fp8(Wq_gate, s_gate, "gate", dev, (G, F, d))
    _require_fp8(Wq_up, s_up, "up", dev, (G, F, d))
    ws, wsb = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    st = lib().moe_experts_gate_up_fp8(ctypes.byref(desc), _ptr(x), _ptr(perm_src),
                                       _ptr(offsets), _ptr(Wq_gate), _ptr(Wq_up), _ptr(s_gate),
                                       _ptr(s_up), _ptr(H), ws, wsb, _stream(dev))
    _check("moe_experts_gate_up_fp8", st)
    return H


def experts_down_fp8(H, offsets, Wq_down, s_down, T, k, n_experts, Yp=None, workspace=None):
    """Down grouped GEMM on 8-bit weights.  Returns Yp (float32)."""
    dev = H.device
    G, d, F = Wq_down.shape
    desc = make_desc(T, d, n_experts, F, k, G - n_experts, 0.0, H.dtype)
    rows = T * k + (G - n_experts) * T
    if Yp is None:
        Yp = torch.empty(rows, d, dtype=torch.float32, device=dev)
    _require(Yp, "Yp", dev, torch.float32, (rows, d))
    _require_fp8(Wq_down, s_down, "down", dev, (G, d, F))
    ws, wsb = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    st = lib().moe_experts_down_fp8(ctypes.byref(desc), _ptr(H), _ptr(offsets), _ptr(Wq_down),
                                    _ptr(s_down), _ptr(Yp), ws, wsb, _stream(dev))
    _check("moe_experts_down_fp8", st)
    return Yp


def route(x, W_router, router_bias, k, workspace=None, W_gate_shape=None, n_shared=0,
          want_gap=False):
    """Router + top-k + renorm + statistics.  Returns (topk_idx, topk_w, f, p), and the
    per-token gap s_(k) - s_(k+1) as a fifth value when want_gap."""
    dev = x.device
    T, d = x.shape
    E = W_router.shape[0]
    desc = make_desc(T, d, E, 64, k, n_shared, 0.0, x.dtype)
    _require(x, "x", dev)
    _require(W_router, "W_router", dev, x.dtype, (E, d))
    _require(router_bias, "router_bias", dev, torch.float32, (E,))
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    f = torch.empty(E, dtype=torch.float32, device=dev)
    p = torch.empty(E, dtype=torch.float32, device=dev)
    gap = torch.empty(T, dtype=torch.float32, device=dev) if want_gap else None
    ws = _ws(desc, dev, workspace)
    st = lib().moe_route(ctypes.byref(desc), _ptr(x), _ptr(W_router), _ptr(router_bias),
                         _ptr(idx), _ptr(w), _ptr(gap), _ptr(f), _ptr(p), _ptr(ws), ws.numel(),
                         _stream(dev))
    _check("moe_route", st)
    return (idx, w, f, p, gap) if want_gap else (idx, w, f, p)


def dispatch(topk_idx, n_experts, capacity_factor=0.0, workspace=None):
    """Histogram, capacity, offsets and the stable permutation.
    Returns (counts, offsets, perm_src, slot_pos)."""
    dev = topk_idx.device
    T, k = topk_idx.shape
    desc = make_desc(T, 64, n_experts, 64, k, 0, capacity_factor, torch.bfloat16)
    _require(topk_idx, "topk_idx", dev, torch.int32)
    counts = torch.empty(n_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    perm_src = torch.full((T * k,), -1, dtype=torch.int32, device=dev)
    slot_pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws = _ws(desc, dev, workspace)
    st = lib().moe_dispatch(ctypes.byref(desc), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                            _ptr(perm_src), _ptr(slot_pos), _ptr(ws), ws.numel(), _stream(dev))
    _check("moe_dispatch", st)
    return counts, offsets, perm_src, slot_pos


def experts(x, perm_src, offsets, W_gate, W_up, W_down, k, n_experts, want_h=False,
            workspace=None, capacity_factor=0.0):
    """Grouped SwiGLU experts.  Returns (Yp [T*k + S*T, d] float32, H or None)."""
    dev = x.device
    T, d = x.shape
    G, F, _ = W_gate.shape
    desc = make_desc(T, d, n_experts, F, k, G - n_experts, capacity_factor, x.dtype)
    for t, n, shp in ((x, "x", (T, d)), (W_gate, "W_gate", (G, F, d)),
                      (W_up, "W_up", (G, F, d)), (W_down, "W_down", (G, d, F))):
        _require(t, n, dev, x.dtype, shp)
    _require(perm_src, "perm_src", dev, torch.int32)
    _require(offsets, "offsets", dev, torch.int32, (n_experts + 1,))
    rows = T * k + (G - n_experts) * T
    Yp = torch.zeros(rows, d, dtype=torch.float32, device=dev)
    H = torch.zeros(rows, F, dtype=x.dtype, device=dev) if want_h else None
    ws = _ws(desc, dev, workspace)
    st = lib().moe_experts(ctypes.byref(desc), _ptr(x), _ptr(perm_src), _ptr(offsets),
                           _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(Yp), _ptr(H), _ptr(ws),
                           ws.numel(), _stream(dev))
    _check("moe_experts", st)
    return Yp, H


def experts_gate_up(x, perm_src, offsets, W_gate, W_up, k, n_experts, H=None, workspace=None):
    """Gate/up grouped GEMM with the fused SiLU*mul epilogue.  Returns H.  With a
    workspace (alloc_workspace of the same description) tiles are balanced dynamically."""
    dev = x.device
    T, d = x.shape
    G, F, _ = W_gate.shape
    desc = make_desc(T, d, n_experts, F, k, G - n_experts, 0.0, x.dtype)
    rows = T * k + (G - n_experts) * T
    if H is None:
        H = torch.empty(rows, F, dtype=x.dtype, device=dev)
    _require(H, "H", dev, x.dtype, (rows, F))
    ws, wsb = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    st = lib().moe_experts_gate_up(ctypes.byref(desc), _ptr(x), _ptr(perm_src), _ptr(offsets),
                                   _ptr(W_gate), _ptr(W_up), _ptr(H), ws, wsb, _stream(dev))
    _check("moe_experts_gate_up", st)
    return H


def experts_down(H, offsets, W_down, T, k, n_experts, Yp=None, workspace=None):
    """Down grouped GEMM.  Returns Yp (float32).  Workspace as for experts_gate_up."""
    dev = H.device
    G, d, F = W_down.shape
    desc = make_desc(T, d, n_experts, F, k, G - n_experts, 0.0, H.dtype)
    rows = T * k + (G - n_experts) * T
    if Yp is None:
        Yp = torch.empty(rows, d, dtype=torch.float32, device=dev)
    _require(Yp, "Yp", dev, torch.float32, (rows, d))
    ws, wsb = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    st = lib().moe_experts_down(ctypes.byref(desc), _ptr(H), _ptr(offsets), _ptr(W_down),
                                _ptr(Yp), ws, wsb, _stream(dev))
    _check("moe_experts_down", st)
    return Yp


def combine(Yp, slot_pos, topk_w, T, d, k, n_shared=0, out_dtype=torch.float32, n_experts=None):
    """Weighted combine back to token order.  Returns out [T, d]."""
    dev = Yp.device
    E = n_experts or k
    desc = make_desc(T, d, E, 64, k, n_shared, 0.0, torch.bfloat16, out_dtype)
    _require(Yp, "Yp", dev, torch.float32)
    _require(slot_pos, "slot_pos", dev, torch.int32)
    _require(topk_w, "topk_w", dev, torch.float32)
    out = torch.empty(T, d, dtype=out_dtype, device=dev)
    st = lib().moe_combine(ctypes.byref(desc), _ptr(Yp), _ptr(slot_pos), _ptr(topk_w), _ptr(out),
                           _stream(dev))
    _check("moe_combine", st)
    return out


class MoELayer:
    """Holds the layer's device weights and a reusable workspace."""

    def __init__(self, W_router, W_gate, W_up, W_down, k, capacity_factor=0.0,
                 router_bias=None, out_dtype=None):
        self.W_router, self.W_gate, self.W_up, self.W_down = W_router, W_gate, W_up, W_down
        self.router_bias = router_bias
        self.k = int(k)
        self.capacity_factor = float(capacity_factor)
        self.out_dtype = out_dtype
        self._ws = None
        self._ws_T = None

    def __call__(self, x, out=None, f=None, p=None):
        if self._ws is None or self._ws_T != x.shape[0]:
            desc = desc_for(x, self.W_router, self.W_gate, self.k, self.capacity_factor,
                            self.out_dtype)
            self._ws = alloc_workspace(desc, x.device)
            self._ws_T = x.shape[0]
        return forward(x, self.W_router, self.router_bias, self.W_gate, self.W_up, self.W_down,
                       self.k, self.capacity_factor, out=out, f=f, p=p, out_dtype=self.out_dtype,
                       workspace=self._ws)


# ----------------------------------------------------------------------------- expert choice
def capacity_expert_choice(desc: MoeDesc) -> int:
    """Tokens per expert under expert-choice routing (-1: invalid description)."""
    return int(lib().moe_capacity_expert_choice(ctypes.byref(desc)))


def alloc_workspace_expert_choice(desc: MoeDesc, device) -> torch.Tensor:
    n = int(lib().moe_workspace_bytes_expert_choice(ctypes.byref(desc)))
    if n == 0:
        _check("moe_workspace_bytes_expert_choice", validate(desc) or 2)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _ws_ec(desc, device, workspace):
    return alloc_workspace_expert_choice(desc, device) if workspace is None else workspace


def forward_expert_choice(x, W_router, W_gate, W_up, W_down, k, capacity_factor, out=None,
                          f=None, p=None, out_dtype=None, workspace=None):
    """The layer with expert-choice routing: each expert takes its C tokens with the
    largest router probability.  Returns (y, f, p)."""
    dev = x.device
    desc = desc_for(x, W_router, W_gate, k, capacity_factor, out_dtype)
    T, d = x.shape
    E = W_router.shape[0]
    G, F, _ = W_gate.shape
    for t, n, shp in ((x, "x", (T, d)), (W_router, "W_router", (E, d)),
                      (W_gate, "W_gate", (G, F, d)), (W_up, "W_up", (G, F, d)),
                      (W_down, "W_down", (G, d, F))):
        _require(t, n, dev, x.dtype, shp)
    odt = out_dtype or x.dtype
    out = torch.empty(T, d, dtype=odt, device=dev) if out is None else out
    f = torch.empty(E, dtype=torch.float32, device=dev) if f is None else f
    p = torch.empty(E, dtype=torch.float32, device=dev) if p is None else p
    _require(out, "out", dev, odt, (T, d))
    ws = _ws_ec(desc, dev, workspace)
    st = lib().moe_forward_expert_choice(ctypes.byref(desc), _ptr(x), _ptr(W_router),
                                         _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(out),
                                         _ptr(f), _ptr(p), _ptr(ws), ws.numel(), _stream(dev))
    _check("moe_forward_expert_choice", st)
    return out, f, p


def route_expert_choice(x, W_router, k, capacity_factor, workspace=None):
    """Router probabilities and the expert-choice selection.  Returns (probs [T, E],
    offsets [E+1], perm_src [E C], slot [T, E], f [E], p [E])."""
    dev = x.device
    T, d = x.shape
    E = W_router.shape[0]
    desc = make_desc(T, d, E, 64, k, 0, capacity_factor, x.dtype)
    _require(x, "x", dev)
    _require(W_router, "W_router", dev, x.dtype, (E, d))
    C = capacity_expert_choice(desc)
    if C < 0:
        _check("moe_capacity_expert_choice", validate(desc) or 2)
    probs = torch.empty(T, E, dtype=torch.float32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(E * C, 1), dtype=torch.int32, device=dev)
    slot = torch.empty(T, E, dtype=torch.int32, device=dev)
    f = torch.empty(E, dtype=torch.float32, device=dev)
    p = torch.empty(E, dtype=torch.float32, device=dev)
    ws = _ws_ec(desc, dev, workspace)
    st = lib().moe_route_expert_choice(ctypes.byref(desc), _ptr(x), _ptr(W_router), _ptr(probs),
                                       _ptr(offsets), _ptr(perm), _ptr(slot), _ptr(f), _ptr(p),
                                       _ptr(ws), ws.numel(), _stream(dev))
    _check("moe_route_expert_choice", st)
    return probs, offsets, perm[:E * C], slot, f, p


def combine_expert_choice(Yp, slot, probs, d, k, capacity_factor, n_shared=0,
                          out_dtype=torch.float32):
    """out[t] = sum_e probs[t, e] Yp[slot[t, e]] over the experts that took t (+ shared)."""
    dev = Yp.device
    T, E = slot.shape
    desc = make_desc(T, d, E, 64, k, n_shared, capacity_factor, torch.bfloat16, out_dtype)
    out = torch.empty(T, d, dtype=out_dtype, device=dev)
    _require(Yp, "Yp", dev, torch.float32)
    _require(slot, "slot", dev, torch.int32, (T, E))
    _require(probs, "probs", dev, torch.float32, (T, E))
    st = lib().moe_combine_expert_choice(ctypes.byref(desc), _ptr(Yp), _ptr(slot), _ptr(probs),
                                         _ptr(out), _stream(dev))
    _check("moe_combine_expert_choice", st)
    return out


# ----------------------------------------------------------------------------- next best
def forward_next_best(x, W_router, router_bias, W_gate, W_up, W_down, k, capacity_factor,
                      out=None, f=None, p=None, out_dtype=None, workspace=None):
    """The layer with capacity overflow handed to each token's next-best experts instead
    of dropped.  Returns (y, f, p)."""
    dev = x.device
    desc = desc_for(x, W_router, W_gate, k, capacity_factor, out_dtype)
    T, d = x.shape
    E = W_router.shape[0]
    G, F, _ = W_gate.shape
    for t, n, shp in ((x, "x", (T, d)), (W_router, "W_router", (E, d)),
                      (W_gate, "W_gate", (G, F, d)), (W_up, "W_up", (G, F, d)),
                      (W_down, "W_down", (G, d, F))):
        _require(t, n, dev, x.dtype, shp)
    _require(router_bias, "router_bias", dev, torch.float32, (E,))
    odt = out_dtype or x.dtype
    out = torch.empty(T, d, dtype=odt, device=dev) if out is None else out
    f = torch.empty(E, dtype=torch.float32, device=dev) if f is None else f
    p = torch.empty(E, dtype=torch.float32, device=dev) if p is None else p
    _require(out, "out", dev, odt, (T, d))
    ws = _ws(desc, dev, workspace)
    st = lib().moe_forward_next_best(ctypes.byref(desc), _ptr(x), _ptr(W_router),
                                     _ptr(router_bias), _ptr(W_gate), _ptr(W_up), _ptr(W_down),
                                     _ptr(out), _ptr(f), _ptr(p), _ptr(ws), ws.numel(),
                                     _stream(dev))
    _check("moe_forward_next_best", st)
    return out, f, p


def route_next_best(x, W_router, router_bias, k, workspace=None):
    """Router + top-k + the next-best candidates.  Returns (topk_idx, topk_w, cand, f, p)."""
    dev = x.device
    T, d = x.shape
    E = W_router.shape[0]
    desc = make_desc(T, d, E, 64, k, 0, 0.0, x.dtype)
    _require(x, "x", dev)
    _require(W_router, "W_router", dev, x.dtype, (E, d))
    _require(router_bias, "router_bias", dev, torch.float32, (E,))
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    cand = torch.empty(T, k, dtype=torch.int32, device=dev)
    f = torch.empty(E, dtype=torch.float32, device=dev)
    p = torch.empty(E, dtype=torch.float32, device=dev)
    ws = _ws(desc, dev, workspace)
    st = lib().moe_route_next_best(ctypes.byref(desc), _ptr(x), _ptr(W_router), _ptr(router_bias),
                                   _ptr(idx), _ptr(w), _ptr(cand), _ptr(f), _ptr(p), _ptr(ws),
                                   ws.numel(), _stream(dev))
    _check("moe_route_next_best", st)
    return idx, w, cand, f, p


def dispatch_next_best(topk_idx, cand, n_experts, capacity_factor, workspace=None):
    """Dispatch with the capacity overflow offered to the candidates.  Returns (counts,
    offsets, perm_src, slot_pos)."""
    dev = topk_idx.device
    T, k = topk_idx.shape
    E = int(n_experts)
    desc = make_desc(T, 64, E, 64, k, 0, capacity_factor, torch.bfloat16)
    _require(topk_idx, "topk_idx", dev, torch.int32, (T, k))
    _require(cand, "cand", dev, torch.int32, (T, k))
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    slot = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws = _ws(desc, dev, workspace)
    st = lib().moe_dispatch_next_best(ctypes.byref(desc), _ptr(topk_idx), _ptr(cand), _ptr(counts),
                                      _ptr(offsets), _ptr(perm), _ptr(slot), _ptr(ws), ws.numel(),
                                      _stream(dev))
    _check("moe_dispatch_next_best", st)
    return counts, offsets, perm, slot
