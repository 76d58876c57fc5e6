"""Seeded synthetic inputs for the sparse MoE FFN layer.

This module only draws random tensors.  It holds none of the layer's arithmetic and is
the one piece of code that both the HIP path (tests, bench) and the CPU oracle use.

Every tensor is drawn on the CPU with ``torch.Generator`` in fixed chunks of 2**24
elements; chunk ``c`` of tensor ``tid`` uses its own seed derived from
``(seed, tid, c)``, so the values do not depend on the thread count.  Normal draws are
float32 ``randn`` times ``1/sqrt(fan_in)`` (fan_in = d_model for the router, gate and up
weights, d_ff for the down weights), then rounded to bfloat16 with round-to-nearest-even
(``Tensor.to(torch.bfloat16)``) for the bf16 workloads; the fp32 workload keeps float32.

Layouts (all row-major, ``nn.Linear``'s out x in convention for weights):
  x [T, d]; W_router [E, d]; router_bias [E] float32 or None;
  W_gate, W_up [E + S, F, d]; W_down [E + S, d, F]  (S = 1 appends the shared expert).

Workloads with 8-bit expert weights draw the same bf16 weights and store them as
``Wq_gate``, ``Wq_up``, ``Wq_down`` (uint8 e4m3 "fn" codes, same shapes) with one float32
scale per output row (``s_gate``, ``s_up`` [E + S, F]; ``s_down`` [E + S, d]): scale =
max |row| / 448, codes = the row divided by its scale, cast with ``torch.float8_e4m3fn``
(round to nearest even); the bf16 tensors are then dropped.  x and the router stay bf16.
"""
from __future__ import annotations

import dataclasses
import json
import math
import os
from concurrent.futures import ThreadPoolExecutor

import torch

_CHUNK = 1 << 24
_HERE = os.path.dirname(os.path.abspath(__file__))

with open(os.path.join(_HERE, "row_scales.json")) as _fh:
    _ROW_SCALES = json.load(_fh)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic MoE-layer workload: shapes, dtype and input structure."""

    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    n_shared: int = 0
    capacity_factor: float = 0.0      # <= 0: no capacity limit
    dtype: str = "bf16"               # "bf16" or "f32" for x and all weights
    bias_range: float = 0.0           # > 0: selection bias ~ U(-r, r)
    row_scales: tuple | None = None   # per-expert router row scale (load skew)
    weights: str = "same"             # "same" (as dtype) or "fp8": e4m3 expert weights
    routing: str = "token"            # "token" (top-k per token), "next_best" (top-k, capacity
                                      # overflow redirected) or "expert" (top-C per expert)
    recipe: str = ""

    def replace(self, **kw) -> "Workload":
        w = dataclasses.replace(self, **kw)
        if w.row_scales is not None and len(w.row_scales) != w.E:
            w = dataclasses.replace(w, row_scales=None)
        return w

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", T=64, d=128, E=8, k=2, F=256, dtype="f32",
        recipe="x~N(0,1); W_router,W_gate,W_up~N(0,1/d); W_down~N(0,1/F); fp32; "
               "no bias, no capacity"),
    "mixtral_prefill": Workload(
        "mixtral_prefill", T=4096, d=4096, E=8, k=2, F=14336,
        row_scales=tuple(_ROW_SCALES["mixtral_prefill"]["scales"]),
        recipe="x~N(0,1); weights N(0,1/fan_in) bf16; router row e scaled by "
               "1+beta*e/7 so top-2 loads are ~3:1"),
    "mixtral_decode": Workload(
        "mixtral_decode", T=16, d=4096, E=8, k=2, F=14336,
        recipe="x~N(0,1); weights N(0,1/fan_in) bf16; router logits ~N(0,1) (uniform)"),
    "fine_grained_shared": Workload(
        "fine_grained_shared", T=8192, d=7168, E=256, k=8, F=2048, n_shared=1,
        bias_range=0.1,
        recipe="x~N(0,1); weights N(0,1/fan_in) bf16; 1 shared expert (d_ff 2048); "
               "selection bias ~U(-0.1,0.1) fp32 added to the softmax probabilities"),
    "switch_capacity": Workload(
        "switch_capacity", T=16384, d=2048, E=64, k=1, F=8192, capacity_factor=1.25,
        row_scales=tuple(_ROW_SCALES["switch_capacity"]["scales"]),
        recipe="x~N(0,1); weights N(0,1/fan_in) bf16; router row scales calibrated so "
               "top-1 loads follow Zipf(1.1); capacity factor 1.25"),
}


WORKLOADS["mixtral_decode_fp8"] = WORKLOADS["mixtral_decode"].replace(
    name="mixtral_decode_fp8", weights="fp8",
    recipe=WORKLOADS["mixtral_decode"].recipe + "; expert weights e4m3 with per-row scales")
WORKLOADS["switch_capacity_fp8"] = WORKLOADS["switch_capacity"].replace(
    name="switch_capacity_fp8", weights="fp8",
    recipe=WORKLOADS["switch_capacity"].recipe + "; expert weights e4m3 with per-row scales")
# The Switch layer's inputs with the capacity overflow handed to the next-best expert.
WORKLOADS["switch_capacity_nb"] = WORKLOADS["switch_capacity"].replace(
    name="switch_capacity_nb", routing="next_best",
    recipe=WORKLOADS["switch_capacity"].recipe + "; overflow redirected to each token's "
    "next-best expert (one round)")
# The prefill layer's inputs (same seeds, same values) under expert-choice routing: each
# expert takes C = T k / E = 1024 tokens.
WORKLOADS["mixtral_prefill_ec"] = WORKLOADS["mixtral_prefill"].replace(
    name="mixtral_prefill_ec", capacity_factor=1.0, routing="expert",
    recipe=WORKLOADS["mixtral_prefill"].recipe + "; expert-choice routing, capacity factor 1 "
    "(C = 1024 tokens per expert)")


def _chunk_seed(seed: int, tid: int, chunk: int) -> int:
    return (seed * 1_000_003 + tid * 65_537 + chunk * 7 + 12_345) % (1 << 62)


def _fill(out_flat: torch.Tensor, seed: int, tid: int, kind: str, scale: float,
          pool: ThreadPoolExecutor) -> None:
    n = out_flat.numel()

    def work(c):
        s, e = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = torch.Generator().manual_seed(_chunk_seed(seed, tid, c))
        if kind == "normal":
            v = torch.randn(e - s, generator=g, dtype=torch.float32)
            v.mul_(scale)
        else:  # uniform on [-scale, scale)
            v = torch.rand(e - s, generator=g, dtype=torch.float32)
            v.mul_(2.0 * scale).sub_(scale)
        out_flat[s:e] = v.to(out_flat.dtype)

    list(pool.map(work, range((n + _CHUNK - 1) // _CHUNK)))


ALL_PARTS = ("x", "W_router", "router_bias", "W_gate", "W_up", "W_down")


def make_inputs(wl: Workload, seed: int = 0, threads: int | None = None,
                parts=ALL_PARTS) -> dict:
    """Draw the inputs of ``wl`` on the CPU.  Returns a dict of torch tensors.

    ``parts`` limits the draw to some tensors; each tensor has its own seed stream, so
    a partial draw gives the same values as the full one.
    """
    dt = wl.torch_dtype
    G = wl.E + wl.n_shared
    threads = threads or min(16, os.cpu_count() or 1)
    shapes = {
        "x": ((wl.T, wl.d), dt, 0, "normal", 1.0),
        "W_router": ((wl.E, wl.d), torch.float32, 1, "normal", 1.0 / math.sqrt(wl.d)),
        "W_gate": ((G, wl.F, wl.d), dt, 2, "normal", 1.0 / math.sqrt(wl.d)),
        "W_up": ((G, wl.F, wl.d), dt, 3, "normal", 1.0 / math.sqrt(wl.d)),
        "W_down": ((G, wl.d, wl.F), dt, 4, "normal", 1.0 / math.sqrt(wl.F)),
        "router_bias": ((wl.E,), torch.float32, 5, "uniform", wl.bias_range),
    }
    out = {"router_bias": None}
    with ThreadPoolExecutor(threads) as pool:
        for name in ALL_PARTS:
            if name not in parts or (name == "router_bias" and wl.bias_range <= 0):
                continue
            shape, dtype, tid, kind, scale = shapes[name]
            t = torch.empty(shape, dtype=dtype)
            _fill(t.view(-1), seed, tid, kind, scale, pool)
            out[name] = t
    if "W_router" in out:
        if wl.row_scales is not None:
            out["W_router"].mul_(torch.tensor(wl.row_scales, dtype=torch.float32)[:, None])
        out["W_router"] = out["W_router"].to(dt)
    if wl.weights == "fp8":
        for name in ("W_gate", "W_up", "W_down"):
            if name in out:
                q, sc = _to_e4m3_rows(out.pop(name))
                out["Wq_" + name[2:]], out["s_" + name[2:]] = q, sc
    return out


def _to_e4m3_rows(W: torch.Tensor):
    """Per-row 8-bit storage of W [G, N, K]: (codes uint8 [G, N, K], scales f32 [G, N])."""
    G, N, K = W.shape
    q = torch.empty((G, N, K), dtype=torch.uint8)
    sc = torch.empty((G, N), dtype=torch.float32)
    for g in range(G):
        w = W[g].to(torch.float32)
        amax = w.abs().amax(dim=1)
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        v = (w / s[:, None]).clamp_(-448.0, 448.0)
        q[g] = v.to(torch.float8_e4m3fn).view(torch.uint8)
        sc[g] = s
    return q, sc


def workload(name: str) -> Workload:
    return WORKLOADS[name]
