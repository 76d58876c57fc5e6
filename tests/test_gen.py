"""The seeded input generator: determinism, shapes, dtypes and the load structure of
each synthetic workload (checked with the oracle's router on the CPU)."""
import numpy as np
import pytest
import torch

import gen
import oracle


def test_deterministic_and_thread_independent():
    wl = gen.workload("tiny_f32")
    a = gen.make_inputs(wl, seed=3, threads=1)
    b = gen.make_inputs(wl, seed=3, threads=4)
    for key in gen.ALL_PARTS:
        if a[key] is None:
            assert b[key] is None
            continue
        assert torch.equal(a[key], b[key])
    c = gen.make_inputs(wl, seed=4)
    assert not torch.equal(a["x"], c["x"])
    part = gen.make_inputs(wl, seed=3, parts=("W_up",))
    assert torch.equal(part["W_up"], a["W_up"]) and "x" not in part


def test_shapes_dtypes_and_scales():
    wl = gen.workload("fine_grained_shared").replace(T=40, d=128, E=16, F=64)
    inp = gen.make_inputs(wl)
    assert inp["x"].shape == (40, 128) and inp["x"].dtype == torch.bfloat16
    assert inp["W_gate"].shape == (17, 64, 128) and inp["W_down"].shape == (17, 128, 64)
    assert inp["router_bias"].dtype == torch.float32
    b = inp["router_bias"]
    assert float(b.abs().max()) <= 0.1 and float(b.min()) < 0 < float(b.max())
    # N(0, 1/fan_in): sample std within a few percent
    assert abs(float(inp["W_up"].float().std()) * np.sqrt(128) - 1) < 0.05
    assert abs(float(inp["W_down"].float().std()) * np.sqrt(64) - 1) < 0.05


def _loads(name, T=None):
    wl = gen.workload(name)
    if T:
        wl = wl.replace(T=T)
    inp = gen.make_inputs(wl, parts=("x", "W_router", "router_bias"))
    r = oracle.route(oracle.moe_oracle._np(inp["x"]), oracle.moe_oracle._np(inp["W_router"]),
                     wl.k, oracle.moe_oracle._np(inp["router_bias"]))
    return np.bincount(r["idx"].ravel(), minlength=wl.E), wl


def test_prefill_loads_are_skewed_about_3_to_1():
    c, _ = _loads("mixtral_prefill")
    assert c.sum() == 4096 * 2
    assert 2.5 <= c.max() / c.min() <= 3.6, c


def test_switch_loads_follow_zipf_and_capacity_drops():
    c, wl = _loads("switch_capacity")
    C = oracle.capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    assert C == 320
    share = c / c.sum()
    pi = (np.arange(64) + 1.0) ** -1.1
    pi /= pi.sum()
    assert abs(share[0] - pi[0]) < 0.03
    kept = np.minimum(c, C).sum()
    assert 0.40 < 1 - kept / c.sum() < 0.60     # about half of the tokens overflow


def test_fp8_workload_stores_codes_and_row_scales():
    """8-bit workloads replace the expert weights by e4m3 codes and per-row scales; the
    largest code of each row decodes to 448 (scale = row max / 448), and the row
    decodes back to the bf16 weights within half a step: 2^-4 relative for normal codes,
    half the subnormal step (2^-10 of the scale) below them."""
    wl = gen.workload("mixtral_decode_fp8").replace(T=4, d=64, F=128)
    inp = gen.make_inputs(wl)
    ref = gen.make_inputs(wl.replace(weights="same"))
    assert "W_gate" not in inp and inp["Wq_gate"].dtype == torch.uint8
    assert inp["Wq_gate"].shape == (wl.E, wl.F, wl.d) and inp["s_gate"].shape == (wl.E, wl.F)
    assert inp["Wq_down"].shape == (wl.E, wl.d, wl.F) and inp["s_down"].shape == (wl.E, wl.d)
    for name in ("gate", "up", "down"):
        vals = inp["Wq_" + name].view(torch.float8_e4m3fn).to(torch.float32)
        assert torch.equal(vals.abs().amax(dim=2), torch.full(vals.shape[:2], 448.0))
        W = ref["W_" + name].to(torch.float32)
        deq = vals * inp["s_" + name][..., None]
        bound = torch.maximum(W.abs() * 2.0 ** -4, inp["s_" + name][..., None] * 2.0 ** -10)
        assert ((deq - W).abs() <= bound * (1 + 1e-6)).all()
    assert torch.equal(inp["x"], ref["x"]) and torch.equal(inp["W_router"], ref["W_router"])


def test_expert_choice_workload_shares_the_prefill_inputs():
    """The expert-choice prefill workload draws the prefill layer's tensors (same seeds)
    and only changes the routing: C = T k / E tokens per expert."""
    a, b = gen.workload("mixtral_prefill"), gen.workload("mixtral_prefill_ec")
    assert b.routing == "expert" and a.routing == "token"
    assert (b.T, b.d, b.E, b.k, b.F, b.row_scales) == (a.T, a.d, a.E, a.k, a.F, a.row_scales)
    assert oracle.expert_choice_capacity(b.T, b.k, b.E, b.capacity_factor) == 1024
    sa = gen.make_inputs(a.replace(T=32, d=64, F=64), parts=("x", "W_router"))
    sb = gen.make_inputs(b.replace(T=32, d=64, F=64), parts=("x", "W_router"))
    assert torch.equal(sa["x"], sb["x"]) and torch.equal(sa["W_router"], sb["W_router"])
