"""GPU parity: every entry point of libmoe against the CPU oracle on the same seeded
inputs, at sizes the oracle finishes in seconds (several tiles, ragged tails, edge
cases).  The full-size workloads are in test_gpu_full.py.

Rules: routing indices, histograms, offsets and the permutation bit-exact (tokens whose
top-k margin is below 1e-6 may route either way; the dispatch test then feeds the
oracle's routing); f and P within 1e-5; outputs within max|dy| <= 2e-2 max|y_ref| and
per-element relative error <= 5e-2 where |y_ref| > 1e-3 max|y_ref|, the layer's outputs with
elements past that explained by validated bf16 roundings of h (the full-size rule).
"""
import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_mixture_experts_24_amd as moe
from gen import Workload
from parity import (STAT_TOL, check_full_layer, check_h_and_down, check_routing, check_y, np32,
                    to_dev, token_choice_groups)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

CASES = {
    "tiny_f32": gen.workload("tiny_f32"),
    "prefill_skewed": gen.workload("mixtral_prefill").replace(T=600, d=256, F=320),
    "decode": gen.workload("mixtral_decode").replace(T=5, d=256, F=512),
    "fine_shared_bias": gen.workload("fine_grained_shared").replace(T=300, d=192, E=40, F=128),
    "switch_capacity": gen.workload("switch_capacity").replace(
        T=1000, d=128, E=16, F=256, row_scales=tuple(np.linspace(2.5, 0.7, 16).round(4))),
    "wide_router_k16": Workload("wide_router_k16", T=200, d=128, E=300, k=16, F=64, bias_range=0.05),
    "mid_router": Workload("mid_router", T=700, d=320, E=64, k=6, F=192, n_shared=1),
    "single_expert": Workload("single_expert", T=70, d=64, E=1, k=1, F=64),
    "k_equals_E": Workload("k_equals_E", T=50, d=64, E=4, k=4, F=128),
    "tight_capacity": Workload("tight_capacity", T=90, d=64, E=6, k=2, F=64, capacity_factor=0.01),
    "one_token": Workload("one_token", T=1, d=128, E=8, k=2, F=128, n_shared=1),
    # one route block: the dispatch runs inside the route kernel, here with drops ...
    "decode_capacity": Workload("decode_capacity", T=12, d=128, E=8, k=2, F=128,
                                capacity_factor=0.5, row_scales=(2.0, 1.6, 1.3, 1.1, 1.0, 0.9,
                                                                 0.8, 0.7)),
    # ... and with k = 16 over 40 experts (160 assignments ranked in the block)
    "decode_k16": Workload("decode_k16", T=10, d=128, E=40, k=16, F=64, capacity_factor=1.0,
                           bias_range=0.05),
    # large groups with ragged remainders (64/128/256-row last tiles), dynamic tile order
    "ragged_large_groups": Workload("ragged_large_groups", T=1500, d=128, E=4, k=2, F=192,
                                    n_shared=1, bias_range=0.05),
    # large groups and a down GEMM 384 columns wide: with tile counters the launch's last
    # down tiles run as two 128-column halves (the second half of the 128-column tail tile
    # is empty), which must sum like the whole tiles
    "ragged_wide_down": Workload("ragged_wide_down", T=1200, d=384, E=4, k=2, F=192,
                                 bias_range=0.05),
    # the largest expert count and top-k the library takes (E 512, k 16), with a shared
    # expert and a capacity
    "max_experts_k16": Workload("max_experts_k16", T=64, d=128, E=512, k=16, F=64, n_shared=1,
                                capacity_factor=1.5, bias_range=0.02),
    # capacity factors whose float32 value sits just below (0.7) or above (0.3) a decimal
    # that makes cf k T / E an integer: C = 6 (one route block, fused dispatch) and 69
    "capacity_boundary_fused": Workload("capacity_boundary_fused", T=40, d=64, E=8, k=2, F=64,
                                        capacity_factor=0.7,
                                        row_scales=tuple(np.linspace(2.0, 0.8, 8).round(4))),
    "capacity_boundary": Workload("capacity_boundary", T=400, d=64, E=8, k=2, F=64,
                                  capacity_factor=0.7,
                                  row_scales=tuple(np.linspace(2.0, 0.8, 8).round(4))),
    "capacity_above_decimal": Workload("capacity_above_decimal", T=400, d=64, E=8, k=2, F=64,
                                       capacity_factor=0.3),
    # at most 32 tokens: every tile is a skinny one and each block streams several tiles
    # back to back (the next tile's first K steps load under the current one's last), in
    # both GEMMs: ~64 groups x 1024 columns; T sits at the 32-row limit
    "stream_many_tiles": Workload("stream_many_tiles", T=32, d=1024, E=64, k=8, F=1024,
                                  n_shared=1, bias_range=0.05),
    # streamed 64-column tiles with drops and uneven, partly empty groups
    "stream_capacity": Workload("stream_capacity", T=24, d=640, E=16, k=4, F=2048,
                                capacity_factor=0.75,
                                row_scales=tuple(np.linspace(2.2, 0.6, 16).round(4))),
    # the batch sizes from which the 8-wave kernel takes the gate/up (65) and the down (81)
    # GEMM; h columns not a multiple of 128 (a half-empty last n-tile), a 384-wide down GEMM
    # (a 128-column tail tile), a shared expert of exactly T rows
    "w8_threshold_T65": Workload("w8_threshold_T65", T=65, d=128, E=2, k=1, F=192, n_shared=1),
    "w8_threshold_T81": Workload("w8_threshold_T81", T=81, d=384, E=3, k=2, F=320, n_shared=1,
                                 bias_range=0.05),
    # skewed groups from a few rows to several 256-row tiles with 64/128/192-row remainders,
    # all in the 8-wave kernel (small groups as its 64-row tiles)
    "w8_mixed_groups": Workload("w8_mixed_groups", T=900, d=256, E=12, k=2, F=448,
                                row_scales=tuple(np.linspace(2.4, 0.5, 12).round(4))),
    "f32_shared_capacity": Workload("f32_shared_capacity", T=130, d=64, E=12, k=3, F=128,
                                    n_shared=1, capacity_factor=1.0, dtype="f32", bias_range=0.02),
}


def run_case(name, seed=0):
    wl = CASES[name]
    inp = gen.make_inputs(wl, seed=seed)
    ref = oracle.forward(inp, wl.k, wl.capacity_factor, wl.n_shared, h_bf16=(wl.dtype == "bf16"))
    return wl, inp, ref


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    name = request.param
    print(f"\n[case] {name}", flush=True)
    wl, inp, ref = run_case(name)
    return name, wl, inp, to_dev(inp, DEV), ref


def test_route(case):
    name, wl, inp, dinp, ref = case
    idx, w, f, p, gap = moe.route(dinp["x"], dinp["W_router"], dinp["router_bias"], wl.k,
                                  want_gap=True)
    torch.cuda.synchronize()
    idx, w, gap = idx.cpu().numpy(), w.cpu().numpy(), gap.cpu().numpy()
    check_routing(idx, w, ref["route"])
    # gap = s_(k) - s_(k+1) of the selection scores (+inf when k == E)
    srt = -np.sort(-ref["route"]["s"].astype(np.float64), axis=1)
    gap_ref = srt[:, wl.k - 1] - srt[:, wl.k] if wl.k < wl.E else np.full(wl.T, np.inf)
    if wl.k < wl.E:
        np.testing.assert_allclose(gap, gap_ref, rtol=0, atol=1e-5)
    else:
        assert np.all(np.isposinf(gap))
    f_ref, p_ref = oracle.aux_stats(ref["route"]["p"], idx, wl.E)   # f of the GPU's valid routing
    np.testing.assert_allclose(f.cpu().numpy(), f_ref, atol=STAT_TOL, rtol=0)
    np.testing.assert_allclose(p.cpu().numpy(), p_ref, atol=STAT_TOL, rtol=0)
    np.testing.assert_allclose(p.cpu().numpy(), ref["p"], atol=STAT_TOL, rtol=0)


def test_dispatch_forced_routing(case):
    name, wl, inp, dinp, ref = case
    idx = torch.from_numpy(ref["route"]["idx"]).to(DEV)
    counts, offsets, perm_src, slot_pos = moe.dispatch(idx, wl.E, wl.capacity_factor)
    torch.cuda.synchronize()
    d = ref["dispatch"]
    N = int(d["offsets"][-1])
    assert counts.cpu().numpy().tolist() == d["counts"].tolist()
    assert offsets.cpu().numpy().tolist() == d["offsets"].tolist()
    assert perm_src.cpu().numpy()[:N].tolist() == d["perm_src"].tolist()
    assert slot_pos.cpu().numpy().tolist() == d["slot_pos"].tolist()


def test_experts_forced_dispatch(case):
    name, wl, inp, dinp, ref = case
    d = ref["dispatch"]
    perm = torch.from_numpy(d["perm_src"]).to(DEV) if d["perm_src"].size else torch.zeros(1, dtype=torch.int32, device=DEV)
    offs = torch.from_numpy(d["offsets"]).to(DEV)
    Yp, H = moe.experts(dinp["x"], perm, offs, dinp["W_gate"], dinp["W_up"], dinp["W_down"],
                        wl.k, wl.E, want_h=True)
    torch.cuda.synchronize()
    Yp = Yp.cpu().numpy()
    H = H.float().cpu().numpy()
    x = np32(inp["x"])
    hb = wl.dtype == "bf16"
    groups = [(e, int(d["offsets"][e]), int(d["offsets"][e + 1]),
               d["perm_src"][int(d["offsets"][e]):int(d["offsets"][e + 1])] // wl.k)
              for e in range(wl.E)]
    if wl.n_shared:
        r0 = wl.T * wl.k
        groups.append((wl.E, r0, r0 + wl.T, np.arange(wl.T)))
    flips = 0
    for e, lo, hi, tok in groups:
        if hi == lo:
            continue
        Wg, Wu, Wd = np32(inp["W_gate"][e]), np32(inp["W_up"][e]), np32(inp["W_down"][e])
        o, parts = oracle.expert_ffn(x[tok], Wg, Wu, Wd, hb, return_h=True)
        if hb:
            flips += check_h_and_down(H[lo:hi], parts, x[tok], Wg, Wu, Wd, Yp[lo:hi], o,
                                      f"{name} expert {e}")
        else:
            np.testing.assert_allclose(H[lo:hi], parts["h"], rtol=1e-4, atol=1e-5)
            check_y(Yp[lo:hi], o, f"{name} expert {e}")
    print(f"[{name}] bf16 h roundings on the other side of a midpoint: {flips}")


def test_combine_forced_inputs(case):
    name, wl, inp, dinp, ref = case
    d = ref["dispatch"]
    rng = np.random.default_rng(5)
    rows = wl.T * wl.k + wl.n_shared * wl.T
    Y = rng.standard_normal((max(rows, 1), wl.d)).astype(np.float32)
    shared = Y[wl.T * wl.k:wl.T * wl.k + wl.T] if wl.n_shared else None
    y_ref = oracle.combine(wl.T, wl.d, ref["route"]["w"], d["slot_pos"], Y, shared)
    for odt in (torch.float32, torch.bfloat16):
        y = moe.combine(torch.from_numpy(Y).to(DEV), torch.from_numpy(d["slot_pos"]).to(DEV),
                        torch.from_numpy(ref["route"]["w"]).to(DEV), wl.T, wl.d, wl.k,
                        wl.n_shared, out_dtype=odt, n_experts=wl.E)
        torch.cuda.synchronize()
        y = y.float().cpu().numpy()
        if odt == torch.float32:
            np.testing.assert_allclose(y, y_ref, rtol=1e-5, atol=1e-6)
        else:
            check_y(y, y_ref, f"{name}: combine bf16")


@pytest.mark.parametrize("odt", ["f32", "native"])
def test_forward(case, odt):
    name, wl, inp, dinp, ref = case
    out_dtype = torch.float32 if odt == "f32" else wl.torch_dtype
    y, f, p = moe.forward(dinp["x"], dinp["W_router"], dinp["router_bias"], dinp["W_gate"],
                          dinp["W_up"], dinp["W_down"], wl.k, wl.capacity_factor,
                          out_dtype=out_dtype)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    r = ref["route"]
    near = r["margin"] < 1e-6
    if near.any():
        # the layer's routing of near-tied tokens is its own: recompute the reference
        # with the GPU's (validated) routing
        idx, w, _, _ = moe.route(dinp["x"], dinp["W_router"], dinp["router_bias"], wl.k)
        idx = idx.cpu().numpy()
        check_routing(idx, w.cpu().numpy(), r)
        ref = oracle.forward(inp, wl.k, wl.capacity_factor, wl.n_shared,
                             h_bf16=(wl.dtype == "bf16"), idx_override=idx)
    np.testing.assert_allclose(f.cpu().numpy(), ref["f"], atol=STAT_TOL, rtol=0)
    np.testing.assert_allclose(p.cpu().numpy(), ref["p"], atol=STAT_TOL, rtol=0)
    # Every output element under the output rule, with the validated bf16-rounding allowance
    # for h (as at full size): the same kernels run stage by stage give the h the layer used
    # and must reproduce y bit for bit.
    idx, w, _, _ = moe.route(dinp["x"], dinp["W_router"], dinp["router_bias"], wl.k)
    _, offs_g, perm_g, slot_g = moe.dispatch(idx, wl.E, wl.capacity_factor)
    Yp, H = moe.experts(dinp["x"], perm_g, offs_g, dinp["W_gate"], dinp["W_up"], dinp["W_down"],
                        wl.k, wl.E, want_h=True, capacity_factor=wl.capacity_factor)
    y_staged = moe.combine(Yp, slot_g, w, wl.T, wl.d, wl.k, wl.n_shared, out_dtype=out_dtype,
                           n_experts=wl.E)
    torch.cuda.synchronize()
    assert np.array_equal(y_staged.float().cpu().numpy(), y), "staged path differs"
    idx = idx.cpu().numpy()
    C = oracle.capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    d_gpu = oracle.dispatch(idx, wl.E, C)
    assert np.array_equal(slot_g.cpu().numpy(), d_gpu["slot_pos"])
    groups = token_choice_groups(d_gpu["offsets"], d_gpu["perm_src"], wl.k, wl.E, wl.n_shared,
                                 wl.T)
    hb = wl.dtype == "bf16"
    check_full_layer(y, inp, groups, wl.T, wl.d, oracle.renorm_weights(r["p"], idx),
                     d_gpu["slot_pos"], hb, out_dtype == torch.bfloat16,
                     H.float().cpu().numpy() if hb else None, wl.T * wl.k + wl.n_shared * wl.T,
                     wl.T * wl.k if wl.n_shared else None, f"{name}: y")


def test_forward_is_deterministic(case):
    name, wl, inp, dinp, ref = case
    args = (dinp["x"], dinp["W_router"], dinp["router_bias"], dinp["W_gate"], dinp["W_up"],
            dinp["W_down"], wl.k, wl.capacity_factor)
    a = [t.clone() for t in moe.forward(*args)]
    b = moe.forward(*args)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("name", ["fine_shared_bias", "ragged_wide_down", "prefill_skewed"])
def test_batch_consistency(name):
    """Without a capacity, a token's output does not depend on the rest of the batch:
    batches of 1, 32 and 64 give bit-identical rows ("Mixture-of-experts in practice",
    inference-stability section, batch-consistency check).  The larger cases run the
    full batch with 256-row tiles (the down GEMM with 192-row ones where they fill its
    rounds better), the dynamic tile order and the down GEMM's column halves, the
    sub-batches with 64-row and skinny tiles."""
    wl = CASES[name]
    inp = to_dev(gen.make_inputs(wl), DEV)
    args = (inp["router_bias"], inp["W_gate"], inp["W_up"], inp["W_down"], wl.k, 0.0)
    full, _, _ = moe.forward(inp["x"], inp["W_router"], *args)
    for sub in ([7], list(range(5, 37)), list(range(64)), list(range(100, 300, 3))):
        y, _, _ = moe.forward(inp["x"][sub].contiguous(), inp["W_router"], *args)
        assert torch.equal(y, full[sub])


def test_empty_batch():
    wl = Workload("empty", T=0, d=128, E=8, k=2, F=128, n_shared=1)
    inp = to_dev(gen.make_inputs(wl), DEV)
    y, f, p = moe.forward(inp["x"], inp["W_router"], None, inp["W_gate"], inp["W_up"],
                          inp["W_down"], wl.k, 1.25)
    torch.cuda.synchronize()
    assert y.shape == (0, 128)
    assert torch.all(f == 0) and torch.all(p == 0)


def test_stage_gemms_dynamic_tiles_match_static(case):
    """With a workspace the stage GEMMs hand tiles out through counters; every tile is
    computed by the same code whichever CU takes it, so the outputs are bit-identical."""
    name, wl, inp, dinp, ref = case
    if wl.dtype != "bf16":
        pytest.skip("tile counters serve the bf16 kernels")
    d = ref["dispatch"]
    perm = torch.from_numpy(d["perm_src"]).to(DEV) if d["perm_src"].size else torch.zeros(1, dtype=torch.int32, device=DEV)
    offs = torch.from_numpy(d["offsets"]).to(DEV)
    desc = moe.make_desc(wl.T, wl.d, wl.E, wl.F, wl.k, wl.n_shared, 0.0, dinp["x"].dtype)
    ws = moe.alloc_workspace(desc, DEV)
    H0 = moe.experts_gate_up(dinp["x"], perm, offs, dinp["W_gate"], dinp["W_up"], wl.k, wl.E)
    Y0 = moe.experts_down(H0, offs, dinp["W_down"], wl.T, wl.k, wl.E)
    for _ in range(2):   # counters are reset by every call
        H1 = moe.experts_gate_up(dinp["x"], perm, offs, dinp["W_gate"], dinp["W_up"], wl.k, wl.E,
                                 workspace=ws)
        Y1 = moe.experts_down(H1, offs, dinp["W_down"], wl.T, wl.k, wl.E, workspace=ws)
        torch.cuda.synchronize()
        N = int(d["offsets"][-1]) + wl.n_shared * wl.T
        if wl.n_shared:
            rows = list(range(int(d["offsets"][-1]))) + list(range(wl.T * wl.k, wl.T * wl.k + wl.T))
        else:
            rows = list(range(N))
        assert torch.equal(H1[rows], H0[rows])
        assert torch.equal(Y1[rows], Y0[rows])


def test_workspace_reuse_and_smaller_second_call():
    wl = CASES["switch_capacity"]
    inp = gen.make_inputs(wl)
    dinp = to_dev(inp, DEV)
    layer = moe.MoELayer(dinp["W_router"], dinp["W_gate"], dinp["W_up"], dinp["W_down"], wl.k,
                         wl.capacity_factor)
    for T in (wl.T, 333):
        sub = {**inp, "x": inp["x"][:T]}
        ref = oracle.forward(sub, wl.k, wl.capacity_factor, 0, h_bf16=True)
        y, f, p = layer(dinp["x"][:T].contiguous())
        torch.cuda.synchronize()
        check_y(y.float().cpu().numpy(), ref["y"], f"T={T}")
        np.testing.assert_allclose(f.cpu().numpy(), ref["f"], atol=STAT_TOL, rtol=0)
