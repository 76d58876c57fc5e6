"""GPU parity of capacity overflow handed to the next-best expert ("Chapter 30", 30.5.2)
against the oracle: one redirect round, each assignment dropped by the capacity offered
to its token's next unused expert by selection score.

Routing and candidates bit-exact except near ties (1e-6; then they must be valid and the
oracle follows them); dispatch bit-exact under the oracle's routing; f and P within 1e-5;
y by the output rule.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_mixture_experts_24_amd as moe
from gen import Workload
from parity import (STAT_TOL, check_candidates, check_full_layer, check_routing, check_y, np32,
                    to_dev, token_choice_groups)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

CASES = {
    # top-1, Zipf-like skew: a third of the tokens overflow
    "switch_like": Workload("switch_like", T=1000, d=128, E=16, k=1, F=256, capacity_factor=1.25,
                            row_scales=tuple(np.linspace(2.5, 0.7, 16).round(4)),
                            routing="next_best"),
    # top-2 on the skewed prefill router
    "prefill_like": gen.workload("mixtral_prefill").replace(T=700, d=256, F=320,
                                                            capacity_factor=1.0,
                                                            routing="next_best"),
    # bias-dominated top-4 over 40 experts: a few experts overflow heavily
    "fine_bias_k4": Workload("fine_bias_k4", T=300, d=192, E=40, k=4, F=128, capacity_factor=1.0,
                             bias_range=0.1, routing="next_best"),
    # capacity at half the expected load: many offers are refused
    "tight": Workload("tight", T=200, d=128, E=8, k=2, F=128, capacity_factor=0.5,
                      row_scales=tuple(np.linspace(2.0, 0.8, 8).round(4)), routing="next_best"),
    # E < 2k: one candidate per token, the second slot's is -1
    "small_E": Workload("small_E", T=64, d=128, E=3, k=2, F=64, capacity_factor=1.0,
                        routing="next_best"),
    "shared": Workload("shared", T=300, d=128, E=16, k=2, F=192, n_shared=1, capacity_factor=1.0,
                       row_scales=tuple(np.linspace(2.0, 0.8, 16).round(4)), routing="next_best"),
    "f32": gen.workload("tiny_f32").replace(capacity_factor=1.0, routing="next_best"),
    # float32 cf just below 0.7: C = 69 at k T / E = 100
    "capacity_boundary": Workload("capacity_boundary", T=400, d=64, E=8, k=2, F=64,
                                  capacity_factor=0.7,
                                  row_scales=tuple(np.linspace(2.0, 0.8, 8).round(4)),
                                  routing="next_best"),
    # E 512, k 16: 16 candidates per token, most experts near their capacity
    "max_experts_k16": Workload("max_experts_k16", T=64, d=128, E=512, k=16, F=64,
                                capacity_factor=0.5, bias_range=0.05, routing="next_best"),
}


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    name = request.param
    print(f"\n[next best] {name}", flush=True)
    wl = CASES[name]
    inp = gen.make_inputs(wl)
    ref = oracle.forward(inp, wl.k, wl.capacity_factor, wl.n_shared,
                         h_bf16=wl.dtype == "bf16", next_best=True)
    return name, wl, inp, to_dev(inp, DEV), ref


def gpu_routing(wl, dinp, ref):
    idx, w, cand, f, p = moe.route_next_best(dinp["x"], dinp["W_router"], dinp["router_bias"],
                                             wl.k)
    torch.cuda.synchronize()
    idx, cand = idx.cpu().numpy(), cand.cpu().numpy()
    check_routing(idx, w.cpu().numpy(), ref["route"])
    near = check_candidates(cand, idx, ref["route"]["s"], wl.k)
    return idx, cand, near, f, p


def test_next_best_route(case):
    name, wl, inp, dinp, ref = case
    idx, cand, near, f, p = gpu_routing(wl, dinp, ref)
    np.testing.assert_allclose(f.cpu().numpy(), ref["f"], atol=STAT_TOL, rtol=0)
    np.testing.assert_allclose(p.cpu().numpy(), ref["p"], atol=STAT_TOL, rtol=0)
    print(f"[{name}] C = {ref['C']}, redirected {ref['dispatch']['redirected']}, "
          f"near-tied candidate lists {int(near.sum())}")


def test_next_best_dispatch_is_bit_exact(case):
    """Under the oracle's routing and candidates, offsets, rows and slots match exactly."""
    name, wl, inp, dinp, ref = case
    r, d = ref["route"], ref["dispatch"]
    counts, offsets, perm, slot = moe.dispatch_next_best(
        torch.from_numpy(r["idx"]).to(DEV), torch.from_numpy(r["cand"]).to(DEV), wl.E,
        wl.capacity_factor)
    torch.cuda.synchronize()
    N = int(d["offsets"][-1])
    assert np.array_equal(counts.cpu().numpy(), d["counts"])
    assert np.array_equal(offsets.cpu().numpy(), d["offsets"])
    assert np.array_equal(perm.cpu().numpy()[:N], d["perm_src"])
    assert np.array_equal(slot.cpu().numpy(), d["slot_pos"])


@pytest.mark.parametrize("odt", ["f32", "native"])
def test_next_best_forward(case, odt):
    name, wl, inp, dinp, ref = case
    out_dtype = torch.float32 if odt == "f32" else wl.torch_dtype
    y, f, p = moe.forward_next_best(dinp["x"], dinp["W_router"], dinp["router_bias"],
                                    dinp["W_gate"], dinp["W_up"], dinp["W_down"], wl.k,
                                    wl.capacity_factor, out_dtype=out_dtype)
    torch.cuda.synchronize()
    idx, cand, near, _, _ = gpu_routing(wl, dinp, ref)
    if near.any() or (ref["route"]["margin"] < 1e-6).any():
        ref = oracle.forward(inp, wl.k, wl.capacity_factor, wl.n_shared,
                             h_bf16=wl.dtype == "bf16", next_best=True, idx_override=idx,
                             cand_override=cand)
    check_y(y.float().cpu().numpy(), ref["y"], f"{name}: next-best y")
    np.testing.assert_allclose(f.cpu().numpy(), ref["f"], atol=STAT_TOL, rtol=0)
    np.testing.assert_allclose(p.cpu().numpy(), ref["p"], atol=STAT_TOL, rtol=0)


def test_next_best_keeps_more_than_dropping():
    """Same inputs: the redirect keeps every assignment the plain capacity cut keeps, and
    more; outputs of tokens with no dropped slot are unchanged."""
    wl = CASES["switch_like"]
    dinp = to_dev(gen.make_inputs(wl), DEV)
    args = (dinp["x"], dinp["W_router"], dinp["router_bias"], dinp["W_gate"], dinp["W_up"],
            dinp["W_down"], wl.k, wl.capacity_factor)
    y0, _, _ = moe.forward(*args)
    y1, _, _ = moe.forward_next_best(*args)
    idx, _, _, _ = moe.route(dinp["x"], dinp["W_router"], dinp["router_bias"], wl.k)
    _, offs0, _, slot0 = moe.dispatch(idx, wl.E, wl.capacity_factor)
    idx2, _, cand, _, _ = moe.route_next_best(dinp["x"], dinp["W_router"], dinp["router_bias"],
                                              wl.k)
    _, offs1, _, slot1 = moe.dispatch_next_best(idx2, cand, wl.E, wl.capacity_factor)
    torch.cuda.synchronize()
    assert int(offs1[-1]) > int(offs0[-1])
    s0, s1 = slot0.cpu().numpy() >= 0, slot1.cpu().numpy() >= 0
    assert np.all(s1[s0])
    whole = s0.reshape(wl.T, wl.k).all(axis=1)
    assert torch.equal(y0[torch.from_numpy(whole).to(DEV)], y1[torch.from_numpy(whole).to(DEV)])


def test_next_best_needs_a_capacity():
    wl = CASES["small_E"]
    dinp = to_dev(gen.make_inputs(wl), DEV)
    with pytest.raises(moe.MoeError):
        moe.forward_next_best(dinp["x"], dinp["W_router"], None, dinp["W_gate"], dinp["W_up"],
                              dinp["W_down"], wl.k, 0.0)


@pytest.mark.timeout(900)
def test_next_best_full_size():
    """The Switch-shaped layer (T 16384, d 2048, E 64, top-1, cf 1.25, Zipf loads) with the
    overflow redirected: routing, candidates, the whole dispatch, f, P and sampled rows."""
    wl = gen.workload("switch_capacity_nb")
    print("\n[full nb] generating", flush=True)
    inp = gen.make_inputs(wl)
    dinp = to_dev(inp, DEV)
    desc = moe.desc_for(dinp["x"], dinp["W_router"], dinp["W_gate"], wl.k, wl.capacity_factor)
    ws = moe.alloc_workspace(desc, DEV)
    print("[full nb] forward", flush=True)
    y, f, p = moe.forward_next_best(dinp["x"], dinp["W_router"], dinp["router_bias"],
                                    dinp["W_gate"], dinp["W_up"], dinp["W_down"], wl.k,
                                    wl.capacity_factor, workspace=ws)
    idx, w, cand, _, _ = moe.route_next_best(dinp["x"], dinp["W_router"], dinp["router_bias"],
                                             wl.k)
    torch.cuda.synchronize()
    print("[full nb] oracle routing", flush=True)
    r = oracle.route(np32(inp["x"]), np32(inp["W_router"]), wl.k, np32(inp["router_bias"]))
    idx_n, cand_n = idx.cpu().numpy(), cand.cpu().numpy()
    check_routing(idx_n, w.cpu().numpy(), r)
    check_candidates(cand_n, idx_n, r["s"], wl.k)
    f_ref, p_ref = oracle.aux_stats(r["p"], idx_n, wl.E)
    np.testing.assert_allclose(f.cpu().numpy(), f_ref, atol=STAT_TOL, rtol=0)
    np.testing.assert_allclose(p.cpu().numpy(), p_ref, atol=STAT_TOL, rtol=0)
    C = oracle.capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    d_ref = oracle.dispatch_next_best(idx_n, cand_n, wl.E, C)
    counts, offsets, perm, slot = moe.dispatch_next_best(idx, cand, wl.E, wl.capacity_factor)
    torch.cuda.synchronize()
    N = int(d_ref["offsets"][-1])
    assert np.array_equal(offsets.cpu().numpy(), d_ref["offsets"])
    assert np.array_equal(perm.cpu().numpy()[:N], d_ref["perm_src"])
    assert np.array_equal(slot.cpu().numpy(), d_ref["slot_pos"])
    print(f"[full nb] kept {N} of {wl.T * wl.k} ({d_ref['redirected']} redirected)", flush=True)
    Yp, H = moe.experts(dinp["x"], perm, offsets, dinp["W_gate"], dinp["W_up"], dinp["W_down"],
                        wl.k, wl.E, want_h=True)
    torch.cuda.synchronize()
    H = H.float().cpu().numpy()
    del Yp
    w_ref = oracle.renorm_weights(r["p"], idx_n)
    print(f"[full nb] oracle experts for all {wl.T} rows", flush=True)
    groups = token_choice_groups(d_ref["offsets"], d_ref["perm_src"], wl.k, wl.E, wl.n_shared,
                                 wl.T)
    nallow, flips = check_full_layer(y.float().cpu().numpy(), inp, groups, wl.T, wl.d, w_ref,
                                     d_ref["slot_pos"], True, True, H,
                                     wl.T * wl.k + wl.n_shared * wl.T,
                                     wl.T * wl.k if wl.n_shared else None,
                                     "full next-best: all rows")
    print(f"[full nb] {nallow} of {wl.T * wl.d} output elements needed the bf16-rounding "
          f"allowance; {flips} h values on the other side of a midpoint", flush=True)
