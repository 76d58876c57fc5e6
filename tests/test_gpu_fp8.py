"""GPU parity of the layer with 8-bit expert weights (e4m3 codes, one float32 scale per
output row) against the oracle, which decodes the codes from the format definition and
dequantises them exactly.  Same rules as the bf16 layer: routing bit-exact except near
ties, f and P within 1e-5, y within max|dy| <= 2e-2 max|y_ref| and 5e-2 per element above
1e-3 max|y_ref| (elements past that explained by validated bf16 roundings of h, as at full
size); the stage test bounds every bf16 rounding of h as for bf16 weights.
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
    # every group small: streaming tiles (128-column down tiles for the few-tile launch)
    "decode": gen.workload("mixtral_decode_fp8").replace(T=5, d=256, F=512),
    # large skewed groups: 256-row tiles with 64/128/256-row remainders, dynamic order
    "prefill_skewed": gen.workload("mixtral_prefill").replace(T=700, d=256, F=320,
                                                              weights="fp8"),
    # capacity-limited top-1, Zipf-skewed: big and streaming tiles in one launch
    "switch_capacity": gen.workload("switch_capacity_fp8").replace(
        T=1000, d=128, E=16, F=256, row_scales=tuple(np.linspace(2.5, 0.7, 16).round(4))),
    # shared expert + selection bias, many small groups
    "fine_shared_bias": gen.workload("fine_grained_shared").replace(T=300, d=192, E=40, F=128,
                                                                    weights="fp8"),
    "one_token": Workload("one_token", T=1, d=128, E=8, k=2, F=192, n_shared=1, weights="fp8"),
    # the 8-wave kernel with 8-bit weights: skewed groups of all tile kinds, a 384-wide down
    # GEMM (128-column tail), h columns not a multiple of 128
    "w8_mixed_groups": Workload("w8_mixed_groups", T=900, d=384, E=12, k=2, F=448, n_shared=1,
                                row_scales=tuple(np.linspace(2.4, 0.5, 12).round(4)),
                                weights="fp8"),
    # 32 tokens, several streamed tiles per block in both GEMMs, shared expert
    "stream_many_tiles": Workload("stream_many_tiles", T=32, d=1536, E=32, k=4, F=1536,
                                  n_shared=1, bias_range=0.05, weights="fp8"),
}


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    name = request.param
    print(f"\n[fp8 case] {name}", flush=True)
    wl = CASES[name]
    inp = gen.make_inputs(wl)
    ref = oracle.forward(inp, wl.k, wl.capacity_factor, wl.n_shared, h_bf16=True)
    return name, wl, inp, to_dev(inp, DEV), ref


def _dispatch_tensors(ref):
    d = ref["dispatch"]
    perm = (torch.from_numpy(d["perm_src"]).to(DEV) if d["perm_src"].size
            else torch.zeros(1, dtype=torch.int32, device=DEV))
    return d, perm, torch.from_numpy(d["offsets"]).to(DEV)


def test_fp8_stage_gemms(case):
    """Gate/up and down on the oracle's dispatch: every h is a bf16 rounding of the exact
    h within its fp32 error bound, and Yp equals the oracle's o up to those roundings."""
    name, wl, inp, dinp, ref = case
    d, perm, offs = _dispatch_tensors(ref)
    H = moe.experts_gate_up_fp8(dinp["x"], perm, offs, dinp["Wq_gate"], dinp["Wq_up"],
                                dinp["s_gate"], dinp["s_up"], wl.k, wl.E)
    Yp = moe.experts_down_fp8(H, offs, dinp["Wq_down"], dinp["s_down"], wl.T, wl.k, wl.E)
    torch.cuda.synchronize()
    H, Yp = H.float().cpu().numpy(), Yp.cpu().numpy()
    x = np32(inp["x"])
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
        Wg, Wu, Wd = oracle.expert_weights(inp, e)
        o, parts = oracle.expert_ffn(x[tok], Wg, Wu, Wd, True, return_h=True)
        flips += check_h_and_down(H[lo:hi], parts, x[tok], Wg, Wu, Wd, Yp[lo:hi], o,
                                  f"{name} expert {e}")
    print(f"[{name}] bf16 h roundings on the other side of a midpoint: {flips}")


def test_fp8_stage_dynamic_tiles_match_static(case):
    name, wl, inp, dinp, ref = case
    d, perm, offs = _dispatch_tensors(ref)
    desc = moe.make_desc(wl.T, wl.d, wl.E, wl.F, wl.k, wl.n_shared, 0.0, dinp["x"].dtype)
    ws = moe.alloc_workspace(desc, DEV)
    args = (dinp["x"], perm, offs, dinp["Wq_gate"], dinp["Wq_up"], dinp["s_gate"], dinp["s_up"],
            wl.k, wl.E)
    H0 = moe.experts_gate_up_fp8(*args)
    Y0 = moe.experts_down_fp8(H0, offs, dinp["Wq_down"], dinp["s_down"], wl.T, wl.k, wl.E)
    H1 = moe.experts_gate_up_fp8(*args, workspace=ws)
    Y1 = moe.experts_down_fp8(H1, offs, dinp["Wq_down"], dinp["s_down"], wl.T, wl.k, wl.E,
                              workspace=ws)
    torch.cuda.synchronize()
    rows = list(range(int(d["offsets"][-1])))
    if wl.n_shared:
        rows += list(range(wl.T * wl.k, wl.T * wl.k + wl.T))
    assert torch.equal(H1[rows], H0[rows]) and torch.equal(Y1[rows], Y0[rows])


@pytest.mark.parametrize("odt", ["f32", "native"])
def test_fp8_forward(case, odt):
    name, wl, inp, dinp, ref = case
    out_dtype = torch.float32 if odt == "f32" else wl.torch_dtype
    y, f, p = moe.forward_fp8(dinp["x"], dinp["W_router"], dinp["router_bias"], dinp["Wq_gate"],
                              dinp["Wq_up"], dinp["Wq_down"], dinp["s_gate"], dinp["s_up"],
                              dinp["s_down"], wl.k, wl.capacity_factor, out_dtype=out_dtype)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    r = ref["route"]
    if (r["margin"] < 1e-6).any():
        idx, w, _, _ = moe.route(dinp["x"], dinp["W_router"], dinp["router_bias"], wl.k)
        idx = idx.cpu().numpy()
        check_routing(idx, w.cpu().numpy(), r)
        ref = oracle.forward(inp, wl.k, wl.capacity_factor, wl.n_shared, h_bf16=True,
                             idx_override=idx)
    np.testing.assert_allclose(f.cpu().numpy(), ref["f"], atol=STAT_TOL, rtol=0)
    np.testing.assert_allclose(p.cpu().numpy(), ref["p"], atol=STAT_TOL, rtol=0)
    # Every output element under the output rule with the validated bf16-rounding allowance
    # for h; the staged kernels give the h the layer used and reproduce y bit for bit.
    idx, w, _, _ = moe.route(dinp["x"], dinp["W_router"], dinp["router_bias"], wl.k)
    _, offs_g, perm_g, slot_g = moe.dispatch(idx, wl.E, wl.capacity_factor)
    H = moe.experts_gate_up_fp8(dinp["x"], perm_g, offs_g, dinp["Wq_gate"], dinp["Wq_up"],
                                dinp["s_gate"], dinp["s_up"], wl.k, wl.E)
    Yp = moe.experts_down_fp8(H, offs_g, dinp["Wq_down"], dinp["s_down"], wl.T, wl.k, wl.E)
    y_staged = moe.combine(Yp, slot_g, w, wl.T, wl.d, wl.k, wl.n_shared, out_dtype=out_dtype,
                           n_experts=wl.E)
    torch.cuda.synchronize()
    assert np.array_equal(y_staged.float().cpu().numpy(), y), "staged path differs"
    idx = idx.cpu().numpy()
    d_gpu = oracle.dispatch(idx, wl.E, oracle.capacity(wl.T, wl.k, wl.E, wl.capacity_factor))
    assert np.array_equal(slot_g.cpu().numpy(), d_gpu["slot_pos"])
    groups = token_choice_groups(d_gpu["offsets"], d_gpu["perm_src"], wl.k, wl.E, wl.n_shared,
                                 wl.T)
    check_full_layer(y, inp, groups, wl.T, wl.d, oracle.renorm_weights(r["p"], idx),
                     d_gpu["slot_pos"], True, out_dtype == torch.bfloat16,
                     H.float().cpu().numpy(), wl.T * wl.k + wl.n_shared * wl.T,
                     wl.T * wl.k if wl.n_shared else None, f"{name}: fp8 y")


def test_fp8_batch_consistency():
    """A token's row does not depend on the rest of the batch (no capacity)."""
    wl = CASES["fine_shared_bias"]
    inp = to_dev(gen.make_inputs(wl), DEV)
    w8 = (inp["Wq_gate"], inp["Wq_up"], inp["Wq_down"], inp["s_gate"], inp["s_up"], inp["s_down"])
    full, _, _ = moe.forward_fp8(inp["x"], inp["W_router"], inp["router_bias"], *w8, wl.k)
    for sub in ([7], list(range(64))):
        y, _, _ = moe.forward_fp8(inp["x"][sub].contiguous(), inp["W_router"],
                                  inp["router_bias"], *w8, wl.k)
        assert torch.equal(y, full[sub])


def test_fp8_scales_enter_linearly():
    """Doubling every scale of the down weights doubles Yp exactly (a power of two), and
    doubling the up scales doubles H up to bf16 rounding of the same values."""
    wl = CASES["decode"]
    inp = gen.make_inputs(wl)
    dinp = to_dev(inp, DEV)
    ref = oracle.forward(inp, wl.k, 0.0, 0)
    d, perm, offs = _dispatch_tensors(ref)
    H = moe.experts_gate_up_fp8(dinp["x"], perm, offs, dinp["Wq_gate"], dinp["Wq_up"],
                                dinp["s_gate"], dinp["s_up"], wl.k, wl.E)
    Y1 = moe.experts_down_fp8(H, offs, dinp["Wq_down"], dinp["s_down"], wl.T, wl.k, wl.E)
    Y2 = moe.experts_down_fp8(H, offs, dinp["Wq_down"], dinp["s_down"] * 2, wl.T, wl.k, wl.E)
    H2 = moe.experts_gate_up_fp8(dinp["x"], perm, offs, dinp["Wq_gate"], dinp["Wq_up"],
                                 dinp["s_gate"], dinp["s_up"] * 2, wl.k, wl.E)
    torch.cuda.synchronize()
    n = int(d["offsets"][-1])
    assert torch.equal(Y2[:n], 2 * Y1[:n])
    assert torch.equal(H2[:n], (2 * H[:n].float()).to(torch.bfloat16))


def test_fp8_requires_scales_and_bf16():
    wl = CASES["one_token"]
    dinp = to_dev(gen.make_inputs(wl), DEV)
    with pytest.raises(moe.MoeError):   # a NULL scale array
        moe.forward_fp8(dinp["x"], dinp["W_router"], None, dinp["Wq_gate"], dinp["Wq_up"],
                        dinp["Wq_down"], None, dinp["s_up"], dinp["s_down"], wl.k)
    with pytest.raises(moe.MoeError):   # fp32 activations
        moe.forward_fp8(dinp["x"].float(), dinp["W_router"].float(), None, dinp["Wq_gate"],
                        dinp["Wq_up"], dinp["Wq_down"], dinp["s_gate"], dinp["s_up"],
                        dinp["s_down"], wl.k)
