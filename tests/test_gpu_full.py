"""GPU parity at the full workload sizes, in the launch configuration the bench times
(MoELayer.__call__ -> moe_forward with a reused workspace).

The oracle routes and dispatches every token (cheap) and runs the experts for a sample
of output rows, one by one.  Routing is bit-exact outside near-ties, dispatch is
bit-exact under the oracle's routing, f and P agree to 1e-5, and the sampled rows of y
satisfy the output rule.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_mixture_experts_24_amd as moe
from parity import STAT_TOL, check_routing, check_y, np32, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

FULL = ["tiny_f32", "mixtral_decode", "mixtral_prefill", "switch_capacity", "fine_grained_shared"]


def sample_rows(T, n, slot_pos, k, seed=0):
    rng = np.random.default_rng(seed)
    rows = set([0, T - 1])
    rows.update(rng.choice(T, min(T, n), replace=False).tolist())
    sp = slot_pos.reshape(T, k)
    dropped = np.nonzero(np.all(sp < 0, axis=1))[0]
    if dropped.size:                      # include fully dropped tokens (output 0)
        rows.update(dropped[:4].tolist())
    return np.array(sorted(rows))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    wl = gen.workload(name)
    print(f"\n[full] {name}: generating", flush=True)
    inp = gen.make_inputs(wl)
    dinp = to_dev(inp, DEV)
    layer = moe.MoELayer(dinp["W_router"], dinp["W_gate"], dinp["W_up"], dinp["W_down"], wl.k,
                         wl.capacity_factor, router_bias=dinp["router_bias"])
    print(f"[full] {name}: forward", flush=True)
    y, f, p = layer(dinp["x"])
    idx, w, _, _ = moe.route(dinp["x"], dinp["W_router"], dinp["router_bias"], wl.k)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    idx = idx.cpu().numpy()

    print(f"[full] {name}: oracle routing", flush=True)
    r = oracle.route(np32(inp["x"]), np32(inp["W_router"]), wl.k, np32(inp["router_bias"]))
    near = check_routing(idx, w.cpu().numpy(), r)
    print(f"[full] {name}: {int(near.sum())} near-tied tokens", flush=True)
    f_ref, p_ref = oracle.aux_stats(r["p"], idx, wl.E)
    np.testing.assert_allclose(f.cpu().numpy(), f_ref, atol=STAT_TOL, rtol=0)
    np.testing.assert_allclose(p.cpu().numpy(), p_ref, atol=STAT_TOL, rtol=0)

    # dispatch under the oracle's routing: bit-exact
    C = oracle.capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    d_ref = oracle.dispatch(r["idx"], wl.E, C)
    counts, offsets, perm, slot = moe.dispatch(torch.from_numpy(r["idx"]).to(DEV), wl.E,
                                               wl.capacity_factor)
    torch.cuda.synchronize()
    N = int(d_ref["offsets"][-1])
    assert np.array_equal(counts.cpu().numpy(), d_ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), d_ref["offsets"])
    assert np.array_equal(perm.cpu().numpy()[:N], d_ref["perm_src"])
    assert np.array_equal(slot.cpu().numpy(), d_ref["slot_pos"])

    # sampled output rows, with the layer's own (validated) routing
    routing = dict(r, idx=idx, w=oracle.renorm_weights(r["p"], idx))
    d_gpu = oracle.dispatch(idx, wl.E, C)
    rows = sample_rows(wl.T, 16 if wl.T > 64 else wl.T, d_gpu["slot_pos"], wl.k)
    print(f"[full] {name}: oracle experts for {rows.size} rows", flush=True)
    y_ref = oracle.forward_rows(inp, rows, wl.k, wl.capacity_factor, wl.n_shared,
                                h_bf16=(wl.dtype == "bf16"), routing=routing, disp=d_gpu)
    check_y(y[rows], y_ref, f"{name}: sampled rows")
    del dinp, layer
    torch.cuda.empty_cache()
