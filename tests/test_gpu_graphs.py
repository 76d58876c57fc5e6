"""The layer under HIP graph capture: the library allocates nothing, synchronises nothing
and clears its work counters with kernels, so a captured forward pass replays correctly.
Each replay is checked bit for bit against the eager result, with eager work of the
program's own between the replays."""
import pytest
import torch

import gen
import sparse_mixture_experts_24_amd as moe
from gen import Workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

CASES = {
    "decode": gen.workload("mixtral_decode").replace(T=16, d=256, F=512),
    "prefill_skewed": gen.workload("mixtral_prefill").replace(T=600, d=256, F=320),
    "capacity_next_best": Workload("capacity_next_best", T=500, d=128, E=16, k=2, F=128,
                                   capacity_factor=1.0, routing="next_best", bias_range=0.1),
    "expert_choice": Workload("expert_choice", T=400, d=128, E=8, k=2, F=192, n_shared=1,
                              capacity_factor=1.0, routing="expert"),
}


def layer_call(wl, d, out, f, p, ws):
    args = (d["x"], d["W_router"])
    experts = (d["W_gate"], d["W_up"], d["W_down"], wl.k, wl.capacity_factor)
    if wl.routing == "expert":
        return lambda: moe.forward_expert_choice(*args, *experts, out=out, f=f, p=p,
                                                 workspace=ws)
    fn = moe.forward_next_best if wl.routing == "next_best" else moe.forward
    return lambda: fn(*args, d["router_bias"], *experts, out=out, f=f, p=p, workspace=ws)


@pytest.mark.parametrize("name", sorted(CASES))
def test_captured_forward_replays_bit_exact(name):
    wl = CASES[name]
    d = {k: (None if v is None else v.to(DEV)) for k, v in gen.make_inputs(wl).items()}
    desc = moe.desc_for(d["x"], d["W_router"], d["W_gate"], wl.k, wl.capacity_factor)
    ws = (moe.alloc_workspace_expert_choice(desc, DEV) if wl.routing == "expert"
          else moe.alloc_workspace(desc, DEV))
    out = torch.empty(wl.T, wl.d, dtype=d["x"].dtype, device=DEV)
    f = torch.empty(wl.E, dtype=torch.float32, device=DEV)
    p = torch.empty(wl.E, dtype=torch.float32, device=DEV)
    call = layer_call(wl, d, out, f, p, ws)
    call()
    torch.cuda.synchronize()
    ref = [out.clone(), f.clone(), p.clone()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        out.zero_()
        f.zero_()
        p.zero_()
        junk = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out, ref[0]), f"{name}: replay {rep} output differs"
        assert torch.equal(f, ref[1]) and torch.equal(p, ref[2])
