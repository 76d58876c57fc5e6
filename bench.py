"""Throughput of the MoE-layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload mixtral_prefill]

One step = one moe_forward over one batch of synthetic tokens (router, top-k, dispatch,
grouped SwiGLU experts, combine, f/P statistics), inputs resident in HBM.  Prints ONE
JSON line (stdout).  Besides the whole-layer rate it times each stage with HIP events on
the launch stream (staged entry points, same kernels) to report the dominant kernel
against its roofline, and times the CPU oracle on a bounded sample of the same batch.

The headline is the Mixtral-shaped prefill layer; with the default workload the same
line also carries timed records of the decode, fine-grained and Switch-shaped layers
("workloads"), each with its layer time, tokens/s and the dominant kernel's roof
fraction (--only: the named workload alone), and, as context for the roof fraction, the
vendor GEMM library timed on dense products of the headline's sizes ("dense_reference").
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec + % of bf16 MFMA peak (prefill) / % HBM BW (decode)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # fp32 vector
PEAK_HBM_GBS = 8000.0         # HBM3E
# Which roof bounds the dominant (gate/up) kernel for each workload.
BOUND = {"mixtral_prefill": "mfma", "fine_grained_shared": "mfma", "mixtral_decode": "hbm",
         "switch_capacity": "hbm", "tiny_f32": "alu", "mixtral_decode_fp8": "hbm",
         "switch_capacity_fp8": "hbm", "mixtral_prefill_ec": "mfma",
         "switch_capacity_nb": "hbm"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)



# Layers timed beside the headline in the default run (one GPU, one after the other).
SIDE_WORKLOADS = ("mixtral_decode", "fine_grained_shared", "switch_capacity", "mixtral_decode_fp8",
                  "switch_capacity_fp8")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--only", action="store_true",
                    help="time the named workload alone (no side workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="tokens in the oracle sample")
    ap.add_argument("--dense-reference", action="store_true",
                    help="time only the vendor GEMM on dense products of the named workload's "
                         "sizes (M = T k + S T kept rows, no capacity), no layer")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) into the traffic record of --workload; no GPU use")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.workload, *args.summarize_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this layer is built and timed on a single "
              "MI355X (no sharding, no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.dense_reference:
        import gen
        wl = gen.workload(args.workload)
        cfg = {"T": wl.T, "d_model": wl.d, "d_ff": wl.F, "n_shared": wl.n_shared}
        rec = {"config": cfg, "layer": {"kept_assignments": wl.T * wl.k}}
        print(json.dumps({"workload": wl.name, "dense_reference": dense_reference(rec, dev)}),
              flush=True)
        return
    rec, inp, wl = run_workload(args.workload, args.steps, args.warmup, dev)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = (cpu_baseline_ec if wl.routing == "expert" else cpu_baseline)(
            wl, inp, args.cpu_sample, rec["layer"]["flops"])
    del inp
    if not args.only and args.workload == "mixtral_prefill":
        rec["dense_reference"] = dense_reference(rec, dev)
        side = {}
        for name in SIDE_WORKLOADS:
            torch.cuda.empty_cache()
            r, inp, _ = run_workload(name, args.steps, args.warmup, dev)
            del inp
            side[name] = {key: r[key] for key in ("value", "unit", "ms_per_step", "dtype",
                                                  "config", "roofline", "layer")}
        rec["workloads"] = side
    print(json.dumps(rec), flush=True)

    if args.copy_calibration:
        # A plain streaming copy of known size (one elementwise dispatch that reads and
        # writes COPY_BYTES), for scaling the HBM byte counters.
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x {COPY_BYTES} bytes read and written")


def run_workload(name, steps, warmup, dev):
    """Times `steps` moe_forward calls of workload `name` (after `warmup`), then its stages;
    returns (record, host inputs, workload)."""
    import numpy as np
    import torch

    import gen
    import sparse_mixture_experts_24_amd as moe

    wl = gen.workload(name)
    args = argparse.Namespace(steps=steps, warmup=warmup)
    log(f"[bench] workload {wl.name}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} F={wl.F} "
        f"S={wl.n_shared} cf={wl.capacity_factor} dtype={wl.dtype}")
    t0 = time.time()
    inp = gen.make_inputs(wl, seed=0)
    dinp = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    torch.cuda.synchronize()
    log(f"[bench] inputs drawn and resident in HBM ({time.time() - t0:.1f}s)")

    T, d, E, k, F, S = wl.T, wl.d, wl.E, wl.k, wl.F, wl.n_shared
    fp8 = wl.weights == "fp8"     # e4m3 expert weights with per-row scales
    ec = wl.routing == "expert"   # expert-choice routing: each expert takes its top-C tokens
    nb = wl.routing == "next_best"   # capacity overflow handed to the next-best expert
    out_dtype = wl.torch_dtype
    desc = moe.make_desc(T, d, E, F, k, S, wl.capacity_factor, wl.torch_dtype, out_dtype)
    ws = moe.alloc_workspace_expert_choice(desc, dev) if ec else moe.alloc_workspace(desc, dev)
    out = torch.empty(T, d, dtype=out_dtype, device=dev)
    f = torch.empty(E, dtype=torch.float32, device=dev)
    p = torch.empty(E, dtype=torch.float32, device=dev)
    L = moe.lib()
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    dref = ctypes.byref(desc)
    if ec:
        fwd_fn = L.moe_forward_expert_choice
        fwd_args = (dref, P(dinp["x"]), P(dinp["W_router"]), P(dinp["W_gate"]),
                    P(dinp["W_up"]), P(dinp["W_down"]), P(out), P(f), P(p), P(ws), ws.numel(), sp)
    elif nb:
        fwd_fn = L.moe_forward_next_best
        fwd_args = (dref, P(dinp["x"]), P(dinp["W_router"]), P(dinp["router_bias"]),
                    P(dinp["W_gate"]), P(dinp["W_up"]), P(dinp["W_down"]), P(out), P(f), P(p),
                    P(ws), ws.numel(), sp)
    elif fp8:
        W8 = [P(dinp[n]) for n in ("Wq_gate", "Wq_up", "Wq_down", "s_gate", "s_up", "s_down")]
        fwd_fn = L.moe_forward_fp8
        fwd_args = (dref, P(dinp["x"]), P(dinp["W_router"]), P(dinp["router_bias"]), *W8,
                    P(out), P(f), P(p), P(ws), ws.numel(), sp)
    else:
        fwd_fn = L.moe_forward
        fwd_args = (dref, P(dinp["x"]), P(dinp["W_router"]), P(dinp["router_bias"]),
                    P(dinp["W_gate"]), P(dinp["W_up"]), P(dinp["W_down"]), P(out), P(f), P(p),
                    P(ws), ws.numel(), sp)

    def step():
        st = fwd_fn(*fwd_args)
        if st:
            raise moe.MoeError("moe_forward", st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] moe_forward: {ms:.4f} ms/step (events), wall {1e3 * wall / args.steps:.4f} ms/step")

    # ---- staged: the same kernels through the stage entry points, events between them
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    slot = torch.empty(T * k, dtype=torch.int32, device=dev)
    rows = T * k + S * T
    out2 = torch.empty_like(out)
    H = torch.empty(rows, F, dtype=wl.torch_dtype, device=dev)
    Yp = torch.empty(rows, d, dtype=torch.float32, device=dev)
    calls = [
        ("route", lambda: L.moe_route(dref, P(dinp["x"]), P(dinp["W_router"]),
                                      P(dinp["router_bias"]), P(idx), P(w), None, P(f), P(p), P(ws),
                                      ws.numel(), sp)),
        ("dispatch", lambda: L.moe_dispatch(dref, P(idx), P(counts), P(offsets), P(perm),
                                            P(slot), P(ws), ws.numel(), sp)),
        ("gate_up", (lambda: L.moe_experts_gate_up_fp8(
            dref, P(dinp["x"]), P(perm), P(offsets), P(dinp["Wq_gate"]), P(dinp["Wq_up"]),
            P(dinp["s_gate"]), P(dinp["s_up"]), P(H), P(ws), ws.numel(), sp)) if fp8 else
         (lambda: L.moe_experts_gate_up(dref, P(dinp["x"]), P(perm), P(offsets),
                                        P(dinp["W_gate"]), P(dinp["W_up"]), P(H), P(ws),
                                        ws.numel(), sp))),
        ("down", (lambda: L.moe_experts_down_fp8(
            dref, P(H), P(offsets), P(dinp["Wq_down"]), P(dinp["s_down"]), P(Yp), P(ws),
            ws.numel(), sp)) if fp8 else
         (lambda: L.moe_experts_down(dref, P(H), P(offsets), P(dinp["W_down"]), P(Yp), P(ws),
                                     ws.numel(), sp))),
        ("combine", lambda: L.moe_combine(dref, P(Yp), P(slot), P(w), P(out2), sp)),
    ]
    if ec:   # the expert-choice layer's own stages
        calls = expert_choice_stages(moe, L, desc, dinp, ws, out2, f, p, P, sp, dev)
        counts, offsets = calls.counts, calls.offsets
    if nb:   # route with the candidates, dispatch with the redirect round
        cand = torch.empty(T, k, dtype=torch.int32, device=dev)
        calls[0] = ("route", lambda: L.moe_route_next_best(
            dref, P(dinp["x"]), P(dinp["W_router"]), P(dinp["router_bias"]), P(idx), P(w),
            P(cand), P(f), P(p), P(ws), ws.numel(), sp))
        calls[1] = ("dispatch", lambda: L.moe_dispatch_next_best(
            dref, P(idx), P(cand), P(counts), P(offsets), P(perm), P(slot), P(ws), ws.numel(),
            sp))
    for _ in range(max(1, args.warmup)):
        for name, c in calls:
            if c():
                raise RuntimeError(f"staged {name} failed")
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
           for _ in range(args.steps)]
    for s in range(args.steps):
        evs[s][0].record(stream)
        for i, (name, c) in enumerate(calls):
            if c():
                raise RuntimeError(f"staged {name} failed")
            evs[s][i + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1])
                                     for s in range(args.steps)]))
                for i, (name, _) in enumerate(calls)}
    log("[bench] stages (ms): " + ", ".join(f"{n} {v:.4f}" for n, v in stage_ms.items()))
    # the staged kernels reproduce moe_forward bit for bit (0 expected)
    dmax = (out.float() - out2.float()).abs().max().item() if out.numel() else 0.0
    ymax = out.float().abs().max().item() if out.numel() else 0.0
    log(f"[bench] staged output vs moe_forward: max|diff| {dmax:.3e} (max|y| {ymax:.3e})")

    # ---- realised routing -> algorithmic work
    cnt = counts.cpu().numpy().astype(np.int64)
    offs = offsets.cpu().numpy().astype(np.int64)
    kept = np.diff(offs)
    N = int(offs[-1])
    touched = int(np.count_nonzero(kept)) + S
    esz = 2 if wl.dtype == "bf16" else 4            # activations, router
    wsz = 1 if fp8 else esz                         # expert weights (+ f32 row scales)
    flops_gate_up = 4.0 * d * F * (N + S * T)
    flops_down = 2.0 * d * F * (N + S * T)
    flops_layer = 2.0 * T * d * E + flops_gate_up + flops_down
    # gate/up algorithmic bytes: the touched experts' gate and up weights (+ row scales)
    # and the token rows; H is implementation traffic (written here, read by the down
    # GEMM) and is not counted
    w_gate_up_bytes = touched * 2.0 * F * (d * wsz + (4 if fp8 else 0))
    bytes_gate_up = w_gate_up_bytes + T * d * esz
    bytes_layer = (touched * (3.0 * F * d * wsz + (4.0 * (2 * F + d) if fp8 else 0.0))
                   + E * d * esz + T * d * esz + T * d * esz)
    log(f"[bench] counts per expert: {cnt.tolist() if E <= 64 else (cnt.min(), cnt.max())}; "
        f"kept N={N} of {T * k}; experts touched {touched}")

    gu_s = stage_ms["gate_up"] / 1e3
    bound = BOUND.get(wl.name, "mfma")
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": flops_gate_up / gu_s / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    elif bound == "hbm":
        roof = {"bound": "hbm", "achieved": bytes_gate_up / gu_s / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "alu", "achieved": flops_gate_up / gu_s / 1e12,
                "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(wl.name)
    roof["kernel"] = gate_up_kernel(wl) + (" (gate/up + SiLU*mul, e4m3 weights)" if fp8
                                           else " (gate/up + SiLU*mul)")
    roof["kernel_ms"] = stage_ms["gate_up"]
    roof["algorithmic_per_launch"] = flops_gate_up if bound != "hbm" else bytes_gate_up

    layer_s = ms / 1e3
    layer = {
        "tflops": flops_layer / layer_s / 1e12,
        "mfma_frac": flops_layer / layer_s / 1e12 / PEAK_BF16_TFLOPS,
        "gbs": bytes_layer / layer_s / 1e9,
        "hbm_frac": bytes_layer / layer_s / 1e9 / PEAK_HBM_GBS,
        "flops": flops_layer, "bytes": bytes_layer, "kept_assignments": N,
        "experts_touched": touched, "stage_ms": stage_ms,
    }

    rec = {
        "metric": METRIC, "value": T / layer_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded; shapes and load structure of the workload)",
        "config": {"workload": wl.name, "T": T, "d_model": d, "n_experts": E, "top_k": k,
                   "d_ff": F, "n_shared": S, "capacity_factor": wl.capacity_factor,
                   "selection_bias": wl.bias_range > 0, "out_dtype": str(out_dtype).split(".")[-1],
                   "expert_weights": "e4m3 + f32 per-row scale" if fp8 else wl.dtype,
                   "routing": "expert choice (top-C tokens per expert)" if ec
                              else "token choice, capacity overflow to the next-best expert"
                              if nb else "token choice (top-k experts per token)"},
        "roofline": roof,
        "layer": layer,
        "cpu_baseline": None,
    }
    log(f"[bench] {wl.name}: {T / layer_s:.4g} tokens/s, {ms:.4f} ms/step; gate/up "
        f"{roof['achieved']:.4g} {roof['unit']} = {roof['frac']:.3f} of peak")
    del dinp, ws, out, H, Yp, calls
    return rec, inp, wl



def dense_reference(rec, dev, steps=10):
    """Context for the roof fraction: the vendor GEMM library (torch.matmul on ROCm, i.e.
    hipBLASLt) on dense bf16 products of the headline layer's sizes, with M = the kept
    rows (no gather, no groups, no fused SiLU*mul): [N, d] x [d, 2F] for gate/up and
    [N, F] x [F, d] for down.  Same HIP-event timing as the stages."""
    import torch

    cfg = rec["config"]
    n = int(rec["layer"]["kept_assignments"]) + cfg["n_shared"] * cfg["T"]
    d, F = cfg["d_model"], cfg["d_ff"]
    out = {"library": "torch.matmul (hipBLASLt), bf16, dense"}
    g = torch.Generator(device=dev).manual_seed(0)
    for name, (m, kk, nn) in (("gate_up", (n, d, 2 * F)), ("down", (n, F, d))):
        a = torch.randn(m, kk, device=dev, dtype=torch.bfloat16, generator=g)
        b = torch.randn(kk, nn, device=dev, dtype=torch.bfloat16, generator=g)
        for _ in range(3):
            c = a @ b
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = 2.0 * m * kk * nn / (ms / 1e3) / 1e12
        out[name] = {"shape": f"{m}x{kk}x{nn}", "ms": ms, "tflops": tf,
                     "frac": tf / PEAK_BF16_TFLOPS}
        log(f"[bench] dense reference {name} {m}x{kk}x{nn}: {ms:.4f} ms, {tf:.1f} TFLOP/s")
        del a, b, c
    torch.cuda.empty_cache()
    return out


# ---- HBM traffic of the dominant kernel, from rocprofv3 counters
COPY_BYTES = 1 << 30
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
GEMM_SOURCES = [os.path.join(ROOT, "sparse_mixture_experts_24_amd", "csrc", f)
                for f in ("gemm.hip", "moe_internal.h")]


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the gate/up kernel from the committed counter record, or None
    when there is none or the kernel source changed since the counters were taken."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != gemm_source_hash():
        return None
    return rec["hbm_bytes_per_launch"]


def summarize_pmc(workload, fetch_csv, write_csv):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the gate/up kernel and of the 1 GiB copy,
    the copy's ratios known/counted as scale factors, written to profiles/."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
            vals[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: list(v.values()) for k, v in vals.items()}

    def pick(d, pred):
        names = [k for k in d if pred(k)]
        if not names:
            raise SystemExit(f"no matching kernel among {sorted(d)}")
        return statistics.median([v for k in names for v in d[k]])

    import gen
    gemm_name = gate_up_kernel(gen.workload(workload))
    is_gemm = lambda k: gemm_name in k
    is_copy = lambda k: "MulFunctor" in k
    f, w = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    gf, gw = pick(f, is_gemm), pick(w, is_gemm)
    cf, cw = pick(f, is_copy), pick(w, is_copy)
    sf, sw = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    rec = {"workload": workload, "kernel": gemm_name + " (gate/up + SiLU*mul)",
           "source_sha256": gemm_source_hash(),
           "fetch_kib_per_launch": gf, "write_kib_per_launch": gw,
           "copy_bytes": COPY_BYTES, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": sf, "write_scale": sw,
           "hbm_bytes_per_launch": gf * 1024.0 * sf + gw * 1024.0 * sw}
    out = os.path.join(TRAFFIC_DIR, f"traffic_{workload}.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def gate_up_kernel(wl):
    """The kernel that runs the gate/up GEMM of workload wl: batches of fewer than 65 tokens
    (no group can be large) take the 4-wave kernel, other bf16 layers the 8-wave one;
    float32 layers the FMA kernel."""
    if wl.dtype != "bf16":
        return "gemm_f32_kernel<true>"
    fp8 = "true" if wl.weights == "fp8" else "false"
    return (f"gemm_w8_kernel<true, {fp8}>" if wl.T >= 65
            else f"gemm_bf16_kernel<true, {fp8}>")


def host_info():
    """Threads the oracle's BLAS uses, the cores this process may run on, and the CPU model."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        blas = os.cpu_count()
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return int(blas), int(nproc), int(os.cpu_count() or 0), model


def timed_runs(fn, runs=3):
    """One untimed warm-up call, then the median wall time of `runs` calls."""
    import statistics
    fn()
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts), ts


def cpu_baseline(wl, inp, sample, layer_flops):
    """The oracle, as it stands, on the host cores: routing + dispatch of the whole batch
    plus the experts of an evenly spaced sample of tokens, scaled to the whole batch.
    Protocol: one warm-up, then the median of three runs of each part."""
    import numpy as np

    import oracle
    from oracle import moe_oracle as mo
    blas, nproc, ncpu, model = host_info()
    if not sample:
        per_tok = 6.0 * wl.d * wl.F * (wl.k + wl.n_shared)
        sample = int(max(8, min(wl.T, 2.0e12 / per_tok)))   # ~2-4 s of oracle work per run
    x = mo._np(inp["x"])
    Wr, b = mo._np(inp["W_router"]), mo._np(inp["router_bias"])
    C = oracle.capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    state = {}

    def route_part():
        r = oracle.route(x, Wr, wl.k, b)
        state["r"] = r
        state["disp"] = oracle.dispatch(r["idx"], wl.E, C)
        oracle.aux_stats(r["p"], r["idx"], wl.E)

    t_route, _ = timed_runs(route_part)
    rows = np.linspace(0, wl.T - 1, sample).astype(np.int64)
    t_exp, ts = timed_runs(lambda: oracle.forward_rows(
        inp, rows, wl.k, wl.capacity_factor, wl.n_shared, h_bf16=(wl.dtype == "bf16"),
        routing=state["r"], disp=state["disp"]))
    full = t_route + t_exp * wl.T / rows.size
    log(f"[bench] oracle: route+dispatch {t_route:.2f}s for {wl.T} tokens, experts "
        f"{t_exp:.2f}s (median of {[round(t, 2) for t in ts]}) for {rows.size} tokens -> "
        f"{full:.1f}s per batch; {blas} BLAS threads, nproc {nproc}, {model}")
    return {"value": wl.T / full, "unit": "tokens/s", "cores": blas, "kind": "oracle",
            "gflops": layer_flops / full / 1e9, "nproc": nproc, "cpu_count": ncpu,
            "cpu_model": model, "runs": "1 warm-up + median of 3",
            "sample": f"routing+dispatch of all {wl.T} tokens ({t_route:.2f}s) + experts of "
                      f"{rows.size} evenly spaced tokens ({t_exp:.2f}s), scaled to the batch"}


class _Stages(list):
    """(name, call) pairs plus the buffers the bench reads back afterwards."""


def expert_choice_stages(moe, L, desc, dinp, ws, out2, f, p, P, sp, dev):
    """The expert-choice layer's kernels through its stage entry points: route +
    selection, gate/up, down, combine.  The two GEMMs are the same launches as inside
    moe_forward_expert_choice, reached through the token-choice stage entry points with
    one row per routed (token, expert) pair: a description with T' = E*C tokens and k = 1,
    and x padded to E*C rows (the rows read are perm_src's, all below T)."""
    import torch
    T, d, E, F, k, S = desc.T, desc.d_model, desc.n_experts, desc.d_ff, desc.top_k, desc.n_shared
    if S:
        raise SystemExit("expert-choice stage timing covers layers without a shared expert")
    dt = dinp["x"].dtype
    C = moe.capacity_expert_choice(desc)
    probs = torch.empty(T, E, dtype=torch.float32, device=dev)
    slot = torch.empty(T, E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(E * C, dtype=torch.int32, device=dev)
    xpad = torch.zeros(E * C, d, dtype=dt, device=dev)
    xpad[:T] = dinp["x"]
    dpad = moe.make_desc(E * C, d, E, F, 1, 0, 0.0, dt, dt)
    wpad = moe.alloc_workspace(dpad, dev)
    H = torch.empty(E * C, F, dtype=dt, device=dev)
    Yp = torch.empty(E * C, d, dtype=torch.float32, device=dev)
    dref, pref = ctypes.byref(desc), ctypes.byref(dpad)
    st = _Stages([
        ("route", lambda: L.moe_route_expert_choice(
            dref, P(dinp["x"]), P(dinp["W_router"]), P(probs), P(offsets), P(perm), P(slot),
            P(f), P(p), P(ws), ws.numel(), sp)),
        ("gate_up", lambda: L.moe_experts_gate_up(pref, P(xpad), P(perm), P(offsets),
                                                  P(dinp["W_gate"]), P(dinp["W_up"]), P(H),
                                                  P(wpad), wpad.numel(), sp)),
        ("down", lambda: L.moe_experts_down(pref, P(H), P(offsets), P(dinp["W_down"]), P(Yp),
                                            P(wpad), wpad.numel(), sp)),
        ("combine", lambda: L.moe_combine_expert_choice(dref, P(Yp), P(slot), P(probs),
                                                        P(out2), sp)),
    ])
    st.counts = torch.full((E,), C, dtype=torch.int32, device=dev)
    st.offsets = offsets
    return st


def cpu_baseline_ec(wl, inp, sample, layer_flops):
    """The oracle on the host for an expert-choice layer: probabilities and the per-expert
    selection of the whole batch, plus the experts of a sample of tokens (each through
    every expert that took it), scaled to the whole batch.  One warm-up, then the median
    of three runs of each part."""
    import numpy as np

    import oracle
    from oracle import moe_oracle as mo
    blas, nproc, ncpu, model = host_info()
    if not sample:
        per_tok = 6.0 * wl.d * wl.F * (wl.k + wl.n_shared)
        sample = int(max(8, min(wl.T, 2.0e12 / per_tok)))
    x = mo._np(inp["x"])
    C = oracle.expert_choice_capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    state = {}

    def route_part():
        state["probs"] = oracle.router_probs(x, mo._np(inp["W_router"]))
        state["sel"], _ = oracle.expert_choice_select(state["probs"], C)

    t_route, _ = timed_runs(route_part)
    rows = np.linspace(0, wl.T - 1, sample).astype(np.int64)
    hb = wl.dtype == "bf16"

    def expert_part():
        probs, sel = state["probs"], state["sel"]
        y = np.zeros((rows.size, wl.d))
        for e in range(wl.E):
            hit = np.nonzero(np.isin(rows, sel[e]))[0]
            if hit.size:
                o = oracle.expert_ffn(x[rows[hit]], *oracle.expert_weights(inp, e), hb)
                y[hit] += probs[rows[hit], e].astype(np.float64)[:, None] * o
        return y

    t_exp, ts = timed_runs(expert_part)
    full = t_route + t_exp * wl.T / rows.size
    log(f"[bench] oracle: probabilities+selection {t_route:.2f}s for {wl.T} tokens, experts "
        f"{t_exp:.2f}s for {rows.size} tokens -> {full:.1f}s per batch")
    return {"value": wl.T / full, "unit": "tokens/s", "cores": blas, "kind": "oracle",
            "gflops": layer_flops / full / 1e9, "nproc": nproc, "cpu_count": ncpu,
            "cpu_model": model, "runs": "1 warm-up + median of 3",
            "sample": f"probabilities and expert-choice selection of all {wl.T} tokens "
                      f"({t_route:.2f}s) + experts of {rows.size} evenly spaced tokens "
                      f"({t_exp:.2f}s), scaled to the batch"}


if __name__ == "__main__":
    main()
