"""Pins for the CPU oracle: values the pages print, closed forms, library routines and
brute force.  CPU only.  Each pin is chosen so that a plausible mistake in the oracle
(a dropped term, a wrong sign or index, a transposed operand) fails at least one test;
the planted-mistake tests at the bottom check that on the CPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import moe_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def probs_as_router(probs):
    """Router inputs whose softmax is exactly ``probs``: x_t = ln p_t, W_router = I."""
    probs = np.asarray(probs, np.float64)
    E = probs.shape[1]
    return np.log(probs).astype(np.float64), np.eye(E)


# --------------------------------------------------------------------------- worked examples
def test_renorm_worked_example():
    g = golden("renorm_example.json")
    x, W = probs_as_router([g["probs"]])
    r = oracle.route(x, W, g["k"])
    np.testing.assert_allclose(r["p"][0], g["probs"], rtol=1e-6)
    assert r["idx"][0].tolist() == g["top_k_indices"]
    np.testing.assert_allclose(r["w"][0], g["weights_exact"], rtol=1e-6)
    assert [round(float(v), 2) for v in r["w"][0]] == g["weights_printed"]
    assert abs(float(r["w"][0].sum()) - 1.0) < 1e-6


def test_aux_loss_worked_example():
    g = golden("aux_loss_example.json")
    x, W = probs_as_router(g["probs"])
    r = oracle.route(x, W, g["k"])
    assert r["idx"][:, 0].tolist() == g["selected"]
    f, P = oracle.aux_stats(r["p"], r["idx"], 2)
    assert f.tolist() == g["f"]                      # exact: 3/4 and 1/4
    np.testing.assert_allclose(P, g["P"], atol=1e-7)
    assert abs(oracle.balance_loss(f, P) - g["loss"]) < 1e-6
    # top-1 weights are the renormalisation of one value
    assert np.all(r["w"] == 1.0)


def test_selection_bias_worked_example():
    g = golden("selection_bias_example.json")
    scores = np.asarray(g["scores"]) / sum(g["scores"])
    bias = (np.asarray(g["bias"]) / sum(g["scores"])).astype(np.float32)
    x, W = probs_as_router([scores])
    r = oracle.route(x, W, g["k"], bias)
    assert (r["idx"][0] + 1).tolist() == g["selected_1based"]
    np.testing.assert_allclose(r["w"][0], g["weights_from_raw"], rtol=1e-6)
    np.testing.assert_allclose(r["s"][0] * sum(g["scores"]), g["selection_scores"], atol=1e-6)
    # without the bias the same token picks experts 1 and 2 (1-based)
    r0 = oracle.route(x, W, g["k"])
    assert (r0["idx"][0] + 1).tolist() == [1, 2]


def test_capacity_closed_form():
    for c in golden("capacity_examples.json")["cases"]:
        assert oracle.capacity(c["T"], c["k"], c["E"], c["cf"]) == c["C"], c
    # top-1: the book's (T/E)*cf is the same number
    assert oracle.capacity(16384, 1, 64, 1.25) == int(16384 / 64 * 1.25)
    assert oracle.capacity(100, 2, 8, 0.0) is None
    assert oracle.capacity(100, 2, 8, -1.0) is None


def test_capacity_of_dyadic_factors_is_integer_division():
    """cf = n/64 is exact in float32, so floor(cf k T / E) is the integer quotient
    (n k T) // (64 E): any rounding of the product, or a wrong operand, shows up on
    some of these."""
    for n in range(1, 400, 3):
        for k, T, E in [(1, 16384, 64), (2, 4096, 8), (2, 250, 3), (8, 8192, 256), (3, 77, 7),
                        (1, 1, 1), (16, 5, 512)]:
            q = (n * k * T) // (64 * E)
            assert oracle.capacity(T, k, E, n / 64) == max(min(q, T * k), k), (n, k, T, E)


# --------------------------------------------------------------------------- closed forms
def test_balance_loss_is_one_when_uniform():
    rng = np.random.default_rng(1)
    E, T, k = 8, 64, 2
    # uniform probabilities, any assignment -> loss 1
    p = np.full((T, E), 1.0 / E, np.float32)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    f, P = oracle.aux_stats(p, idx, E)
    assert abs(oracle.balance_loss(f, P) - 1.0) < 1e-6
    # uniform assignment counts, any probabilities -> loss 1
    p = rng.dirichlet(np.ones(E), T).astype(np.float32)
    idx = np.arange(T * k, dtype=np.int32).reshape(T, k) % E
    f, P = oracle.aux_stats(p, idx, E)
    assert np.allclose(f, 1.0 / E)
    assert abs(oracle.balance_loss(f, P) - 1.0) < 1e-6


def test_balance_loss_grows_with_imbalance():
    E, T = 4, 400
    losses = []
    for a in [0.25, 0.4, 0.6, 0.8, 0.95]:
        p = np.tile(np.array([a] + [(1 - a) / 3] * 3, np.float32), (T, 1))
        idx = np.zeros((T, 1), np.int32)
        idx[: int(T * (1 - a))] = 1
        f, P = oracle.aux_stats(p, idx, E)
        losses.append(oracle.balance_loss(f, P))
    assert abs(losses[0] - 1.0) < 1e-6 or losses[0] >= 1.0
    assert all(b > a for a, b in zip(losses, losses[1:]))


def test_topk_weights_sum_to_one_and_ordered():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 32))
    W = rng.standard_normal((16, 32)) / math.sqrt(32)
    for k in (1, 2, 5, 16):
        r = oracle.route(x, W, k)
        np.testing.assert_allclose(r["w"].sum(axis=1), 1.0, atol=1e-6)
        sel = np.take_along_axis(r["s"], r["idx"].astype(np.int64), axis=1)
        assert np.all(np.diff(sel, axis=1) <= 0)


def test_topk_ties_go_to_lower_index():
    p = np.array([[0.25, 0.25, 0.25, 0.25], [0.1, 0.3, 0.3, 0.3]], np.float32)
    idx, s, margin = oracle.select_topk(p, 2)
    assert idx.tolist() == [[0, 1], [1, 2]]
    assert np.all(margin == 0.0)


# --------------------------------------------------------------------------- library routines
def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    a = rng.standard_normal(100_000).astype(np.float32) * np.float32(10.0) ** rng.integers(-6, 6, 100_000)
    # exact midpoints between neighbouring bf16 values, both parities
    odd = (np.arange(128, dtype=np.uint32) * 2 + 1) << np.uint32(15)     # bit 15 set, low bits 0
    expo = (np.arange(100, 150, dtype=np.uint32) << np.uint32(23))
    mid = (odd[None, :] | expo[:, None]).ravel().view(np.float32)
    for v in (a, mid, -mid):
        ref = torch.from_numpy(v.copy()).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(oracle.bf16_round(v), ref)


def test_softmax_and_silu_match_torch():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((40, 24))
    W = rng.standard_normal((12, 24))
    ref = torch.softmax(torch.from_numpy(x) @ torch.from_numpy(W).T, dim=-1).numpy()
    np.testing.assert_allclose(oracle.router_probs(x, W), ref, rtol=1e-6, atol=1e-9)
    z = rng.standard_normal(1000) * 8
    np.testing.assert_allclose(oracle.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-12, atol=1e-15)


def test_expert_ffn_matches_torch_swiglu():
    rng = np.random.default_rng(5)
    d, F, n = 48, 80, 17                   # d != F so a transposed weight cannot pass
    x = rng.standard_normal((n, d)).astype(np.float32)
    Wg = (rng.standard_normal((F, d)) / math.sqrt(d)).astype(np.float32)
    Wu = (rng.standard_normal((F, d)) / math.sqrt(d)).astype(np.float32)
    Wd = (rng.standard_normal((d, F)) / math.sqrt(F)).astype(np.float32)
    t = lambda a: torch.from_numpy(a.astype(np.float64))
    h = torch.nn.functional.silu(t(x) @ t(Wg).T) * (t(x) @ t(Wu).T)
    ref = (h.float().double() @ t(Wd).T).numpy()
    np.testing.assert_allclose(oracle.expert_ffn(x, Wg, Wu, Wd, False), ref, rtol=1e-5, atol=1e-6)
    hb = h.float().to(torch.bfloat16).double()
    refb = (hb @ t(Wd).T).numpy()
    np.testing.assert_allclose(oracle.expert_ffn(x, Wg, Wu, Wd, True), refb, rtol=1e-5, atol=1e-6)


# --------------------------------------------------------------------------- brute force
def brute_dispatch(idx, E, C):
    T, k = idx.shape
    seen = [0] * E
    rank = {}
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            rank[(t, j)] = seen[e]
            seen[e] += 1
    kept = [min(c, C) if C is not None else c for c in seen]
    offs = [0]
    for e in range(E):
        offs.append(offs[-1] + kept[e])
    slot = []
    perm = [None] * offs[-1]
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            r = rank[(t, j)]
            if C is None or r < C:
                slot.append(offs[e] + r)
                perm[offs[e] + r] = t * k + j
            else:
                slot.append(-1)
    return seen, kept, offs, perm, slot


@pytest.mark.parametrize("T,E,k,C", [(37, 5, 2, None), (64, 8, 1, 6), (50, 7, 3, 19), (1, 4, 4, None),
                                     (20, 3, 1, 1), (0, 4, 2, None)])
def test_dispatch_brute_force(T, E, k, C):
    rng = np.random.default_rng(T * 100 + E)
    # distinct experts per token, skewed toward low ids
    pr = np.linspace(2, 1, E) / np.linspace(2, 1, E).sum()
    idx = np.array([rng.choice(E, k, replace=False, p=pr) for _ in range(T)],
                   dtype=np.int32).reshape(T, k)
    d = oracle.dispatch(idx, E, C)
    seen, kept, offs, perm, slot = brute_dispatch(idx, E, C)
    assert d["counts"].tolist() == seen
    assert d["kept"].tolist() == kept
    assert d["offsets"].tolist() == offs
    assert d["perm_src"].tolist() == perm
    assert d["slot_pos"].tolist() == slot
    assert sum(seen) == T * k
    kept_pos = d["slot_pos"][d["slot_pos"] >= 0]
    assert sorted(kept_pos.tolist()) == list(range(offs[-1]))     # bijection


def make_small(T, d, E, k, F, S=0, seed=0, bias=0.0, dtype=np.float32):
    rng = np.random.default_rng(seed)
    inp = {
        "x": rng.standard_normal((T, d)).astype(np.float32),
        "W_router": (rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32),
        "W_gate": (rng.standard_normal((E + S, F, d)) / math.sqrt(d)).astype(np.float32),
        "W_up": (rng.standard_normal((E + S, F, d)) / math.sqrt(d)).astype(np.float32),
        "W_down": (rng.standard_normal((E + S, d, F)) / math.sqrt(F)).astype(np.float32),
        "router_bias": (rng.uniform(-bias, bias, E).astype(np.float32) if bias else None),
    }
    return inp


def per_token_loop(inp, k, S, cf, h_bf16):
    """Independent formulation: one token at a time, no permutation."""
    x = inp["x"].astype(np.float64)
    T, d = x.shape
    E = inp["W_router"].shape[0]
    C = None if cf <= 0 else max(int(math.floor(cf * k * T / E)), k)
    used = [0] * E
    y = np.zeros((T, d))
    for t in range(T):
        logits = [float(np.dot(x[t], inp["W_router"][e].astype(np.float64))) for e in range(E)]
        m = max(logits)
        ex = [math.exp(v - m) for v in logits]
        p = np.array([v / sum(ex) for v in ex], np.float32)
        s = p if inp["router_bias"] is None else (p + inp["router_bias"]).astype(np.float32)
        chosen = []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or s[e] > s[best]:
                    best = e
            chosen.append(best)
        tot = sum(float(p[e]) for e in chosen)
        for e in chosen:
            w = np.float32(float(p[e]) / tot)
            keep = C is None or used[e] < C
            used[e] += 1
            if not keep:
                continue
            g = inp["W_gate"][e].astype(np.float64) @ x[t]
            u = inp["W_up"][e].astype(np.float64) @ x[t]
            h = np.float32(1) * (g / (1 + np.exp(-g)) * u).astype(np.float32)
            if h_bf16:
                h = oracle.bf16_round(h)
            o = (inp["W_down"][e].astype(np.float64) @ h.astype(np.float64)).astype(np.float32)
            y[t] += float(w) * o.astype(np.float64)
        if S:
            g = inp["W_gate"][E].astype(np.float64) @ x[t]
            u = inp["W_up"][E].astype(np.float64) @ x[t]
            h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
            if h_bf16:
                h = oracle.bf16_round(h)
            y[t] += (inp["W_down"][E].astype(np.float64) @ h.astype(np.float64)).astype(np.float32)
    return y.astype(np.float32)


@pytest.mark.parametrize("T,d,E,k,F,S,cf,bias,hb", [
    (24, 16, 6, 2, 20, 0, 0.0, 0.0, False),
    (30, 12, 5, 1, 8, 0, 1.0, 0.0, True),
    (40, 16, 8, 3, 12, 1, 1.25, 0.05, True),
    (9, 8, 4, 4, 8, 0, 0.0, 0.0, False),
])
def test_forward_matches_per_token_loop(T, d, E, k, F, S, cf, bias, hb):
    inp = make_small(T, d, E, k, F, S, seed=T + d, bias=bias)
    out = oracle.forward(inp, k, cf, S, h_bf16=hb)
    ref = per_token_loop(inp, k, S, cf, hb)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-5, atol=1e-6)


def test_identical_experts_reduce_to_dense_ffn():
    """With every expert identical, sum_j w_tj = 1 gives the dense FFN for any k,
    including k = E, where the layer is a dense mixture ([book ch.30] 30.2.5)."""
    T, d, E, F = 20, 16, 6, 24
    inp = make_small(T, d, E, 1, F, seed=7)
    for key in ("W_gate", "W_up", "W_down"):
        inp[key] = np.repeat(inp[key][:1], E, axis=0)
    dense = oracle.expert_ffn(inp["x"], inp["W_gate"][0], inp["W_up"][0], inp["W_down"][0], False)
    for k in (1, 2, 3, E):
        y = oracle.forward(inp, k, 0.0, 0, h_bf16=False)["y"]
        np.testing.assert_allclose(y, dense, rtol=2e-6, atol=1e-6)


def test_shared_expert_alone_when_routed_outputs_are_zero():
    T, d, E, F = 16, 12, 4, 10
    inp = make_small(T, d, E, 2, F, S=1, seed=8)
    inp["W_down"][:E] = 0.0
    y = oracle.forward(inp, 2, 0.0, 1, h_bf16=False)["y"]
    shared = oracle.expert_ffn(inp["x"], inp["W_gate"][E], inp["W_up"][E], inp["W_down"][E], False)
    np.testing.assert_allclose(y, shared, rtol=1e-6, atol=1e-7)


def test_dropped_tokens_give_zero():
    T, d, E, F = 32, 8, 4, 8
    inp = make_small(T, d, E, 1, F, seed=9)
    out = oracle.forward(inp, 1, 0.25, 0, h_bf16=False)       # C = max(floor(2), 1) = 2
    assert out["C"] == 2
    dropped = out["dispatch"]["slot_pos"] < 0
    assert dropped.sum() == T - 2 * np.count_nonzero(out["dispatch"]["counts"])
    assert np.all(out["y"][dropped] == 0.0)
    assert np.all(np.abs(out["y"][~dropped]).sum(axis=1) > 0)


def test_row_independence_without_capacity():
    """The same tokens at batch 1 and in a batch route and compute identically
    ([MoE practice] inference-stability section: batch-consistency check)."""
    T, d, E, F, k = 30, 16, 6, 12, 2
    inp = make_small(T, d, E, k, F, seed=10, bias=0.02)
    full = oracle.forward(inp, k, 0.0, 0, h_bf16=True)["y"]
    for sub in ([3], [0, 7, 29], list(range(5, 17))):
        part = {key: (v[sub] if key == "x" else v) for key, v in inp.items()}
        y = oracle.forward(part, k, 0.0, 0, h_bf16=True)["y"]
        np.testing.assert_array_equal(y, full[sub])


def test_forward_rows_matches_forward_with_capacity():
    T, d, E, F, k = 48, 16, 6, 12, 2
    inp = make_small(T, d, E, k, F, S=1, seed=11, bias=0.03)
    out = oracle.forward(inp, k, 1.0, 1, h_bf16=True)
    rows = [0, 5, 17, 33, 47]
    y = oracle.forward_rows(inp, rows, k, 1.0, 1, h_bf16=True)
    np.testing.assert_allclose(y, out["y"][rows], rtol=1e-6, atol=1e-7)


# --------------------------------------------------------------------------- planted mistakes
def _pins_fail(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    """Each plausible oracle mistake below, planted on the CPU, fails some pin."""
    # 1. renormalisation dropped
    with monkeypatch.context() as m:
        m.setattr(mo, "renorm_weights",
                  lambda p, idx: np.take_along_axis(p, idx.astype(np.int64), axis=1).astype(np.float32))
        assert _pins_fail(test_renorm_worked_example)
    # 2. bias used for the weights as well
    orig_renorm = mo.renorm_weights
    with monkeypatch.context() as m:
        def route_bias_weights(x, W, k, bias=None):
            r = orig_route(x, W, k, bias)
            s = r["s"]
            r["w"] = orig_renorm(s, r["idx"])
            return r
        orig_route = mo.route
        m.setattr(mo, "route", route_bias_weights)
        m.setattr(oracle, "route", route_bias_weights)
        assert _pins_fail(test_selection_bias_worked_example)
    # 3. f normalised by T instead of T*k
    with monkeypatch.context() as m:
        def bad_stats(p, idx, E):
            c = np.bincount(idx.ravel(), minlength=E)
            return (c / idx.shape[0]).astype(np.float32), p.mean(axis=0).astype(np.float32)
        m.setattr(oracle, "aux_stats", bad_stats)
        assert _pins_fail(test_balance_loss_is_one_when_uniform)
    # 4. SiLU on the up projection instead of the gate
    with monkeypatch.context() as m:
        def swapped(x_rows, Wg, Wu, Wd, h_bf16):
            return orig_ffn(x_rows, Wu, Wg, Wd, h_bf16)
        orig_ffn = mo.expert_ffn
        m.setattr(oracle, "expert_ffn", swapped)
        assert _pins_fail(test_expert_ffn_matches_torch_swiglu)
    # 5. capacity kept by reverse order (last-come wins)
    with monkeypatch.context() as m:
        orig_dispatch = mo.dispatch
        def reversed_dispatch(idx, E, C=None):
            T, k = idx.shape
            d = orig_dispatch(idx[::-1].copy(), E, C)
            sp = d["slot_pos"].reshape(T, k)[::-1].reshape(-1)
            return dict(d, slot_pos=sp)
        m.setattr(oracle, "dispatch", reversed_dispatch)
        assert _pins_fail(lambda: test_dispatch_brute_force(64, 8, 1, 6))
    # 6. combine ignores the mixing weights
    with monkeypatch.context() as m:
        orig_combine = mo.combine
        m.setattr(mo, "combine", lambda T, d, w, sp, Y, shared=None:
                  orig_combine(T, d, np.ones_like(w), sp, Y, shared))
        assert _pins_fail(test_identical_experts_reduce_to_dense_ffn)


# ------------------------------------------------------------------ 8-bit expert weights
def test_e4m3_decode_matches_torch_for_every_code():
    """The oracle's e4m3 decoder (written from the format definition) against the
    library's float8_e4m3fn conversion, for all 256 codes (NaN where it is NaN)."""
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (mine == lib) | (np.isnan(mine) & np.isnan(lib))
    assert same.all(), codes[~same]


def test_e4m3_decode_fixed_values():
    """Values fixed by the encoding: 1.0, the largest finite value 448, the smallest
    subnormal 2^-9, the smallest normal 2^-6, the largest subnormal 7/8 * 2^-6, signs,
    and the two NaN codes."""
    v = oracle.e4m3_decode(np.array([0x00, 0x38, 0x7E, 0x01, 0x08, 0x07, 0xB8, 0x80, 0x40],
                                    np.uint8))
    assert list(v) == [0.0, 1.0, 448.0, 2.0 ** -9, 2.0 ** -6, 7 / 8 * 2.0 ** -6, -1.0, 0.0, 2.0]
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def _fp8_small(T, d, E, k, F, S=0, seed=0, bias=0.0):
    """make_small with the expert weights stored as per-row e4m3 codes and scales."""
    inp = make_small(T, d, E, k, F, S, seed, bias)
    for name in ("W_gate", "W_up", "W_down"):
        W = torch.from_numpy(inp.pop(name))
        s = (W.abs().amax(dim=2) / 448.0).to(torch.float32)
        q = (W / s[..., None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        inp["Wq_" + name[2:]], inp["s_" + name[2:]] = q.numpy(), s.numpy()
    return inp


def _fp8_dequant_torch(inp, name, e):
    q = torch.from_numpy(np.ascontiguousarray(inp["Wq_" + name][e]))
    s = torch.from_numpy(np.ascontiguousarray(inp["s_" + name][e])).to(torch.float64)
    return (q.view(torch.float8_e4m3fn).to(torch.float64) * s[:, None]).numpy()


def test_fp8_expert_weights_are_scale_times_code():
    """W[n, :] = s[n] * decode(q[n, :]) exactly (library decode, float64 product)."""
    inp = _fp8_small(4, 16, 3, 1, 24, S=1, seed=11)
    for e in range(4):
        for name, got in zip(("gate", "up", "down"), oracle.expert_weights(inp, e)):
            np.testing.assert_array_equal(got, _fp8_dequant_torch(inp, name, e))


@pytest.mark.parametrize("T,d,E,k,F,S,cf,bias", [
    (24, 16, 6, 2, 20, 0, 0.0, 0.0),
    (40, 16, 8, 3, 12, 1, 1.25, 0.05),
])
def test_fp8_forward_matches_per_token_loop(T, d, E, k, F, S, cf, bias):
    """The layer with 8-bit expert weights equals the independent per-token loop run on
    the weights the library decodes."""
    inp = _fp8_small(T, d, E, k, F, S, seed=T + d, bias=bias)
    out = oracle.forward(inp, k, cf, S, h_bf16=True)
    deq = {key: v for key, v in inp.items() if not key.startswith(("Wq_", "s_"))}
    for name in ("gate", "up", "down"):
        deq["W_" + name] = np.stack([_fp8_dequant_torch(inp, name, e) for e in range(E + S)])
    ref = per_token_loop(deq, k, S, cf, True)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-5, atol=1e-6)


def test_fp8_planted_mistakes_are_caught(monkeypatch):
    """An exponent bias of 8 instead of 7, or scales applied per input column instead of
    per output row, fail the pins above."""
    orig = mo.e4m3_decode
    with monkeypatch.context() as m:
        m.setattr(mo, "e4m3_decode", lambda q: orig(q) / 2.0)
        m.setattr(oracle, "e4m3_decode", mo.e4m3_decode)
        assert _pins_fail(test_e4m3_decode_fixed_values)
        assert _pins_fail(test_e4m3_decode_matches_torch_for_every_code)
    with monkeypatch.context() as m:
        m.setattr(mo, "dequant_rows",
                  lambda q, s: np.resize(np.asarray(s, np.float64), q.shape[1])[None, :]
                  * orig(q))
        assert _pins_fail(test_fp8_expert_weights_are_scale_times_code)


# --------------------------------------------------------------------------- expert choice
def brute_expert_choice(p, C):
    """Python-sorted selection: per expert, tokens ordered by (-p, t), first C, ascending."""
    T, E = p.shape
    out = []
    for e in range(E):
        ranked = sorted(range(T), key=lambda t: (-float(p[t, e]), t))
        out.append(sorted(ranked[:C]))
    return np.array(out, np.int32).reshape(E, C)


def test_expert_choice_hand_example():
    """4 tokens, 2 experts, C = 2: expert 0 takes token 0 and the lower of the tied
    tokens 1 and 2; expert 1 takes token 3 and again token 1; nobody takes token 2."""
    p = np.array([[0.9, 0.1], [0.5, 0.5], [0.5, 0.5], [0.1, 0.9]], np.float32)
    sel, margin = oracle.expert_choice_select(p, 2)
    assert sel.tolist() == [[0, 1], [1, 3]]
    assert margin.tolist() == [0.0, 0.0]
    disp = oracle.expert_choice_dispatch(sel, 4)
    assert disp["slot"].tolist() == [[0, -1], [1, 2], [-1, -1], [-1, 3]]
    assert disp["offsets"].tolist() == [0, 2, 4]


@pytest.mark.parametrize("T,E,C,seed", [(12, 3, 4, 0), (40, 8, 7, 1), (9, 5, 9, 2), (33, 4, 1, 3)])
def test_expert_choice_select_brute_force(T, E, C, seed):
    rng = np.random.default_rng(seed)
    # coarse values so that ties occur
    p = (rng.integers(0, 6, (T, E)) / 8.0).astype(np.float32)
    sel, margin = oracle.expert_choice_select(p, C)
    np.testing.assert_array_equal(sel, brute_expert_choice(p, C))
    for e in range(E):
        col = np.sort(p[:, e].astype(np.float64))[::-1]
        assert margin[e] == (np.inf if C == T else col[C - 1] - col[C])


def test_expert_choice_capacity():
    assert oracle.expert_choice_capacity(4096, 2, 8, 1.0) == 1024
    assert oracle.expert_choice_capacity(10, 2, 8, 1.0) == 2          # at least k
    assert oracle.expert_choice_capacity(10, 2, 8, 100.0) == 10       # at most T
    with pytest.raises(ValueError):
        oracle.expert_choice_capacity(10, 2, 8, 0.0)


def per_token_expert_choice(inp, k, cf, S, h_bf16):
    """Independent formulation: the selection by Python sorting, then one token at a
    time over the experts that took it."""
    x = inp["x"].astype(np.float64)
    T, d = x.shape
    E = inp["W_router"].shape[0]
    C = min(T, max(int(math.floor(cf * k * T / E)), k))
    logits = x @ inp["W_router"].astype(np.float64).T
    ex = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    taken = [set(s) for s in brute_expert_choice(p, C).tolist()]
    y = np.zeros((T, d))
    for t in range(T):
        for e in range(E + S):
            if e < E and t not in taken[e]:
                continue
            g = inp["W_gate"][e].astype(np.float64) @ x[t]
            u = inp["W_up"][e].astype(np.float64) @ x[t]
            h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
            if h_bf16:
                h = oracle.bf16_round(h)
            o = (inp["W_down"][e].astype(np.float64) @ h.astype(np.float64)).astype(np.float32)
            y[t] += (float(p[t, e]) if e < E else 1.0) * o.astype(np.float64)
    return y.astype(np.float32)


@pytest.mark.parametrize("T,d,E,k,F,S,cf,hb", [
    (24, 16, 6, 2, 20, 0, 1.0, False),
    (30, 12, 5, 1, 8, 1, 1.25, True),
    (17, 8, 4, 3, 12, 0, 0.5, True),
])
def test_expert_choice_forward_matches_per_token_loop(T, d, E, k, F, S, cf, hb):
    inp = make_small(T, d, E, k, F, S, seed=3 * T + d)
    out = oracle.forward_expert_choice(inp, k, cf, S, h_bf16=hb)
    ref = per_token_expert_choice(inp, k, cf, S, hb)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-5, atol=1e-6)
    C = out["C"]
    assert out["sel"].shape == (E, C)
    np.testing.assert_allclose(out["f"], np.full(E, 1.0 / E), rtol=1e-6)
    np.testing.assert_allclose(out["p"], oracle.router_probs(inp["x"], inp["W_router"]).mean(0),
                               rtol=1e-6)


def test_expert_choice_every_token_reduces_to_dense_mixture():
    """With C = T every expert takes every token, so y_t = sum_e p[t, e] FFN_e(x_t); with
    identical experts the probabilities sum to one and y is the dense FFN."""
    T, d, E, F = 20, 16, 5, 24
    inp = make_small(T, d, E, 1, F, seed=5)
    out = oracle.forward_expert_choice(inp, E, 1.0, 0, h_bf16=False)   # C = T
    assert out["C"] == T
    p = oracle.router_probs(inp["x"], inp["W_router"]).astype(np.float64)
    mix = sum(p[:, e:e + 1] * oracle.expert_ffn(inp["x"], inp["W_gate"][e], inp["W_up"][e],
                                                inp["W_down"][e], False).astype(np.float64)
              for e in range(E))
    np.testing.assert_allclose(out["y"], mix, rtol=1e-5, atol=1e-6)
    for key in ("W_gate", "W_up", "W_down"):
        inp[key] = np.repeat(inp[key][:1], E, axis=0)
    dense = oracle.expert_ffn(inp["x"], inp["W_gate"][0], inp["W_up"][0], inp["W_down"][0], False)
    y = oracle.forward_expert_choice(inp, E, 1.0, 0, h_bf16=False)["y"]
    np.testing.assert_allclose(y, dense, rtol=2e-6, atol=1e-6)


def test_expert_choice_loads_are_equal_and_untaken_tokens_give_zero():
    T, d, E, F = 64, 8, 4, 8
    inp = make_small(T, d, E, 1, F, seed=9)
    out = oracle.forward_expert_choice(inp, 1, 0.25, 0, h_bf16=False)   # C = 4 of 64
    C = out["C"]
    assert C == 4
    slot = out["dispatch"]["slot"]
    assert ((slot >= 0).sum(axis=0) == C).all()
    untaken = np.nonzero((slot < 0).all(axis=1))[0]
    assert untaken.size >= T - E * C
    assert not out["y"][untaken].any()


def test_expert_choice_planted_mistakes_are_caught(monkeypatch):
    """Ties to the higher token index, the lowest instead of the highest scores, tokens
    ranked by logits instead of probabilities, or renormalised weights fail a pin."""
    with monkeypatch.context() as m:
        m.setattr(mo, "expert_choice_select",
                  lambda p, C: (np.sort(np.array([np.argsort(-p[:, e].astype(np.float64)[::-1],
                                                              kind="stable")[:C] * -1 + p.shape[0] - 1
                                                  for e in range(p.shape[1])]), axis=1)
                                .astype(np.int32), np.zeros(p.shape[1])))
        m.setattr(oracle, "expert_choice_select", mo.expert_choice_select)
        assert _pins_fail(test_expert_choice_hand_example)
    with monkeypatch.context() as m:
        m.setattr(mo, "expert_choice_select",
                  lambda p, C: (np.sort(np.argsort(p.T.astype(np.float64), axis=1,
                                                   kind="stable")[:, :C], axis=1).astype(np.int32),
                                np.zeros(p.shape[1])))
        m.setattr(oracle, "expert_choice_select", mo.expert_choice_select)
        assert _pins_fail(lambda: test_expert_choice_select_brute_force(40, 8, 7, 1))
    orig_probs = mo.router_probs
    with monkeypatch.context() as m:
        m.setattr(mo, "router_probs",
                  lambda x, W: (x.astype(np.float64) @ W.astype(np.float64).T).astype(np.float32))
        assert _pins_fail(lambda: test_expert_choice_forward_matches_per_token_loop(
            24, 16, 6, 2, 20, 0, 1.0, False))
    orig_combine = mo.combine
    with monkeypatch.context() as m:
        m.setattr(mo, "combine",
                  lambda T, d, w, sp, Y, sh=None: orig_combine(
                      T, d, (w / np.maximum(np.where(sp.reshape(w.shape) >= 0, w, 0).sum(1,
                             keepdims=True), 1e-30)).astype(np.float32), sp, Y, sh))
        assert _pins_fail(lambda: test_expert_choice_forward_matches_per_token_loop(
            24, 16, 6, 2, 20, 0, 1.0, False))
    assert orig_probs is mo.router_probs


# --------------------------------------------------------------------------- next best
def brute_next_best(idx, s, E, C):
    """Sequential formulation: per-expert load counters; first every assignment in
    row-major order takes its top-k expert if it has room; then every assignment that
    found none, in row-major order, takes its token's next unused expert by score (the
    m-th such slot of the token its (k+1+m)-th best) if that one has room."""
    T, k = idx.shape
    load = [0] * E
    final = [[-1] * k for _ in range(T)]
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if load[e] < C:
                load[e] += 1
                final[t][j] = e
    for t in range(T):
        ranked = sorted(range(E), key=lambda e: (-float(s[t, e]), e))
        rest = [e for e in ranked if e not in set(int(v) for v in idx[t])]
        m = 0
        for j in range(k):
            if final[t][j] >= 0:
                continue
            if m < len(rest) and m < k:
                e = rest[m]
                if load[e] < C:
                    load[e] += 1
                    final[t][j] = e
            m += 1
    return np.array(final, np.int64)


def test_next_best_hand_example():
    """3 experts, C = 1: tokens 0-2 pick expert 0, token 3 expert 1.  Token 0 keeps
    expert 0; token 1 moves to its next best, expert 2; token 2's next best, expert 1, is
    full, so it is dropped."""
    idx = np.array([[0], [0], [0], [1]])
    s = np.array([[.5, .3, .2], [.6, .1, .3], [.7, .2, .1], [.1, .8, .1]], np.float32)
    cand = oracle.next_best_candidates(s, 1, idx)
    assert cand.ravel().tolist() == [1, 2, 1, 0]
    d = oracle.dispatch_next_best(idx, cand, 3, 1)
    assert d["expert"].tolist() == [0, 2, -1, 1]
    assert d["offsets"].tolist() == [0, 1, 2, 3]
    assert d["perm_src"].tolist() == [0, 3, 1]
    assert d["slot_pos"].tolist() == [0, 2, -1, 1]


@pytest.mark.parametrize("T,E,k,C,seed", [(40, 6, 2, 9, 0), (64, 8, 1, 5, 1), (30, 5, 3, 20, 2),
                                          (25, 4, 2, 15, 3), (25, 4, 2, 3, 3), (50, 16, 4, 14, 4)])
def test_next_best_matches_sequential_loop(T, E, k, C, seed):
    rng = np.random.default_rng(seed)
    s = (rng.integers(0, 9, (T, E)) / 16.0 + rng.random((T, E)) * 1e-3).astype(np.float32)
    s[:, 0] += 0.5                                   # skew: expert 0 overflows
    idx = np.argsort(-s.astype(np.float64), axis=1, kind="stable")[:, :k]
    d = oracle.dispatch_next_best(idx, oracle.next_best_candidates(s, k, idx), E, C)
    final = brute_next_best(idx, s, E, C)
    np.testing.assert_array_equal(d["expert"].reshape(T, k), final)
    kept = np.bincount(final[final >= 0], minlength=E)
    assert (kept <= C).all()
    np.testing.assert_array_equal(np.diff(d["offsets"]), kept)
    for t in range(T):                               # never two rows of one expert per token
        used = final[t][final[t] >= 0]
        assert len(set(used.tolist())) == used.size
    # rows: round-0 assignments, then the redirected ones, each in row-major order
    for e in range(E):
        rows = d["perm_src"][d["offsets"][e]:d["offsets"][e + 1]]
        moved = np.array([idx.reshape(-1)[i] != e for i in rows])
        assert not (moved[:-1] & ~moved[1:]).any()
        assert np.all(np.diff(rows[~moved]) > 0) and np.all(np.diff(rows[moved]) > 0)
    if E * C >= T * k:                               # room left somewhere: some moved
        assert d["redirected"] > 0


def test_next_best_reduces_to_dispatch():
    """Without overflow, or with no candidate left, nothing moves."""
    rng = np.random.default_rng(5)
    T, E, k = 40, 6, 2
    s = rng.random((T, E)).astype(np.float32)
    idx = np.argsort(-s.astype(np.float64), axis=1, kind="stable")[:, :k]
    for C, cand in [(T * k, oracle.next_best_candidates(s, k, idx)),
                    (4, np.full((T, k), -1, np.int32))]:
        a = oracle.dispatch_next_best(idx, cand, E, C)
        b = oracle.dispatch(idx, E, C)
        for key in ("offsets", "perm_src", "slot_pos"):
            np.testing.assert_array_equal(a[key], b[key])


def per_token_next_best(inp, k, cf, h_bf16):
    """The layer with redirected overflow, one token at a time over brute_next_best."""
    x = inp["x"].astype(np.float64)
    T, d = x.shape
    E = inp["W_router"].shape[0]
    C = max(int(math.floor(cf * k * T / E)), k)
    logits = x @ inp["W_router"].astype(np.float64).T
    ex = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    s = p if inp["router_bias"] is None else (p + inp["router_bias"]).astype(np.float32)
    idx = np.array([sorted(range(E), key=lambda e: (-float(s[t, e]), e))[:k] for t in range(T)])
    final = brute_next_best(idx, s, E, C)
    y = np.zeros((T, d))
    for t in range(T):
        tot = sum(float(p[t, e]) for e in idx[t])
        for j in range(k):
            e = int(final[t, j])
            if e < 0:
                continue
            w = np.float32(float(p[t, idx[t, j]]) / tot)
            g = inp["W_gate"][e].astype(np.float64) @ x[t]
            u = inp["W_up"][e].astype(np.float64) @ x[t]
            h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
            if h_bf16:
                h = oracle.bf16_round(h)
            o = (inp["W_down"][e].astype(np.float64) @ h.astype(np.float64)).astype(np.float32)
            y[t] += float(w) * o.astype(np.float64)
    return y.astype(np.float32)


@pytest.mark.parametrize("T,d,E,k,F,cf,bias,hb", [
    (40, 16, 6, 2, 20, 1.0, 0.0, False),
    (48, 12, 8, 1, 8, 1.25, 0.2, True),
    (36, 16, 5, 3, 12, 0.8, 0.05, True),
])
def test_next_best_forward_matches_per_token_loop(T, d, E, k, F, cf, bias, hb):
    inp = make_small(T, d, E, k, F, 0, seed=7 * T + d, bias=bias)
    out = oracle.forward(inp, k, cf, 0, h_bf16=hb, next_best=True)
    ref = per_token_next_best(inp, k, cf, hb)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-5, atol=1e-6)
    # forward_rows follows the redirected experts too
    rows = np.arange(0, T, 3)
    yr = oracle.forward_rows(inp, rows, k, cf, 0, h_bf16=hb, routing=out["route"],
                             disp=out["dispatch"])
    np.testing.assert_allclose(yr, out["y"][rows], rtol=1e-5, atol=1e-6)


def test_next_best_planted_mistakes_are_caught(monkeypatch):
    """Offering the overflow to the token's k-th instead of (k+1)-th best expert, taking
    offers last-come first, or ignoring the capacity fails a pin."""
    orig = mo.next_best_candidates
    with monkeypatch.context() as m:
        m.setattr(mo, "next_best_candidates",
                  lambda s, k, idx=None: np.roll(orig(s, k, idx), 1, axis=1))
        m.setattr(oracle, "next_best_candidates", mo.next_best_candidates)
        assert _pins_fail(test_next_best_hand_example) or _pins_fail(
            lambda: test_next_best_matches_sequential_loop(50, 16, 4, 14, 4))
    orig_d = mo.dispatch_next_best
    with monkeypatch.context() as m:
        def last_come(idx, cand, E, C):
            T, k = idx.shape
            d = orig_d(idx[::-1].copy(), np.asarray(cand)[::-1].copy(), E, C)
            ex = d["expert"].reshape(T, k)[::-1].reshape(-1)
            return dict(d, expert=ex)
        m.setattr(mo, "dispatch_next_best", last_come)
        m.setattr(oracle, "dispatch_next_best", mo.dispatch_next_best)
        assert _pins_fail(lambda: test_next_best_matches_sequential_loop(40, 6, 2, 9, 0))
    with monkeypatch.context() as m:
        m.setattr(mo, "dispatch_next_best",
                  lambda idx, cand, E, C: orig_d(idx, cand, E, 10 ** 9) if C else None)
        m.setattr(oracle, "dispatch_next_best", mo.dispatch_next_best)
        assert _pins_fail(test_next_best_hand_example)
