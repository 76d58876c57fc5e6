"""Helpers for the GPU-vs-oracle parity tests: the comparison rules, and running the
oracle on the same seeded inputs the GPU gets."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import moe_oracle as mo

NEAR_TIE = 1e-6        # routing margin below which several routings are correct
STAT_TOL = 1e-5        # f and P
Y_MAX_REL = 2e-2       # max|y - y_ref| <= 2e-2 * max|y_ref|
Y_ELEM_REL = 5e-2      # per element, where |y_ref| > 1e-3 * max|y_ref|
Y_FLOOR = 1e-3


def check_y(y, y_ref, what=""):
    """The output rule: max|y - y_ref| <= 2e-2 max|y_ref| and per-element relative error
    <= 5e-2 wherever |y_ref| > 1e-3 max|y_ref|."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), what
    m = np.abs(y_ref).max() if y_ref.size else 0.0
    err = np.abs(y - y_ref)
    if m == 0.0:
        assert err.max(initial=0.0) == 0.0, what
        return
    assert err.max() <= Y_MAX_REL * m, f"{what}: max err {err.max():.3e} > {Y_MAX_REL} * {m:.3e}"
    mask = np.abs(y_ref) > Y_FLOOR * m
    rel = err[mask] / np.abs(y_ref[mask])
    bad = np.count_nonzero(rel > Y_ELEM_REL)
    assert bad == 0, f"{what}: {bad} elements over {Y_ELEM_REL} relative error (worst {rel.max():.3e})"


def np32(t):
    return mo._np(t)


def check_routing(idx_gpu, w_gpu, ref):
    """Routing indices bit-exact wherever the oracle's margin is >= 1e-6; near-tied tokens
    may differ, but their choice must still be a valid top-k within that margin.
    Returns the mask of near-tied tokens."""
    idx_gpu = np.asarray(idx_gpu)
    near = ref["margin"] < NEAR_TIE
    ok = ~near
    mism = np.nonzero(np.any(idx_gpu[ok] != ref["idx"][ok], axis=1))[0]
    assert mism.size == 0, f"{mism.size} tokens routed differently (first {np.nonzero(ok)[0][mism[:5]]})"
    s = ref["s"].astype(np.float64)
    k = idx_gpu.shape[1]
    for t in np.nonzero(near)[0]:
        chosen = s[t, idx_gpu[t]]
        assert len(set(idx_gpu[t].tolist())) == k
        kth = np.sort(s[t])[::-1][k - 1]
        assert np.all(chosen >= kth - NEAR_TIE)
        assert np.all(np.diff(chosen) <= NEAR_TIE)
    # weights: renormalised unbiased probabilities of the GPU's own choice
    w_ref = oracle.renorm_weights(ref["p"], idx_gpu)
    np.testing.assert_allclose(np.asarray(w_gpu), w_ref, rtol=2e-5, atol=1e-6)
    return near


def to_dev(inputs, device):
    return {k: (None if v is None else v.to(device)) for k, v in inputs.items()}


def bf16_ulp(v):
    """Spacing of bfloat16 numbers at |v| (8 significant bits)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


# fp32 evaluation of h = SiLU(g) * u from g and u: the bf16 kernels use the hardware exp2
# and reciprocal (about 1-2 ulp each, plus the rounding of -g*log2(e) scaled by |g|), so
# 16 ulp of |h| is allowed on top of the dot-product errors.
H_EVAL_ULPS = 16.0


def fp32_dot_error(x, W):
    """Statistical bound on the fp32 accumulation error of the dot products x W^T over K
    terms: the products of bf16 values are exact, each of the K additions rounds with
    relative error <= 2^-24 of a partial sum whose size grows like sqrt(i) times the rms
    term, so the error has standard deviation ~ 2^-24 * rms_term * K / sqrt(2); eight
    standard deviations are allowed."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    K = x.shape[1]
    rms = np.sqrt(np.maximum((x * x) @ (W * W).T, 0.0) / K)
    return 8.0 * 2.0 ** -24 * rms * K / np.sqrt(2.0)


def check_h_and_down(H_gpu, parts, x, Wg, Wu, Wd, Yp_gpu, o_ref, what=""):
    """Stage check of the expert FFN where h is rounded to bf16.

    Rounding h to bf16 decides a discrete value from a float.  The GPU's fp32 h differs
    from the oracle's float64 h by at most dh = |SiLU(g)| du + |u SiLU'(g)| dg + 4 ulp32(h)
    (du, dg from fp32_dot_error), so every GPU h must be the round-to-nearest-even bf16
    of some value in [h - dh, h + dh]: equal to the oracle's rounding except near a
    midpoint, where both neighbours are correct.  Given those h, Yp must equal the
    oracle's o up to the effect of the differences,
        |Yp - o| <= |W_down| |H - hq| + 4 sqrt(F) 2^-24 |W_down| |hq|,
    the second term covering fp32 accumulation over F products.
    """
    g, u, h64 = parts["g"], parts["u"], parts["h"]
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    dh = (np.abs(g * sig) * fp32_dot_error(x, Wu) + np.abs(u * dsilu) * fp32_dot_error(x, Wg)
          + H_EVAL_ULPS * 2.0 ** -24 * np.abs(h64))
    H_gpu = np.asarray(H_gpu, np.float64)
    hq = oracle.bf16_round(h64.astype(np.float32)).astype(np.float64)
    lo = oracle.bf16_round((h64 - dh).astype(np.float32)).astype(np.float64)
    hi = oracle.bf16_round((h64 + dh).astype(np.float32)).astype(np.float64)
    out = (H_gpu < np.minimum(lo, hi)) | (H_gpu > np.maximum(lo, hi))
    assert not out.any(), f"{what}: {out.sum()} h values are no rounding of [h-dh, h+dh] " \
                          f"(e.g. gpu {H_gpu[out][:3]} vs oracle {h64[out][:3]})"
    diff = H_gpu != hq
    assert diff.mean() < 1e-2, f"{what}: {diff.mean():.2e} of h values differ"
    Wd = np.abs(np.asarray(Wd, np.float64))
    F = Wd.shape[1]
    bound = np.abs(H_gpu - hq) @ Wd.T + 4.0 * np.sqrt(F) * 2.0 ** -24 * (np.abs(hq) @ Wd.T)
    err = np.abs(np.asarray(Yp_gpu, np.float64) - o_ref)
    bad = err > bound + 1e-30
    assert not bad.any(), f"{what}: {bad.sum()} Yp elements beyond the rounding bound " \
                          f"(worst excess {(err - bound).max():.3e})"
    return int(diff.sum())


def expert_rows_reference(inp, rows, k, n_shared, h_bf16, routing, disp):
    """For each sampled token row: the oracle's output row, and for every (slot, expert)
    that contributes, the oracle's g/u/h and o plus the row of H it occupies.
    Returns (y_ref [n, d], contributions list of (i, weight, e, pos, parts, o, x_row, W))."""
    x = np32(inp["x"])
    T, d = x.shape
    E = routing["p"].shape[1]
    rows = np.asarray(rows, np.int64)
    sp = disp["slot_pos"].reshape(T, k)[rows]
    idx = routing["idx"][rows]
    w = routing["w"][rows]
    items = []
    for e in np.unique(idx[sp >= 0]):
        sel = np.argwhere((idx == e) & (sp >= 0))
        Wg, Wu, Wd = oracle.expert_weights(inp, int(e))
        o, parts = oracle.expert_ffn(x[rows[sel[:, 0]]], Wg, Wu, Wd, h_bf16, return_h=True)
        for q, (i, j) in enumerate(sel):
            items.append((int(i), float(w[i, j]), int(e), int(sp[i, j]),
                          {key: v[q:q + 1] for key, v in parts.items()}, o[q:q + 1],
                          x[rows[i]:rows[i] + 1], (Wg, Wu, Wd)))
    if n_shared:
        Wg, Wu, Wd = oracle.expert_weights(inp, E)
        o, parts = oracle.expert_ffn(x[rows], Wg, Wu, Wd, h_bf16, return_h=True)
        for i in range(rows.size):
            items.append((i, 1.0, E, T * k + int(rows[i]),
                          {key: v[i:i + 1] for key, v in parts.items()}, o[i:i + 1],
                          x[rows[i]:rows[i] + 1], (Wg, Wu, Wd)))
    y = np.zeros((rows.size, d))
    for i, wt, e, pos, parts, o, xr, W in items:
        y[i] += wt * o[0].astype(np.float64)
    return y.astype(np.float32), items


def check_y_rounding_aware(y, y_ref, items, H_gpu, h_bf16, out_bf16, what=""):
    """The output rule on y, where the expert intermediate h is rounded to bf16.

    max|y - y_ref| <= 2e-2 max|y_ref| must hold outright.  The per-element rule (<= 5e-2
    relative where |y_ref| > 1e-3 max|y_ref|) must hold except where the difference is
    explained by bf16 roundings of h that went to the other neighbour of a midpoint:
    each such h is first validated (check_h_and_down on that row), and the element is
    then accepted if |y - y_ref| <= sum_j w_j |W_down| |H - hq| + accumulation and
    output rounding.  Returns the number of elements that needed that allowance."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    m = np.abs(y_ref).max()
    err = np.abs(y - y_ref)
    assert err.max() <= Y_MAX_REL * m, f"{what}: max err {err.max():.3e} > {Y_MAX_REL} * {m:.3e}"
    allow = np.zeros_like(y)
    for i, wt, e, pos, parts, o, xr, (Wg, Wu, Wd) in items:
        Hrow = np.asarray(H_gpu[pos:pos + 1], np.float64)
        Wda = np.abs(np.asarray(Wd, np.float64))
        if h_bf16:
            # every h of the row must be a correct rounding (raises otherwise)
            _check_h_only(Hrow, parts, xr, Wg, Wu, f"{what} expert {e}")
            hq = oracle.bf16_round(parts["h"].astype(np.float32)).astype(np.float64)
            allow[i] += wt * (np.abs(Hrow - hq) @ Wda.T)[0]
            F = Wda.shape[1]
            allow[i] += wt * 4.0 * np.sqrt(F) * 2.0 ** -24 * (np.abs(hq) @ Wda.T)[0]
        else:
            allow[i] += wt * 1e-6 * (np.abs(parts["h"]) @ Wda.T)[0]
    if out_bf16:
        allow += 2.0 ** -8 * np.abs(y_ref)
    mask = np.abs(y_ref) > Y_FLOOR * m
    rel = np.where(mask, err / np.where(mask, np.abs(y_ref), 1.0), 0.0)
    strict_bad = mask & (rel > Y_ELEM_REL)
    unexplained = strict_bad & (err > allow)
    assert not unexplained.any(), (
        f"{what}: {unexplained.sum()} elements over {Y_ELEM_REL} relative error not explained "
        f"by validated bf16 roundings of h (worst rel {rel[unexplained].max():.3e})")
    return int(strict_bad.sum())


def _check_h_only(H_gpu, parts, x, Wg, Wu, what=""):
    g, u, h64 = parts["g"], parts["u"], parts["h"]
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    dh = (np.abs(g * sig) * fp32_dot_error(x, Wu) + np.abs(u * dsilu) * fp32_dot_error(x, Wg)
          + H_EVAL_ULPS * 2.0 ** -24 * np.abs(h64))
    lo = oracle.bf16_round((h64 - dh).astype(np.float32)).astype(np.float64)
    hi = oracle.bf16_round((h64 + dh).astype(np.float32)).astype(np.float64)
    H_gpu = np.asarray(H_gpu, np.float64)
    out = (H_gpu < np.minimum(lo, hi)) | (H_gpu > np.maximum(lo, hi))
    assert not out.any(), f"{what}: {out.sum()} h values are no rounding of [h-dh, h+dh]"


def check_expert_choice(perm_gpu, offsets_gpu, slot_gpu, probs_ref, sel_ref, margin, C):
    """Expert-choice selection: each expert's tokens bit-exact wherever the oracle's margin
    (C-th minus (C+1)-th largest probability) is >= 1e-6; a near-tied expert's tokens must
    still be C distinct tokens, ascending, none below the C-th largest probability by more
    than 1e-6.  offsets are e*C and slot is the inverse of perm.  Returns the GPU's
    selection [E, C]."""
    T, E = probs_ref.shape
    perm_gpu = np.asarray(perm_gpu)[:E * C].reshape(E, C)
    assert np.array_equal(np.asarray(offsets_gpu), np.arange(E + 1) * C)
    for e in range(E):
        if margin[e] >= NEAR_TIE:
            assert np.array_equal(perm_gpu[e], sel_ref[e]), f"expert {e} took other tokens"
        else:
            col = probs_ref[:, e].astype(np.float64)
            kth = np.sort(col)[::-1][C - 1]
            assert len(set(perm_gpu[e].tolist())) == C
            assert np.all(col[perm_gpu[e]] >= kth - NEAR_TIE)
        assert np.all(np.diff(perm_gpu[e]) > 0), f"expert {e}: rows not in token order"
    slot_ref = np.full((T, E), -1, np.int64)
    for e in range(E):
        slot_ref[perm_gpu[e], e] = e * C + np.arange(C)
    assert np.array_equal(np.asarray(slot_gpu), slot_ref)
    return perm_gpu


def expert_choice_rows_reference(inp, rows, sel, probs, n_shared, h_bf16):
    """Like expert_rows_reference, for expert choice: token rows[i] gets p[t, e] * o_e for
    every expert e whose selection holds it (row e*C + its rank), plus the shared expert
    (row E*C + t)."""
    x = np32(inp["x"])
    T, d = x.shape
    E, C = sel.shape
    rows = np.asarray(rows, np.int64)
    items = []
    for e in range(E):
        pos = {int(t): e * C + r for r, t in enumerate(sel[e])}
        hit = [i for i, t in enumerate(rows) if int(t) in pos]
        if not hit:
            continue
        Wg, Wu, Wd = oracle.expert_weights(inp, e)
        o, parts = oracle.expert_ffn(x[rows[hit]], Wg, Wu, Wd, h_bf16, return_h=True)
        for q, i in enumerate(hit):
            t = int(rows[i])
            items.append((i, float(probs[t, e]), e, pos[t],
                          {key: v[q:q + 1] for key, v in parts.items()}, o[q:q + 1],
                          x[t:t + 1], (Wg, Wu, Wd)))
    if n_shared:
        Wg, Wu, Wd = oracle.expert_weights(inp, E)
        o, parts = oracle.expert_ffn(x[rows], Wg, Wu, Wd, h_bf16, return_h=True)
        for i in range(rows.size):
            items.append((i, 1.0, E, E * C + int(rows[i]),
                          {key: v[i:i + 1] for key, v in parts.items()}, o[i:i + 1],
                          x[rows[i]:rows[i] + 1], (Wg, Wu, Wd)))
    items.sort(key=lambda it: (it[0], it[2]))      # per row, experts ascending
    y = np.zeros((rows.size, d))
    for i, wt, e, pos, parts, o, xr, W in items:
        y[i] += wt * o[0].astype(np.float64)
    return y.astype(np.float32), items


def check_candidates(cand_gpu, idx_gpu, s_ref, k):
    """The next-best candidates: bit-exact for tokens whose remaining selection scores
    (outside the chosen k) are separated by >= 1e-6 among the first min(k, E-k)+1; else
    they must still be the best-scored remaining experts within 1e-6, in descending
    order.  Entries past E - k are -1."""
    cand_gpu = np.asarray(cand_gpu, np.int64)
    idx_gpu = np.asarray(idx_gpu, np.int64)
    T, E = s_ref.shape
    m = min(k, E - k)
    assert np.all(cand_gpu[:, m:] == -1)
    exp = oracle.next_best_candidates(s_ref, k, idx_gpu)
    s2 = s_ref.astype(np.float64).copy()
    np.put_along_axis(s2, idx_gpu, -np.inf, axis=1)
    srt = -np.sort(-s2, axis=1)[:, :E - k]
    q = min(m + 1, E - k)
    gaps = (srt[:, :q - 1] - srt[:, 1:q]).min(axis=1) if q >= 2 else np.full(T, np.inf)
    sure = gaps >= NEAR_TIE
    bad = np.nonzero(np.any(cand_gpu[sure, :m] != exp[sure, :m], axis=1))[0]
    assert bad.size == 0, f"{bad.size} tokens with other candidates"
    for t in np.nonzero(~sure)[0]:
        c = cand_gpu[t, :m]
        assert len(set(c.tolist())) == m and not set(c.tolist()) & set(idx_gpu[t].tolist())
        sc = s2[t, c]
        assert np.all(np.diff(sc) <= NEAR_TIE)
        rest = np.delete(s2[t], np.concatenate([idx_gpu[t], c]))
        assert rest.size == 0 or sc.min() >= rest.max() - NEAR_TIE
    return ~sure


# Share of output elements that may need the bf16-rounding allowance at full size before
# the test fails: a midpoint flip of h moves y by about one bf16 step of h times a down
# weight, so only a handful of elements in a million should need it.
MAX_ALLOWANCE_SHARE = 1e-4


def check_full_layer(y_gpu, inp, groups, T, d, w, slot, h_bf16, out_bf16, H_gpu,
                     n_rows, shared_row0=None, what=""):
    """Every output row of a full-size layer against the oracle.

    groups: (e, lo, hi, tokens) per expert: rows [lo, hi) of H / Yp hold expert e's
    outputs for `tokens`.  w [T, K] and slot [T, K] are the combine's weights and rows
    (-1: no contribution).  The oracle's Y is expert_ffn per group (float64 sums), and
    y_ref = oracle.combine(T, d, w, slot, Y, shared), as in oracle.forward.

    Rule: max|y - y_ref| <= 2e-2 max|y_ref| outright; per element <= 5e-2 relative
    where |y_ref| > 1e-3 max|y_ref|, except where validated bf16 roundings of h (every
    GPU h in [lo, hi) must be the RNE bf16 of a value within the fp32 error bound of the
    oracle's h) explain the difference:
        allow = sum_j |w_j| (|W_down| |H - hq| + 4 sqrt(F) 2^-24 |W_down| |hq|)  (+ 2^-8 |y_ref|
    for a bf16 output).  Returns (elements needing the allowance, h values on the other
    side of a midpoint); fails when more than MAX_ALLOWANCE_SHARE of the elements need it.
    """
    x = np32(inp["x"])
    Y = np.zeros((n_rows, d), np.float32)
    A = np.zeros((n_rows, d), np.float64)
    flips = 0
    for e, lo, hi, tok in groups:
        if hi == lo:
            continue
        Wg, Wu, Wd = oracle.expert_weights(inp, e)
        xr = x[tok]
        o, parts = oracle.expert_ffn(xr, Wg, Wu, Wd, h_bf16, return_h=True)
        Y[lo:hi] = o
        Wda = np.abs(np.asarray(Wd, np.float64))
        if h_bf16:
            Hg = np.asarray(H_gpu[lo:hi], np.float64)
            _check_h_only(Hg, parts, xr, Wg, Wu, f"{what} expert {e}")
            hq = oracle.bf16_round(parts["h"].astype(np.float32)).astype(np.float64)
            dq = np.abs(Hg - hq)
            flips += int(np.count_nonzero(dq))
            F = Wda.shape[1]
            A[lo:hi] = dq @ Wda.T + 4.0 * np.sqrt(F) * 2.0 ** -24 * (np.abs(hq) @ Wda.T)
        else:
            A[lo:hi] = 1e-6 * (np.abs(parts["h"]) @ Wda.T)
        del parts
    shared = None
    if shared_row0 is not None:
        # the shared expert's rows follow the routed ones, token order, weight 1
        Ysh = Y[shared_row0:shared_row0 + T]
        shared = Ysh.copy()
    y_ref = oracle.combine(T, d, w, slot, Y, shared)
    K = w.shape[1]
    sp = np.asarray(slot).reshape(T, K)
    allow = np.zeros((T, d), np.float64)
    for j in range(K):
        rows = np.nonzero(sp[:, j] >= 0)[0]
        allow[rows] += np.abs(w[rows, j].astype(np.float64))[:, None] * A[sp[rows, j]]
    if shared_row0 is not None:
        allow += A[shared_row0:shared_row0 + T]
    y = np.asarray(y_gpu, np.float64)
    y_ref = y_ref.astype(np.float64)
    assert y.shape == y_ref.shape
    assert np.all(np.isfinite(y)), what
    m = np.abs(y_ref).max()
    err = np.abs(y - y_ref)
    assert err.max() <= Y_MAX_REL * m, f"{what}: max err {err.max():.3e} > {Y_MAX_REL} * {m:.3e}"
    if out_bf16:
        allow += 2.0 ** -8 * np.abs(y_ref)
    mask = np.abs(y_ref) > Y_FLOOR * m
    rel = np.where(mask, err / np.where(mask, np.abs(y_ref), 1.0), 0.0)
    strict_bad = mask & (rel > Y_ELEM_REL)
    unexplained = strict_bad & (err > allow)
    assert not unexplained.any(), (
        f"{what}: {unexplained.sum()} elements over {Y_ELEM_REL} relative error not explained "
        f"by validated bf16 roundings of h (worst rel {rel[unexplained].max():.3e})")
    nb = int(strict_bad.sum())
    assert nb <= MAX_ALLOWANCE_SHARE * y.size, f"{what}: {nb} elements needed the allowance"
    if h_bf16:
        nh = sum((hi - lo) for _, lo, hi, _ in groups) * np.asarray(H_gpu).shape[1]
        assert flips <= 1e-2 * max(nh, 1), f"{what}: {flips} of {nh} h values differ"
    return nb, flips


def token_choice_groups(offsets, perm_src, k, E, n_shared, T):
    """(e, lo, hi, tokens) of the token-choice rows: expert e's rows [offsets[e],
    offsets[e+1]) take tokens perm_src // k; the shared expert's T rows start at T k."""
    groups = []
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        groups.append((e, lo, hi, np.asarray(perm_src[lo:hi], np.int64) // k))
    if n_shared:
        groups.append((E, T * k, T * k + T, np.arange(T)))
    return groups
