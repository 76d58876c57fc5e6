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
          + 4.0 * 2.0 ** -24 * np.abs(h64))
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
