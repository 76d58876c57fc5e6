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
