"""Calibrate per-expert router row scales for the skewed synthetic workloads.

The router weight rows are drawn as N(0, s_e^2 / d).  With x ~ N(0, 1) the logit of
expert e for one token is then close to N(0, s_e^2), independently across experts, so
an expert with a larger scale lands in the top-k more often.  This script picks the
scales by simulation on Gaussian logits only (it never touches the layer itself) and
writes them to ``row_scales.json`` beside this file.

* Mixtral-shaped prefill (8 experts, top-2): s_e = 1 + beta * e / 7, beta chosen so the
  largest / smallest expert load is about 3 : 1.
* Switch-shaped capacity layer (64 experts, top-1): loads follow a Zipf law with
  exponent 1.1 over the experts, share_e proportional to (e + 1)^-1.1; the scales are
  found by a fixed number of multiplicative updates toward those shares.

Run:  python gen/calibrate.py
"""
import json
import os

import numpy as np


def _shares(rng, scales, k, n):
    z = rng.standard_normal((n, len(scales))) * scales
    top = np.argpartition(-z, k - 1, axis=1)[:, :k]
    c = np.bincount(top.ravel(), minlength=len(scales)).astype(np.float64)
    return c / c.sum()


def calibrate_prefill(rng, E=8, k=2, target=3.0):
    lo, hi = 1.0, 6.0
    for _ in range(24):
        beta = 0.5 * (lo + hi)
        sh = _shares(rng, 1.0 + beta * np.arange(E) / (E - 1), k, 200_000)
        if sh.max() / sh.min() < target:
            lo = beta
        else:
            hi = beta
    beta = round(0.5 * (lo + hi), 3)
    return (1.0 + beta * np.arange(E) / (E - 1)).tolist(), beta


def calibrate_zipf(rng, E=64, k=1, s=1.1, iters=80):
    pi = (np.arange(E) + 1.0) ** -s
    pi /= pi.sum()
    scales = np.ones(E)
    for _ in range(iters):
        sh = _shares(rng, scales, k, 400_000)
        scales *= (pi / np.maximum(sh, 1e-7)) ** 0.3
    return [round(float(v), 4) for v in scales]


def main():
    rng = np.random.default_rng(20261203)
    prefill, beta = calibrate_prefill(rng)
    zipf = calibrate_zipf(rng)
    out = {
        "mixtral_prefill": {"beta": beta, "scales": [round(v, 4) for v in prefill]},
        "switch_capacity": {"zipf_s": 1.1, "scales": zipf},
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "row_scales.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print("wrote", path, "beta =", beta)


if __name__ == "__main__":
    main()
