"""Find the lognormal logit-bias scale of the capacity workloads (test infrastructure).

The capacity workloads add b_e = exp(sigma * z_e), z_e ~ N(0, 1), to every
token's router logits so that the per-expert counts reach a chosen routing
Gini: the two bands (about 0.10 and about 0.30) of the DODOCO abstract
(fugumt.com summary of arXiv 2605.20982).  This script bisects sigma with
the oracle's routing at seed 0 and prints the values stored in
workloads/configs.py (CAPACITY_BIAS_SIGMA).  Only the oracle is called.

    python -m oracle.calibrate_bias
"""
from __future__ import annotations

import dataclasses
import json
import sys

import numpy as np

from oracle import moe_oracle as O


def realised_gini(base_logits: np.ndarray, z: np.ndarray, sigma: float, k: int) -> float:
    lg = base_logits + np.exp(sigma * z).astype(np.float32).astype(np.float64)[None, :]
    ids, _ = O.route_from_logits(lg, k)
    return O.gini(np.bincount(ids.ravel(), minlength=z.size))


def calibrate(target: float, seed: int = 0, tol: float = 0.002):
    from workloads import get_workload, make_inputs
    wl = get_workload(f"capacity_gini{target:.2f}", bias_sigma=1.0)
    inp = make_inputs(wl, seed, experts=False)
    # the bias is exp(sigma * z); recover z from the sigma = 1 draw
    z = np.log(inp.bias.astype(np.float64))
    base = O.router_logits(inp.x, inp.wr, wl.dtype)
    lo, hi = 0.0, 4.0
    g = realised_gini(base, z, hi, wl.k)
    if g < target:
        raise RuntimeError("target Gini not reachable")
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        g = realised_gini(base, z, mid, wl.k)
        if abs(g - target) <= tol:
            return round(mid, 6), g
        if g < target:
            lo = mid
        else:
            hi = mid
    return round(0.5 * (lo + hi), 6), g


def main(argv=None):
    out = {}
    for target in (0.10, 0.30):
        s, g = calibrate(target)
        out[f"{target:.2f}"] = {"sigma": s, "gini": g}
    json.dump(out, sys.stdout, indent=1)
    print()


if __name__ == "__main__":
    main()
