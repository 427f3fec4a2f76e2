"""The MoE-layer workloads, as data.

Shapes and distributions follow the problem statement of the TritonMoE review
(pith.science verdict for arXiv 2605.23911: Mixtral-8x7B and 64-expert
configurations, the Zipfian skew study of its section 4.7) and the capacity
setting of the Cap-and-Spill critique (juhe.plus, section "Cap-and-Spill").
The routing-skew targets (count Gini about 0.10 and 0.30) are the two Gini
bands reported in the DODOCO abstract (fugumt.com summary of arXiv
2605.20982).

Distribution notation: "std" is the standard deviation of a normal draw.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    dtype: str  # "f32" or "bf16"
    x_std: float
    wr_std: float
    w_std: float
    routing: str  # "router" (x.Wr^T), "router_bias" (+ lognormal bias), "zipf"
    capacity: int = 0
    zipf_alpha: Optional[float] = None
    gini_target: Optional[float] = None
    bias_sigma: Optional[float] = None
    weights: str = "dtype"  # expert weights: "dtype" (as x), or "e4m3" (OCP E4M3 codes + per-row fp32 scales)

    @property
    def rows(self) -> int:
        return self.T * self.k

    def flops(self) -> float:
        """Algorithmic FLOPs of the two grouped GEMMs: 2 * (T*k) * 3 * d * F."""
        return 2.0 * self.T * self.k * 3.0 * self.d * self.F


# Lognormal per-expert logit bias scale (b_e = exp(sigma * z_e)) for the
# capacity workloads, found by bisection so the count Gini under the oracle's
# routing hits the target at seed 0.  Written by oracle/calibrate_bias.py; the
# test suite re-checks the realised Gini with the oracle.
CAPACITY_BIAS_SIGMA = {0.10: 0.074219, 0.30: 0.238281}


def _mixtral(T: int, name: str, weights: str = "dtype") -> Workload:
    return Workload(name=name, T=T, d=4096, E=8, k=2, F=14336, dtype="bf16",
                    x_std=1.0, wr_std=0.02, w_std=0.02, routing="router", weights=weights)


def _build() -> Dict[str, Workload]:
    w: Dict[str, Workload] = {}
    tiny = Workload(name="tiny_f32", T=64, d=128, E=8, k=2, F=256, dtype="f32",
                    x_std=1.0, wr_std=1.0 / math.sqrt(128), w_std=1.0 / math.sqrt(128),
                    routing="router")
    w[tiny.name] = tiny
    w["mixtral_t512"] = _mixtral(512, "mixtral_t512")
    for a in (0.0, 1.2, 2.0):
        n = f"e64_zipf_a{a:.1f}"
        w[n] = Workload(name=n, T=512, d=3584, E=64, k=8, F=2560, dtype="bf16",
                        x_std=1.0, wr_std=0.02, w_std=0.02, routing="zipf", zipf_alpha=a)
    for T in (1, 8, 32, 128, 256):
        n = f"mixtral_decode_t{T}"
        w[n] = _mixtral(T, n)
    for g in (0.10, 0.30):
        n = f"capacity_gini{g:.2f}"
        w[n] = Workload(name=n, T=4096, d=2048, E=64, k=6, F=1408, dtype="bf16",
                        x_std=1.0, wr_std=0.02, w_std=0.02, routing="router_bias",
                        capacity=384, gini_target=g, bias_sigma=CAPACITY_BIAS_SIGMA[g])
    # Compute-bound point at the Mixtral shape (at least 512 rows per expert).
    w["mixtral_t4096"] = _mixtral(4096, "mixtral_t4096")
    # fp8 expert weights (E4M3 codes, one fp32 scale per output channel) at the
    # Mixtral layer and decode sizes; the same fp32 draws as the bf16 workloads.
    for T in (512, 1, 8, 32, 128, 256):
        n = f"mixtral_t{T}_fp8" if T == 512 else f"mixtral_decode_t{T}_fp8"
        w[n] = _mixtral(T, n, weights="e4m3")
    return w


WORKLOADS: Dict[str, Workload] = _build()


def get_workload(name: str, **overrides) -> Workload:
    base = WORKLOADS[name]
    return dataclasses.replace(base, **overrides) if overrides else base
