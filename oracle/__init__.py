"""CPU oracle (test infrastructure only; never imported by the library).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg use this package.
"""
from . import brute, moe_oracle

__all__ = ["brute", "moe_oracle"]
