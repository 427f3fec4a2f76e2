"""Which workgroup-to-XCD mapping the grouped GEMMs take at each full-size workload.

The GEMM kernel deals units to the XCDs in chunks when the routing is skewed:
max tiles of one expert * active experts > 2 * tiles of the pass, computed on
the device from the tile map.  This test evaluates that rule on the oracle's
tile map, so it states which full-size GPU parity tests run the chunked
mapping (the Zipf 1.2 and 2.0 workloads) and which run contiguous ranges.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import get_workload, make_inputs

BM = {"mixtral_t512": 160, "e64_zipf_a0.0": 192, "e64_zipf_a1.2": 192, "e64_zipf_a2.0": 192,
      "capacity_gini0.10": 192, "mixtral_t4096": 384}


def skewed(tile_off):
    t = np.diff(np.asarray(tile_off, dtype=np.int64))
    return int(t.max()) * int((t > 0).sum()) > 2 * int(t.sum())


@pytest.mark.parametrize("name,expect", [
    ("mixtral_t512", [False]),
    ("e64_zipf_a0.0", [False]),
    ("e64_zipf_a1.2", [True]),
    ("e64_zipf_a2.0", [True]),
    ("capacity_gini0.10", [False, False]),
])
def test_mapping_per_workload(name, expect):
    wl = get_workload(name)
    inp = make_inputs(wl, 0, experts=False)
    if inp.topk_ids is not None:
        ids = inp.topk_ids
    else:
        ids, _, _ = O.route(inp.x, inp.wr, wl.k, wl.dtype, inp.bias)
    disp = O.dispatch(ids, wl.E, wl.capacity, BM[name])
    got = [skewed(disp["tile_off"][p]) for p in range(len(expect))]
    assert got == expect
