"""CPU checks of the seeded input generators (no GPU)."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import WORKLOADS, bf16_bits_from_f32, f32_from_bf16_bits, get_workload, make_inputs, zipf_routing


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.0e38, -1e-40], np.float32)])
    ours = bf16_bits_from_f32(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(f32_from_bf16_bits(ours), torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic_and_seeded():
    wl = get_workload("tiny_f32")
    a, b, c = make_inputs(wl, 0), make_inputs(wl, 0), make_inputs(wl, 1)
    for n in ("x", "wr", "wg", "wu", "wd"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
        assert not np.array_equal(getattr(a, n), getattr(c, n))
    assert a.x.dtype == np.float32 and a.wg.shape == (8, 256, 128) and a.wd.shape == (8, 128, 256)
    # std of N(0, 1/d) draws
    assert abs(a.wg.std() * np.sqrt(128) - 1) < 0.02


def test_bf16_workload_draws():
    wl = get_workload("e64_zipf_a1.2", T=64, d=64, F=32)
    inp = make_inputs(wl, 0)
    assert inp.x.dtype == np.uint16 and inp.wg.dtype == np.uint16
    assert abs(f32_from_bf16_bits(inp.wg).std() / 0.02 - 1) < 0.05
    assert inp.topk_ids.shape == (64, 8) and inp.topk_w.dtype == np.float32


def test_zipf_routing_properties():
    for a in (0.0, 1.2, 2.0):
        ids, w = zipf_routing(512, 64, 8, a, 0)
        assert all(len(set(r)) == 8 for r in ids.tolist())
        assert ids.min() >= 0 and ids.max() < 64
        np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-6)
    counts = [np.bincount(zipf_routing(512, 64, 8, a, 0)[0].ravel(), minlength=64) for a in (0.0, 1.2, 2.0)]
    g = [O.gini(c) for c in counts]
    assert g[0] < 0.15 < g[1] < g[2]
    # alpha = 2: the top-ranked expert is chosen by (almost) every token
    assert counts[2].max() >= 500


@pytest.mark.parametrize("target", [0.10, 0.30])
def test_capacity_bias_reaches_gini_target(target):
    wl = WORKLOADS[f"capacity_gini{target:.2f}"]
    inp = make_inputs(wl, 0, experts=False)
    ids, _, _ = O.route(inp.x, inp.wr, wl.k, wl.dtype, inp.bias)
    g = O.gini(np.bincount(ids.ravel(), minlength=wl.E))
    assert abs(g - target) <= 0.005
    d = O.dispatch(ids, wl.E, wl.capacity, 64)
    assert d["spill_counts"].sum() > 0
