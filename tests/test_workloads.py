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


def test_e4m3_encoder_round_trip_and_ties():
    from oracle import moe_oracle as O
    from workloads import gen
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_to_f64(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(gen.e4m3_codes_from_f32(vals[fin].astype(np.float32)), codes[fin])
    pos = vals[:0x7F]
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact in fp32
    even = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    assert np.array_equal(gen.e4m3_codes_from_f32(mid), even)
    assert np.array_equal(gen.e4m3_codes_from_f32(-mid), even | 0x80)
    assert gen.e4m3_codes_from_f32(np.array([470.0, -1e9], np.float32)).tolist() == [0x7E, 0xFE]


def test_e4m3_encoder_matches_torch():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    from workloads import gen
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(200000) * rng.choice([1e-3, 0.05, 1.0, 60.0], 200000)).astype(np.float32)
    v = np.clip(v, -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(gen.e4m3_codes_from_f32(v), ref)


def test_fp8_workload_inputs():
    from oracle import moe_oracle as O
    wl = get_workload("mixtral_decode_t1_fp8")
    assert wl.weights == "e4m3" and wl.dtype == "bf16"
    # a small slice of the quantiser's contract on one expert row block
    from workloads import gen
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    c, s = gen.quantize_rows_e4m3(w, block=16)
    deq = s.astype(np.float64)[:, None] * O.e4m3_to_f64(c)
    assert np.abs(c.view(np.int8)).max() <= 0x7E                  # no NaN codes
    assert (np.abs(deq).max(axis=1) == s.astype(np.float64) * 448).all()  # row max maps to 448
    # nearest rounding: within half a spacing, 2^-4 of the value in the normal
    # range and 2^-10 of the scale (half the subnormal step 2^-9) below it
    bound = 2.0 ** -4 * np.abs(w).astype(np.float64) + 2.0 ** -10 * s.astype(np.float64)[:, None]
    assert (np.abs(deq - w) <= bound * (1 + 1e-6)).all()
