"""Pins of the CPU oracle against things other than itself.

Closed forms and textbook values (tests/golden/worked_examples.json), special
cases that reduce to a library routine, invariants of the definition, and a
scalar brute-force re-implementation on tiny inputs.  Each test is chosen so
that a plausible slip in the oracle (a dropped term, a wrong sign, index or
tie-break, gate and up swapped, an unstable order, a mis-sized spill region)
fails it.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import brute
from oracle import moe_oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _f32(a):
    return np.asarray(a, dtype=np.float32)


# ---------------------------------------------------------------- routing ---

def test_routing_golden_softmax_top2():
    g = GOLDEN["routing_softmax_top2"]
    ids, w, lg = O.route(_f32(g["x"]), _f32(g["wr"]), g["k"], "f32")
    assert ids.tolist() == g["ids"]
    np.testing.assert_allclose(w, g["w"], rtol=0, atol=1e-15)
    # k = E returns the full softmax in logit order
    _, wall = O.route_from_logits(lg, 3)
    np.testing.assert_allclose(wall[0], g["softmax"], rtol=0, atol=1e-15)


def test_routing_golden_tie():
    g = GOLDEN["routing_tie_lowest_index"]
    ids, w, _ = O.route(_f32(g["x"]), _f32(g["wr"]), g["k"], "f32")
    assert ids.tolist() == g["ids"]
    assert w.tolist() == g["w"]


def test_routing_zero_router_gives_first_k_uniform():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 16)).astype(np.float32)
    for E, k in [(8, 2), (5, 5), (64, 8)]:
        ids, w, _ = O.route(x, np.zeros((E, 16), np.float32), k, "f32")
        assert (ids == np.arange(k)[None, :]).all()
        assert (w == 1.0 / k).all() or np.abs(w - 1.0 / k).max() == 0.0


def test_routing_k1_weight_is_one():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((50, 9))
    ids, w = O.route_from_logits(lg, 1)
    assert (w == 1.0).all()
    assert (ids[:, 0] == lg.argmax(axis=1)).all()


def test_routing_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((40, 6)) * 3
    ids, w = O.route_from_logits(lg, 6)
    ref = scipy.special.softmax(lg, axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids, axis=1), rtol=1e-13, atol=0)
    assert (np.diff(np.take_along_axis(lg, ids, axis=1), axis=1) <= 0).all()


def test_routing_brute_force_subsets():
    rng = np.random.default_rng(4)
    for E in range(1, 9):
        for k in range(1, E + 1):
            lg = np.round(rng.standard_normal((20, E)) * 4) / 4  # coarse grid makes ties
            ids, w = O.route_from_logits(lg, k)
            for t in range(lg.shape[0]):
                best = max(itertools.combinations(range(E), k),
                           key=lambda s: (sum(lg[t, list(s)]), [-i for i in s]))
                assert sorted(ids[t].tolist()) == sorted(best) or \
                    math.isclose(sum(lg[t, ids[t]]), sum(lg[t, list(best)]))
                chosen = set(ids[t].tolist())
                rest = [e for e in range(E) if e not in chosen]
                if rest:
                    assert lg[t, list(chosen)].min() >= lg[t, rest].max()
                # among equal logits, the lower index is chosen first
                for e in rest:
                    for c in chosen:
                        if lg[t, e] == lg[t, c]:
                            assert c < e


def test_routing_invariants_and_shift():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((100, 64)) * 2
    ids, w = O.route_from_logits(lg, 8)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-12)
    assert (np.diff(w, axis=1) <= 1e-15).all()
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert ids.min() >= 0 and ids.max() < 64
    ids2, w2 = O.route_from_logits(lg + 123.0, 8)
    assert (ids2 == ids).all()
    np.testing.assert_allclose(w2, w, rtol=1e-12)


def test_routing_matches_brute():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((9, 5)).astype(np.float32)
    wr = rng.standard_normal((6, 5)).astype(np.float32)
    bias = rng.standard_normal(6).astype(np.float32)
    ids, w, _ = O.route(x, wr, 3, "f32", bias)
    bids, bw = brute.route(x.astype(np.float64), wr.astype(np.float64), 3, bias.astype(np.float64))
    assert ids.tolist() == bids
    np.testing.assert_allclose(w, bw, rtol=1e-12)


def test_topk_gap():
    lg = np.array([[3.0, 1.0, 2.0, 0.5]])
    assert O.topk_gap(lg, 2)[0] == 1.0
    assert O.topk_gap(lg, 4)[0] == np.inf


# --------------------------------------------------------- count and scan ---

def _check_dispatch_golden(d, g):
    for key in ("counts", "offsets", "row_of", "token_of", "spill_counts", "spill_offsets"):
        if key in g:
            assert d[key].tolist() == g[key], key
    for p in (0, 1):
        if f"tile_map_pass{p}" in g:
            assert d["tile_map"][p].tolist() == g[f"tile_map_pass{p}"]
            assert d["tile_off"][p].tolist() == g[f"tile_off_pass{p}"]


def test_dispatch_golden():
    g = GOLDEN["dispatch_small"]
    ids = np.array(g["ids"])
    d = O.dispatch(ids, g["E"], 0, g["tile_rows"])
    _check_dispatch_golden(d, g["uncapped"])
    c = g["capacity2"]
    d = O.dispatch(ids, g["E"], c["capacity"], g["tile_rows"])
    assert d["R"] == c["R"]
    _check_dispatch_golden(d, c)


def test_counts_closed_form_round_robin():
    for T, k, E in [(64, 2, 8), (512, 8, 64), (96, 6, 16)]:
        ids = (np.arange(T)[:, None] + np.arange(k)[None, :]) % E
        d = O.dispatch(ids, E)
        assert (d["counts"] == T * k // E).all()
        assert (d["offsets"] == np.arange(E + 1) * (T * k // E)).all()


def test_counts_vs_bincount():
    rng = np.random.default_rng(7)
    ids = rng.integers(0, 37, size=(300, 5))
    d = O.dispatch(ids, 37)
    assert (d["counts"] == np.bincount(ids.ravel(), minlength=37)).all()
    assert d["offsets"][0] == 0 and d["offsets"][-1] == ids.size
    assert (np.diff(d["offsets"]) == d["counts"]).all()


def _perm_invariants(d, ids, k, C):
    flat = np.asarray(ids).ravel()
    Tk = flat.size
    ro, to = d["row_of"], d["token_of"]
    assert len(set(ro.tolist())) == Tk                      # injective
    assert ((to >= 0).sum()) == Tk                          # live rows = T*k
    assert (to[ro] == np.arange(Tk) // k).all()
    # within each expert block of each pass, tokens ascend
    for p in (0, 1):
        for e in range(len(d["counts"])):
            b, n = d["pass_base"][p][e], d["pass_rows"][p][e]
            toks = to[b:b + n]
            assert (toks >= 0).all()
            assert (np.diff(toks) >= 0).all()
    assert d["kept_counts"].sum() + d["spill_counts"].sum() == Tk   # nothing dropped
    if C > 0:
        assert d["spill_counts"].sum() <= O.spill_rows_bound(len(ids), k, C)


def test_dispatch_exhaustive_tiny_vs_brute():
    for T in (1, 2, 3):
        for k in (1, 2):
            for E in (1, 2, 3):
                for assign in itertools.product(range(E), repeat=T * k):
                    ids = np.array(assign).reshape(T, k)
                    for C in (0, 1, 2):
                        for BM in (1, 2, 3):
                            d = O.dispatch(ids, E, C, BM)
                            b = brute.dispatch(ids.tolist(), E, C, BM)
                            for key in ("counts", "offsets", "spill_counts", "spill_offsets",
                                        "rank", "row_of", "token_of"):
                                assert d[key].tolist() == b[key], (key, ids, C, BM)
                            assert d["R"] == b["R"]
                            for p in (0, 1):
                                assert d["tile_map"][p].tolist() == [list(x) for x in b["tile_map"][p]]
                                assert d["tile_off"][p].tolist() == b["tile_off"][p]
                                assert d["n_tiles"][p] <= O.max_tiles(T, k, E, C, BM, p)
                            _perm_invariants(d, ids, k, C)


def test_dispatch_random_invariants_and_tile_bound():
    rng = np.random.default_rng(8)
    for trial in range(40):
        T = int(rng.integers(1, 300))
        E = int(rng.integers(1, 70))
        k = int(rng.integers(1, min(E, 8) + 1))
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        C = int(rng.choice([0, 1, 3, 17, T * k]))
        BM = int(rng.choice([1, 16, 32, 64, 128]))
        d = O.dispatch(ids, E, C, BM)
        _perm_invariants(d, ids, k, C)
        for p in (0, 1):
            assert d["n_tiles"][p] <= O.max_tiles(T, k, E, C, BM, p)
            tm = d["tile_map"][p]
            if len(tm):
                assert (tm[:, 2] >= 1).all() and (tm[:, 2] <= BM).all()
            # tiles cover exactly the rows of the pass
            covered = sum(int(r) for r in tm[:, 2]) if len(tm) else 0
            assert covered == d["pass_rows"][p].sum()


def test_gather_is_bitwise_copy():
    rng = np.random.default_rng(9)
    x = rng.integers(0, 2**16, size=(20, 8), dtype=np.uint16)
    ids = np.stack([rng.permutation(5)[:2] for _ in range(20)])
    for C in (0, 3):
        d = O.dispatch(ids, 5, C)
        xp = O.gather(x, d)
        f = np.arange(40)
        assert (xp[d["row_of"][f]] == x[f // 2]).all()
        assert (xp[d["token_of"] < 0] == 0).all()


# ------------------------------------------------------- capacity / spill ---

def test_capacity_adversarial_all_to_one_expert():
    T, k, E, C = 100, 3, 8, 10
    ids = np.stack([[0] + list(np.random.default_rng(t).permutation(np.arange(1, E))[:k - 1])
                    for t in range(T)])
    d = O.dispatch(ids, E, C, 16)
    assert d["spill_counts"][0] == T - C
    _perm_invariants(d, ids, k, C)
    # worst case over any distinct-per-token ids stays within the reserved rows
    assert d["spill_counts"].sum() <= O.spill_rows_bound(T, k, C)


def test_capacity_spill_bound_is_attained():
    # one expert takes every entry (duplicates allowed): overflow = T*k - C exactly
    T, k, E, C = 10, 2, 4, 3
    ids = np.zeros((T, k), dtype=np.int64)
    d = O.dispatch(ids, E, C, 4)
    assert d["spill_counts"].sum() == O.spill_rows_bound(T, k, C) == T * k - C


def test_capacity_large_c_has_empty_spill():
    rng = np.random.default_rng(10)
    ids = np.stack([rng.permutation(16)[:4] for _ in range(64)])
    d0 = O.dispatch(ids, 16, 0, 8)
    C = int(d0["counts"].max())
    d = O.dispatch(ids, 16, C, 8)
    assert d["spill_counts"].sum() == 0 and d["n_tiles"][1] == 0
    assert (d["kept_counts"] == d0["counts"]).all()


# ------------------------------------------------------------- expert FFN ---

def test_swiglu_golden_gate_not_up():
    g = GOLDEN["swiglu_gate_vs_up"]
    y = O.swiglu_ffn(np.array(g["x"]), np.array(g["wg"][0]), np.array(g["wu"][0]), np.array(g["wd"][0]))
    assert abs(y[0, 0] - g["y"]) < 1e-15
    assert abs(y[0, 0] - g["y_if_gate_and_up_swapped"]) > 0.1


def test_silu_matches_library_logistic():
    z = np.linspace(-60, 60, 2001)
    np.testing.assert_allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0


def _tiny_inputs(rng, T, d, E, F):
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    wg = (rng.standard_normal((E, F, d)) / np.sqrt(d)).astype(np.float32)
    wu = (rng.standard_normal((E, F, d)) / np.sqrt(d)).astype(np.float32)
    wd = (rng.standard_normal((E, d, F)) / np.sqrt(F)).astype(np.float32)
    return x, wr, wg, wu, wd


def test_dense_mlp_reduction_E1_k1():
    rng = np.random.default_rng(11)
    x, wr, wg, wu, wd = _tiny_inputs(rng, 5, 6, 1, 7)
    r = O.forward(x, wr, wg, wu, wd, 1, "f32")
    assert (r["w"] == 1.0).all()
    for t in range(5):
        y = brute.expert(x[t].astype(np.float64), wg[0].astype(np.float64),
                         wu[0].astype(np.float64), wd[0].astype(np.float64))
        np.testing.assert_allclose(r["out"][t], y, rtol=1e-12, atol=1e-14)


def test_zero_gate_or_up_gives_zero_and_down_scales():
    rng = np.random.default_rng(12)
    x, wr, wg, wu, wd = _tiny_inputs(rng, 12, 8, 4, 16)
    r0 = O.forward(x, wr, np.zeros_like(wg), wu, wd, 2, "f32")
    assert (r0["out"] == 0).all()
    r1 = O.forward(x, wr, wg, np.zeros_like(wu), wd, 2, "f32")
    assert (r1["out"] == 0).all()
    r = O.forward(x, wr, wg, wu, wd, 2, "f32")
    r2 = O.forward(x, wr, wg, wu, 2 * wd, 2, "f32")
    assert (r2["out"] == 2 * r["out"]).all()


def test_token_permutation_equivariance():
    rng = np.random.default_rng(13)
    x, wr, wg, wu, wd = _tiny_inputs(rng, 30, 8, 5, 12)
    r = O.forward(x, wr, wg, wu, wd, 2, "f32")
    p = rng.permutation(30)
    rp = O.forward(x[p], wr, wg, wu, wd, 2, "f32")
    np.testing.assert_allclose(rp["out"], r["out"][p], rtol=1e-12, atol=1e-14)


def test_identity_experts_return_input():
    # permute -> (identity expert) -> combine with renormalised weights gives x back
    rng = np.random.default_rng(14)
    x = rng.standard_normal((40, 10))
    lg = rng.standard_normal((40, 6))
    ids, w = O.route_from_logits(lg, 3)
    for C in (0, 5):
        d = O.dispatch(ids, 6, C)
        y = O.gather(x, d)
        out = O.combine(y, w, d["row_of"])
        np.testing.assert_allclose(out, x, rtol=1e-14, atol=1e-14)


def test_combine_k1_is_exact_row():
    rng = np.random.default_rng(15)
    y = rng.standard_normal((9, 4))
    row_of = rng.permutation(9)
    out = O.combine(y, np.ones((9, 1)), row_of)
    assert (out == y[row_of]).all()


# ------------------------------------------------------------ whole layer ---

@pytest.mark.parametrize("C", [0, 2, 5])
def test_forward_matches_brute(C):
    rng = np.random.default_rng(16 + C)
    x, wr, wg, wu, wd = _tiny_inputs(rng, 9, 6, 4, 5)
    bias = rng.standard_normal(4).astype(np.float32)
    r = O.forward(x, wr, wg, wu, wd, 2, "f32", bias=bias, capacity=C, tile_rows=2)
    b = brute.forward(x.astype(np.float64), wr.astype(np.float64), wg.astype(np.float64),
                      wu.astype(np.float64), wd.astype(np.float64), 2,
                      bias=bias.astype(np.float64), capacity=C, tile_rows=2)
    assert r["ids"].tolist() == b["ids"]
    np.testing.assert_allclose(r["out"], b["out"], rtol=1e-11, atol=1e-13)
    assert r["disp"]["row_of"].tolist() == b["disp"]["row_of"]


def test_spill_output_equals_uncapped_bitwise():
    rng = np.random.default_rng(20)
    x, wr, wg, wu, wd = _tiny_inputs(rng, 64, 16, 8, 24)
    r0 = O.forward(x, wr, wg, wu, wd, 2, "f32")
    for C in (1, 4, 9, 16):
        rc = O.forward(x, wr, wg, wu, wd, 2, "f32", capacity=C)
        assert (rc["out"] == r0["out"]).all()
        assert rc["disp"]["spill_counts"].sum() > 0 or C >= r0["disp"]["counts"].max()


def test_forward_tokens_matches_forward():
    rng = np.random.default_rng(21)
    x, wr, wg, wu, wd = _tiny_inputs(rng, 20, 8, 6, 10)
    r = O.forward(x, wr, wg, wu, wd, 3, "f32")
    toks = [0, 7, 19, 3]
    o = O.forward_tokens(x, wg, wu, wd, "f32", r["ids"], r["w"], toks)
    np.testing.assert_allclose(o, r["out"][toks], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("C", [0, 3])
def test_expert_rows_match_brute(C):
    # every live row of each expert, in stable order, with h and y of its token
    rng = np.random.default_rng(22 + C)
    x, wr, wg, wu, wd = _tiny_inputs(rng, 11, 6, 4, 5)
    r = O.forward(x, wr, wg, wu, wd, 2, "f32", capacity=C)
    disp = r["disp"]
    flat = r["ids"].reshape(-1)
    for e in range(4):
        rows, h, y = O.expert_rows(x, wg, wu, wd, "f32", disp, e)
        fs = [f for f in range(flat.size) if flat[f] == e]          # ascending f: the stable order
        assert rows.tolist() == [int(disp["row_of"][f]) for f in fs]
        for i, f in enumerate(fs):
            xr = x[f // 2].astype(np.float64)
            hb = brute.hidden(xr, wg[e].astype(np.float64), wu[e].astype(np.float64))
            yb = brute.expert(xr, wg[e].astype(np.float64), wu[e].astype(np.float64), wd[e].astype(np.float64))
            np.testing.assert_allclose(h[i], hb, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(y[i], yb, rtol=1e-11, atol=1e-13)
            np.testing.assert_array_equal(y[i], r["y"][rows[i]])


def test_bf16_decode_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(0, 2**16, 7, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]   # finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(O.to_f64(bits, "bf16"), ref)


def test_gini_closed_forms():
    assert O.gini(np.full(8, 5)) == 0.0
    E = 10
    assert abs(O.gini(np.array([7] + [0] * (E - 1))) - (E - 1) / E) < 1e-15
    # two-level: half the experts at a, half at b: G = (b-a) / (2 (a+b))
    a, b = 1.0, 3.0
    assert abs(O.gini(np.array([a] * 4 + [b] * 4)) - (b - a) / (2 * (a + b))) < 1e-15


# ----------------------------------------------------------------------------
# fp8 (OCP E4M3) expert weights
# ----------------------------------------------------------------------------

def test_e4m3_decode_format_values():
    # values fixed by the OCP 8-bit floating point definition (E4M3, bias 7)
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
            0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
            0xB8: -1.0, 0xFE: -448.0}
    got = O.e4m3_to_f64(np.array(list(want), dtype=np.uint8))
    assert got.tolist() == list(want.values())
    assert np.signbit(O.e4m3_to_f64(np.array([0x80], np.uint8)))[0]
    assert np.isnan(O.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()
    pos = O.e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8))
    assert (np.diff(pos) > 0).all()                      # positive codes are ordered
    neg = O.e4m3_to_f64(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def test_e4m3_decode_matches_torch():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_to_f64(codes)
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~fin)
    assert np.array_equal(got[fin], ref[fin])


def _fp8_pair(rng, E, N, K):
    """fp8 weights and the same matrices built independently as bf16 bits.

    Each value is sign * (1 + m/8) * 2^p (or 0); the row scale is 2^q.  The
    code is written from the E4M3 bit layout (exponent field p - q + 7), the
    bf16 bits from the bf16 layout, so neither side uses the oracle's decoder.
    """
    m = rng.integers(0, 8, size=(E, N, K))
    p = rng.integers(-3, 4, size=(E, N, K))
    s = rng.integers(0, 2, size=(E, N, K))
    zero = rng.random((E, N, K)) < 0.05
    q = rng.integers(-12, -4, size=(E, N))
    ef = p + 7                                           # E4M3 exponent field of the code
    codes = np.where(zero, 0, (s << 7) | (ef << 3) | m).astype(np.uint8)
    scales = np.exp2(q).astype(np.float32)
    eb = p + q[:, :, None] + 127                         # bf16 exponent field of the value
    bits = np.where(zero, 0, (s << 15) | (eb << 7) | (m << 4)).astype(np.uint16)
    return O.Fp8Weights(codes, scales), bits


def test_fp8_expert_table_equals_the_definition():
    # Fp8Weights looks codes up in the values of all 256 codes: the same as
    # decoding every code with e4m3_to_f64 (NaN codes included)
    rng = np.random.default_rng(23)
    codes = rng.integers(0, 256, size=(2, 16, 40), dtype=np.uint8)
    codes[1].reshape(-1)[:256] = np.arange(256, dtype=np.uint8)
    scales = rng.random((2, 16)).astype(np.float32)
    w = O.Fp8Weights(codes, scales)
    for e in range(2):
        direct = scales[e].astype(np.float64)[:, None] * O.e4m3_to_f64(codes[e])
        np.testing.assert_array_equal(w.expert(e), direct)


def test_fp8_forward_equals_bf16_on_same_values():
    rng = np.random.default_rng(21)
    T, d, E, F, k = 9, 32, 4, 48, 2
    wg8, wgb = _fp8_pair(rng, E, F, d)
    wu8, wub = _fp8_pair(rng, E, F, d)
    wd8, wdb = _fp8_pair(rng, E, d, F)
    x = (rng.standard_normal((T, d)) * 4).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)     # truncated: exact bf16 values
    wr = (rng.standard_normal((E, d))).astype(np.float32)
    wrb = (wr.view(np.uint32) >> 16).astype(np.uint16)
    a = O.forward(xb, wrb, wg8, wu8, wd8, k, "bf16")
    b = O.forward(xb, wrb, wgb, wub, wdb, k, "bf16")
    assert np.array_equal(a["out"], b["out"])


def test_fp8_scale_is_per_output_channel():
    # codes 0x38 (1.0) everywhere: W[n, i] = scale[n]; for one token routed to
    # expert 0 with weight 1, g_n = sg[n] * sum(x), u_n = su[n] * sum(x),
    # y_o = sd[o] * sum_n silu(g_n) * u_n
    d, F = 8, 6
    sg = np.array([[0.5, 1.0, 2.0, 0.25, 1.5, 3.0]], np.float32)
    su = np.array([[1.0, 0.5, 0.125, 2.0, 1.0, 0.75]], np.float32)
    sd = np.arange(1, d + 1, dtype=np.float32)[None, :] / 8
    one = lambda N, K: np.full((1, N, K), 0x38, np.uint8)
    x = np.linspace(-1, 1.5, d).astype(np.float32)[None, :]
    ids = np.zeros((1, 1), np.int32)
    w = np.ones((1, 1), np.float32)
    r = O.forward(x, np.zeros((1, d), np.float32), O.Fp8Weights(one(F, d), sg), O.Fp8Weights(one(F, d), su),
                  O.Fp8Weights(one(d, F), sd), 1, "f32", topk_ids=ids, topk_w=w)
    sx = float(x.astype(np.float64).sum())
    g = sg[0].astype(np.float64) * sx
    u = su[0].astype(np.float64) * sx
    hsum = float(np.sum(g / (1 + np.exp(-g)) * u))
    np.testing.assert_allclose(r["out"][0], sd[0].astype(np.float64) * hsum, rtol=1e-13)


def test_blocked16_layout_by_hand():
    # 2 matrices of 32 rows x 128 bytes: byte (m, r, b) must land at
    # m*4096 + (r // 16)*2048 + (b // 64)*1024 + (r % 16)*64 + b % 64
    rng = np.random.default_rng(4)
    a = rng.integers(0, 256, size=(2, 32, 128), dtype=np.uint8)
    out = O.blocked16(a).reshape(-1)
    for m in range(2):
        for r in range(32):
            for b in range(0, 128, 7):
                pos = m * 4096 + (r // 16) * 2048 + (b // 64) * 1024 + (r % 16) * 64 + b % 64
                assert out[pos] == a[m, r, b]
    # a permutation of bytes; element types keep their bytes together
    assert sorted(out.tolist()) == sorted(a.reshape(-1).tolist())
    w = rng.standard_normal((3, 16, 64)).astype(np.float32)
    assert sorted(O.blocked16(w).reshape(-1).tolist()) == sorted(w.reshape(-1).tolist())
