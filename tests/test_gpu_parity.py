"""GPU parity: every call of libmoe against the CPU oracle on seeded inputs.

Sizes are small enough for the oracle to finish in seconds while spanning
several row tiles, several column tiles and ragged tails.  Integer outputs
(ids up to near-ties, counts, offsets, permutation, tile map) must be
bit-exact; floating-point outputs must satisfy
max|gpu - oracle| / max|oracle| <= 2e-2 (bf16) or 1e-4 (fp32).
"""
import dataclasses
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.gpu_helpers import TOL, bits, check_dispatch, check_routing, dev, host64, rel_err, torch_dtype
from workloads import get_workload, make_inputs, zipf_routing

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# name, base workload, overrides, routing override
CASES = {
    "tiny_f32": ("tiny_f32", {}),
    "bf16_ragged": ("mixtral_t512", dict(T=200, d=256, F=320)),
    "bf16_e64_zipf": ("e64_zipf_a1.2", dict(T=96, d=192, F=128)),
    "bf16_e64_zipf2": ("e64_zipf_a2.0", dict(T=160, d=128, F=192)),
    "bf16_capacity": ("capacity_gini0.30", dict(T=300, d=128, E=16, k=4, F=192, capacity=40)),
    "bf16_t1": ("mixtral_t512", dict(T=1, d=256, F=128)),
    "bf16_dense": ("mixtral_t512", dict(T=50, d=128, E=1, k=1, F=128)),
    "f32_e256": ("tiny_f32", dict(T=40, d=64, E=256, k=8, F=64)),
    "f32_capacity": ("tiny_f32", dict(T=64, E=4, k=2, capacity=20)),
    # tile heights 48 / 96 / 128 / 160 and column tails (F or d not a multiple of the column tile)
    "bf16_bm48": ("mixtral_t512", dict(T=152, d=128, F=128)),
    "bf16_bm96": ("mixtral_t512", dict(T=256, d=128, F=192)),
    "bf16_bm128": ("mixtral_t512", dict(T=400, d=128, F=256)),
    "bf16_bm160": ("mixtral_t512", dict(T=512, d=256, F=128)),
    "bf16_bm192": ("mixtral_t512", dict(T=512, d=128, E=4, F=192)),
    # degenerate and extreme cases: no overflow region at all (C = T*k), one
    # entry per expert in the fixed region (C = 1), every entry routed to one
    # expert (k = 1, Zipf with an overwhelming first rank), the largest E and k
    "bf16_cap_no_spill": ("capacity_gini0.30", dict(T=64, d=128, E=8, k=2, F=128, capacity=128)),
    "bf16_cap_c1": ("capacity_gini0.30", dict(T=100, d=64, E=8, k=2, F=64, capacity=1)),
    "bf16_one_expert": ("e64_zipf_a2.0", dict(T=300, d=128, E=16, k=1, F=128, zipf_alpha=60.0)),
    # a few dominant experts among 64 (the top Zipf ranks take nearly every
    # token), each with several row tiles, beside many one-tile experts
    "bf16_dominant_e64": ("e64_zipf_a2.0", dict(T=600, d=128, F=192, zipf_alpha=4.0)),
    "bf16_e256_k64": ("mixtral_t512", dict(T=33, d=64, E=256, k=64, F=64)),
    # decode batches (T <= 16, E <= 64): moe_forward routes and dispatches
    # them in one workgroup (route_dispatch_kernel), which the step-by-step
    # path (moe_route, then moe_permute) checks bitwise, at each router tile
    # (E <= 16, 32, 64), with a router bias and the capacity split; T = 17
    # takes the separate router and dispatch launches in moe_forward too
    "bf16_t8": ("mixtral_t512", dict(T=8, d=256, F=128)),
    "bf16_t16_e64": ("mixtral_t512", dict(T=16, d=256, E=64, k=6, F=128)),
    "bf16_t1_e64": ("mixtral_t512", dict(T=1, d=128, E=64, k=8, F=64)),
    "f32_t16_e32": ("tiny_f32", dict(T=16, E=32, k=4)),
    "bf16_t12_cap_bias": ("capacity_gini0.30", dict(T=12, d=128, E=16, k=4, F=128, capacity=2)),
    "bf16_t17": ("mixtral_t512", dict(T=17, d=128, F=64)),
    # one or two (token, slot) entries: moe_forward computes the combine inside
    # the down GEMM, which the step-by-step path checks bitwise
    "f32_t1": ("tiny_f32", dict(T=1)),
    "bf16_t2_k1": ("mixtral_t512", dict(T=2, d=192, k=1, F=320)),
    "bf16_t1_k1": ("mixtral_t512", dict(T=1, d=128, E=4, k=1, F=64)),
    # 384-row tiles, worked in pieces (three of 128 rows by gate+up, two of
    # 192 by down): experts of two and three map tiles with ragged and empty
    # last pieces, the capacity split, and fp32
    "bf16_bm384": ("mixtral_t512", dict(T=900, d=128, E=2, k=1, F=192), dict(tile_rows=384)),
    "bf16_bm384_cap": ("capacity_gini0.30", dict(T=400, d=64, E=4, k=2, F=128, capacity=150),
                       dict(tile_rows=384)),
    "f32_bm384": ("tiny_f32", dict(T=300, E=3, k=2, F=128), dict(tile_rows=384)),
}


def _workload(case):
    base, over = CASES[case][:2]
    return get_workload(base, **over)


def _shape(wl, case=None):
    from grouped_gemm_gemv_amd import Shape
    extra = CASES[case][2] if case is not None and len(CASES[case]) > 2 else {}
    return Shape(T=wl.T, d=wl.d, E=wl.E, k=wl.k, F=wl.F, capacity=wl.capacity, dtype=torch_dtype(wl.dtype),
                 **extra)


class Run:
    """Inputs on host and device plus every GPU stage, run step by step."""

    def __init__(self, case, seed=0):
        import grouped_gemm_gemv_amd as M
        wl = _workload(case)
        self.wl = wl
        self.inp = make_inputs(wl, seed)
        inp = self.inp
        self.shape = _shape(wl, case)
        self.q = M.query(self.shape)
        dt = torch_dtype(wl.dtype)
        self.x, self.wr = dev(inp.x), dev(inp.wr)
        self.wg, self.wu, self.wd = dev(inp.wg), dev(inp.wu), dev(inp.wd)
        self.bias = dev(inp.bias)
        T, k = wl.T, wl.k
        if inp.topk_ids is not None:
            self.ids = dev(inp.topk_ids)
            self.w = dev(inp.topk_w)
            self.logits = None
        else:
            self.ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
            self.w = torch.empty((T, k), dtype=torch.float32, device="cuda")
            M.moe_route(self.shape, self.x, self.wr, self.bias, self.ids, self.w)
            self.logits = O.router_logits(inp.x, inp.wr, wl.dtype, inp.bias)
        R = self.q.rows
        self.disp = M.Dispatch(self.shape)
        self.xp = torch.zeros((R, wl.d), dtype=dt, device="cuda")
        ws = M.workspace(self.q.permute_ws_bytes)
        M.moe_permute(self.shape, self.x, self.ids, self.disp, self.xp, ws)
        self.h = torch.zeros((R, wl.F), dtype=dt, device="cuda")
        self.y = torch.zeros((R, wl.d), dtype=dt, device="cuda")
        M.moe_grouped_ffn(self.shape, self.xp, self.wg, self.wu, self.wd, self.disp, self.h, self.y)
        self.out = torch.empty((T, wl.d), dtype=dt, device="cuda")
        M.moe_combine(self.shape, self.y, self.w, self.disp, self.out)
        torch.cuda.synchronize()
        self.gpu_ids = self.ids.cpu().numpy()
        self.gpu_w = self.w.cpu().numpy().astype(np.float64)
        self.ref_disp = O.dispatch(self.gpu_ids, wl.E, wl.capacity, self.q.tile_rows)


@pytest.fixture(scope="module")
def runs():
    _need_gpu()
    cache = {}

    def get(case):
        if case not in cache:
            print(f"\n[gpu parity] case {case}", flush=True)
            cache[case] = Run(case)
        return cache[case]
    return get


@pytest.mark.parametrize("case", sorted(CASES))
def test_route(runs, case):
    r = runs(case)
    if r.logits is None:
        pytest.skip("routing supplied (Zipf ids)")
    differ = check_routing(r.gpu_ids, r.gpu_w, r.logits, r.wl.k)
    assert differ <= max(1, r.wl.T // 100)


@pytest.mark.parametrize("case", sorted(CASES))
def test_dispatch_bit_exact(runs, case):
    r = runs(case)
    check_dispatch(r.disp.arrays(), r.ref_disp, r.wl.E)


def test_degenerate_cases_are_what_they_claim(runs):
    r = runs("bf16_cap_no_spill")
    assert r.ref_disp["spill_counts"].sum() == 0 and O.spill_rows_bound(64, 2, 128) == 0
    r = runs("bf16_one_expert")
    assert len(np.unique(r.gpu_ids)) == 1
    r = runs("bf16_cap_c1")
    assert (r.ref_disp["kept_counts"] <= 1).all() and r.ref_disp["spill_counts"].sum() > 0


@pytest.mark.parametrize("case", sorted(CASES))
def test_gather_bitwise(runs, case):
    r = runs(case)
    ref = O.gather(r.inp.x, r.ref_disp)
    live = r.ref_disp["token_of"] >= 0
    assert np.array_equal(bits(r.xp)[live], ref[live].view(bits(r.xp).dtype))


def _oracle_rows(r):
    """Oracle h and y for every live row (float64)."""
    wl, inp, d = r.wl, r.inp, r.ref_disp
    x64 = O.to_f64(inp.x, wl.dtype)
    h = np.zeros((d["R"], wl.F))
    y = np.zeros((d["R"], wl.d))
    ids = r.gpu_ids.reshape(-1)
    for e in range(wl.E):
        fs = np.nonzero(ids == e)[0]
        if fs.size == 0:
            continue
        X = x64[fs // wl.k]
        G = X @ O.to_f64(inp.wg[e], wl.dtype).T
        U = X @ O.to_f64(inp.wu[e], wl.dtype).T
        H = O.silu(G) * U
        rows = d["row_of"][fs]
        h[rows] = H
        y[rows] = H @ O.to_f64(inp.wd[e], wl.dtype).T
    return h, y


@pytest.mark.parametrize("case", sorted(CASES))
def test_grouped_ffn(runs, case):
    r = runs(case)
    h_ref, y_ref = _oracle_rows(r)
    live = r.ref_disp["token_of"] >= 0
    tol = TOL[r.wl.dtype]
    assert rel_err(host64(r.h)[live], h_ref[live]) <= tol
    assert rel_err(host64(r.y)[live], y_ref[live]) <= tol


@pytest.mark.parametrize("case", sorted(CASES))
def test_layer_output(runs, case):
    r = runs(case)
    wl, inp = r.wl, r.inp
    w_ref = r.gpu_w if r.logits is None else None
    if w_ref is None:
        m = r.logits.max(axis=1, keepdims=True)
        p = np.exp(r.logits - m)
        sel = np.take_along_axis(p, r.gpu_ids.astype(np.int64), axis=1)
        w_ref = sel / sel.sum(axis=1, keepdims=True)
    ref = O.forward(inp.x, inp.wr, inp.wg, inp.wu, inp.wd, wl.k, wl.dtype, topk_ids=r.gpu_ids,
                    topk_w=w_ref, capacity=wl.capacity, tile_rows=r.q.tile_rows)
    err = rel_err(host64(r.out), ref["out"])
    print(f"[{case}] layer rel err {err:.3e}")
    assert err <= TOL[wl.dtype]


@pytest.mark.parametrize("case", sorted(CASES))
def test_forward_matches_steps_and_is_deterministic(runs, case):
    import grouped_gemm_gemv_amd as M
    r = runs(case)
    ws = M.workspace(r.q.forward_ws_bytes)
    supplied = r.logits is None
    outs = []
    for _ in range(2):
        out = torch.empty_like(r.out)
        v = M.moe_forward(r.shape, r.x, r.wr, r.bias, r.ids if supplied else None, r.w if supplied else None,
                          r.wg, r.wu, r.wd, out, ws)
        torch.cuda.synchronize()
        outs.append(bits(out))
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[0], bits(r.out))
    assert np.array_equal(v.topk_ids.cpu().numpy(), r.gpu_ids)
    assert np.array_equal(bits(v.topk_w), bits(r.w))
    # the dispatch the layer built is the one moe_permute builds, array by
    # array (tile map entries past n_tiles are unused)
    fa, sa = v.disp.arrays(), r.disp.arrays()
    for name in ("counts", "offsets", "spill_counts", "spill_offsets", "row_of", "token_of", "tile_off",
                 "n_tiles", "err_flags"):
        assert torch.equal(fa[name].cpu(), sa[name].cpu()), name
    nt = sa["n_tiles"].cpu().numpy()
    for p in range(2):
        assert torch.equal(fa["tile_map"][p, :nt[p]].cpu(), sa["tile_map"][p, :nt[p]].cpu()), p


@pytest.mark.parametrize("case", ["bf16_capacity", "f32_capacity"])
def test_capacity_equals_uncapped(runs, case):
    """Capacity + overflow pass gives the uncapped layer output; with the same
    tile configuration every (token, expert) row runs the same K loop, so the
    two are bitwise equal."""
    import grouped_gemm_gemv_amd as M
    r = runs(case)
    assert r.ref_disp["spill_counts"].sum() > 0, "case must overflow"
    bm = r.q.tile_rows
    for shape0 in (dataclasses.replace(r.shape, capacity=0),
                   dataclasses.replace(r.shape, capacity=0, tile_rows=bm)):
        q0 = M.query(shape0)
        ws = M.workspace(q0.forward_ws_bytes)
        out0 = torch.empty_like(r.out)
        M.moe_forward(shape0, r.x, r.wr, r.bias, r.ids, r.w, r.wg, r.wu, r.wd, out0, ws)
        torch.cuda.synchronize()
        assert rel_err(host64(r.out), host64(out0)) <= TOL[r.wl.dtype]
    assert np.array_equal(bits(r.out), bits(out0))


def test_identity_path_returns_input(runs):
    """moe_permute then moe_combine with y := x_perm returns x (weights sum to 1)."""
    import grouped_gemm_gemv_amd as M
    r = runs("bf16_e64_zipf")
    out = torch.empty_like(r.x)
    M.moe_combine(r.shape, r.xp, r.w, r.disp, out)
    torch.cuda.synchronize()
    x = host64(r.x)
    err = np.abs(host64(out) - x)
    # sum_j w_j * x is x * (1 + O(k * 2^-24)); after bf16 rounding at most 1 ulp away
    assert (err <= np.abs(x) * 2.0 ** -7 + 1e-30).all()
    assert (err == 0).mean() > 0.99


@pytest.mark.parametrize("E,k,dt", [(24, 3, "bf16"), (64, 8, "bf16"), (100, 6, "f32"), (128, 16, "bf16"),
                                    (256, 64, "bf16"), (5, 5, "f32")])
def test_route_every_expert_range(E, k, dt):
    """Router kernels for E <= 16, 32, 64, 128, 256 (one instantiation each), k up to 64 and k = E."""
    _need_gpu()
    import grouped_gemm_gemv_amd as M
    base = "tiny_f32" if dt == "f32" else "mixtral_t512"
    wl = get_workload(base, T=70, d=320, E=E, k=k, F=64, wr_std=0.5 if dt == "bf16" else 1.0)
    inp = make_inputs(wl, 3, experts=False)
    shape = _shape(wl)
    ids = torch.empty((wl.T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, k), dtype=torch.float32, device="cuda")
    print(f"\n[gpu parity] route E={E} k={k} {dt}", flush=True)
    M.moe_route(shape, dev(inp.x), dev(inp.wr), None, ids, w)
    torch.cuda.synchronize()
    logits = O.router_logits(inp.x, inp.wr, wl.dtype)
    differ = check_routing(ids.cpu().numpy(), w.cpu().numpy().astype(np.float64), logits, k)
    assert differ <= 1


@pytest.mark.parametrize("E,k,dt", [(8, 2, "bf16"), (24, 3, "f32"), (64, 6, "bf16"), (100, 6, "bf16")])
def test_route_large_batch(E, k, dt):
    """Batches of 2048 tokens and more: 16 tokens per router workgroup at each
    router tile; T = 2100 leaves a last workgroup of 4 tokens."""
    _need_gpu()
    import grouped_gemm_gemv_amd as M
    base = "tiny_f32" if dt == "f32" else "mixtral_t512"
    wl = get_workload(base, T=2100, d=128, E=E, k=k, F=64, wr_std=0.5 if dt == "bf16" else 1.0)
    inp = make_inputs(wl, 4, experts=False)
    shape = _shape(wl)
    ids = torch.empty((wl.T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, k), dtype=torch.float32, device="cuda")
    print(f"\n[gpu parity] route T={wl.T} E={E} k={k} {dt}", flush=True)
    M.moe_route(shape, dev(inp.x), dev(inp.wr), None, ids, w)
    torch.cuda.synchronize()
    logits = O.router_logits(inp.x, inp.wr, wl.dtype)
    differ = check_routing(ids.cpu().numpy(), w.cpu().numpy().astype(np.float64), logits, k)
    assert differ <= wl.T // 100  # tokens whose k-th and (k+1)-th logits nearly tie


@pytest.mark.parametrize("C", [0, 200])
def test_dispatch_multiblock_path(C):
    """T*k above the single-workgroup limit: count + scan + scatter kernels."""
    _need_gpu()
    import grouped_gemm_gemv_amd as M
    T, k, E = 5000, 4, 64
    rng = np.random.default_rng(7)
    # skewed ids, distinct per token
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.0
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    shape = M.Shape(T=T, d=64, E=E, k=k, F=64, capacity=C, dtype=torch.bfloat16)
    q = M.query(shape)
    x = torch.randn((T, 64), device="cuda").to(torch.bfloat16)
    disp = M.Dispatch(shape)
    xp = torch.zeros((q.rows, 64), dtype=torch.bfloat16, device="cuda")
    print(f"\n[gpu parity] multiblock dispatch C={C}", flush=True)
    M.moe_permute(shape, x, dev(ids), disp, xp, M.workspace(q.permute_ws_bytes))
    torch.cuda.synchronize()
    ref = O.dispatch(ids, E, C, q.tile_rows)
    if C:
        assert ref["spill_counts"].sum() > 0
    check_dispatch(disp.arrays(), ref, E)
    xb = bits(x)
    live = ref["token_of"] >= 0
    assert np.array_equal(bits(xp)[live], xb[ref["token_of"][live]])


# (T, k, E, C, invalid ids): one-wavefront dispatch (T*k <= 64, E <= 64,
# rows <= 4096) at its limits, with the capacity split, dead rows and
# invalid ids; and the same kinds of input just past each limit (1024-thread
# block)
TINY = {
    "t1_k2": (1, 2, 8, 0, False),
    "tk64_e8": (32, 2, 8, 0, False),
    "tk64_e64": (64, 1, 64, 0, False),
    "cap_overflow": (16, 4, 16, 3, False),
    "cap_rows_4032": (1, 1, 64, 63, False),
    "bad_ids": (20, 3, 10, 0, True),
    "cap_bad_ids": (20, 2, 8, 2, True),
    "tk65_block": (65, 1, 8, 0, False),
    "e65_block": (8, 2, 65, 0, True),
    "rows_4160_block": (1, 1, 64, 65, False),
}


@pytest.mark.parametrize("name", sorted(TINY))
def test_small_dispatch_paths(name):
    """Dispatch of small batches against the oracle, array by array.  Invalid
    ids (outside [0, E)) are skipped: every other entry gets the row and rank
    the oracle gives the batch without them, so the expected arrays are the
    oracle's dispatch of the valid entries (one per row, k = 1), mapped back
    to their flat index f and token f // k."""
    _need_gpu()
    import grouped_gemm_gemv_amd as M
    T, k, E, C, bad = TINY[name]
    rng = np.random.default_rng(11)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if bad:
        ids[1, 0] = E
        ids[T - 2, k - 1] = -1
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    fv = np.nonzero(valid)[0]
    shape = M.Shape(T=T, d=64, E=E, k=k, F=64, capacity=C, dtype=torch.bfloat16)
    q = M.query(shape)
    print(f"\n[gpu parity] small dispatch {name}: T={T} k={k} E={E} C={C} rows={q.rows}", flush=True)
    x = torch.randn((T, 64), device="cuda").to(torch.bfloat16)
    disp = M.Dispatch(shape)
    xp = torch.zeros((q.rows, 64), dtype=torch.bfloat16, device="cuda")
    M.moe_permute(shape, x, dev(ids), disp, xp, M.workspace(q.permute_ws_bytes))
    torch.cuda.synchronize()
    sub = O.dispatch(flat[fv].reshape(-1, 1), E, C, q.tile_rows)
    ref = dict(sub)
    ref["row_of"] = np.full(T * k, -1, dtype=np.int64)
    ref["row_of"][fv] = sub["row_of"]
    ref["token_of"] = np.full(q.rows, -1, dtype=np.int64)
    live = sub["token_of"] >= 0
    ref["token_of"][np.nonzero(live)[0]] = fv[sub["token_of"][live]] // k
    a = disp.arrays()
    assert int(a["err_flags"].cpu().numpy()[0]) == (1 if bad else 0)
    a = dict(a)
    a["err_flags"] = torch.zeros_like(a["err_flags"])
    check_dispatch(a, ref, E)
    xb = bits(x)
    rows = ref["token_of"] >= 0
    assert np.array_equal(bits(xp)[rows], xb[ref["token_of"][rows]])


def test_invalid_ids_flagged_and_skipped():
    """Ids outside [0, E) set err_flags bit 0, get row -1 and contribute nothing."""
    _need_gpu()
    import grouped_gemm_gemv_amd as M
    T, k, E = 40, 2, 8
    rng = np.random.default_rng(8)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[3, 1] = E
    ids[17, 0] = -1
    shape = M.Shape(T=T, d=64, E=E, k=k, F=64, dtype=torch.bfloat16)
    q = M.query(shape)
    x = torch.randn((T, 64), device="cuda").to(torch.bfloat16)
    disp = M.Dispatch(shape)
    xp = torch.zeros((q.rows, 64), dtype=torch.bfloat16, device="cuda")
    M.moe_permute(shape, x, dev(ids), disp, xp, M.workspace(q.permute_ws_bytes))
    torch.cuda.synchronize()
    a = disp.arrays()
    assert int(a["err_flags"].cpu()[0]) & 1
    row_of = a["row_of"].cpu().numpy()
    assert row_of[3 * k + 1] == -1 and row_of[17 * k + 0] == -1
    valid = np.ones(T * k, bool)
    valid[[3 * k + 1, 17 * k]] = False
    assert a["counts"].cpu().numpy().sum() == valid.sum()
    # the identity combine of the valid slots: weight 1 on each valid slot
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    w[:, 0] = 1.0
    w[17, 1] = 1.0
    out = torch.empty_like(x)
    M.moe_combine(shape, xp, w, disp, out)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(x))


@pytest.mark.parametrize("case", ["bf16_capacity", "f32_capacity", "bf16_bm384_cap", "bf16_cap_c1",
                                  "bf16_cap_no_spill", "bf16_ragged"])
def test_both_passes_in_one_launch(runs, case):
    """pass = PASS_BOTH (each expert's overflow tiles in the same launch as its
    first-pass tiles) gives h and y bitwise equal to the two separate passes;
    without capacity it is pass 0."""
    import grouped_gemm_gemv_amd as M
    r = runs(case)
    h2, y2, h3 = torch.zeros_like(r.h), torch.zeros_like(r.y), torch.zeros_like(r.h)
    M.moe_ffn_gate_up(r.shape, r.xp, r.wg, r.wu, r.disp, M.PASS_BOTH, h2)
    M.moe_ffn_down(r.shape, h2, r.wd, r.disp, M.PASS_BOTH, y2)
    M.moe_ffn_gate_up_gather(r.shape, r.x, r.wg, r.wu, r.disp, M.PASS_BOTH, h3)
    torch.cuda.synchronize()
    live = r.ref_disp["token_of"] >= 0
    assert np.array_equal(bits(h2)[live], bits(r.h)[live])
    assert np.array_equal(bits(y2)[live], bits(r.y)[live])
    assert np.array_equal(bits(h3)[live], bits(r.h)[live])


@pytest.mark.parametrize("case", sorted(CASES))
def test_gate_up_gather_equals_gate_up(runs, case):
    """The gather folded into the gate+up loads gives h bitwise equal to
    moe_permute's gather followed by moe_ffn_gate_up."""
    import grouped_gemm_gemv_amd as M
    r = runs(case)
    h2 = torch.zeros_like(r.h)
    for p in range(r.q.n_passes):
        M.moe_ffn_gate_up_gather(r.shape, r.x, r.wg, r.wu, r.disp, p, h2)
    torch.cuda.synchronize()
    live = r.ref_disp["token_of"] >= 0
    assert np.array_equal(bits(h2)[live], bits(r.h)[live])
