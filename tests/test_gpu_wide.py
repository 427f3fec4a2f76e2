"""GPU parity of the two-width gate+up kernel (bf16, 160-row tile map, a
mean of 48 to 160 rows per expert): tiles of at most 144 rows run 224 columns per
workgroup, longer tiles 112 columns, in one launch.

Routing is set explicitly so that every kind of unit appears: short last
tiles, tiles of 145-160 rows, experts of several tiles, an expert with no
rows, and column tails (F not a multiple of 224 or 112).  h is compared with
the oracle on every live row of every expert, the layer output on every
token; the output must equal the one-width kernel's bitwise (capacity mode
with room for every entry runs both passes in one launch, which takes the
one-width kernel, and every output element sums the same products in the
same order in both kernels); and the gather folded into the loads must give
the same h as the gathered x_perm.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.gpu_helpers import TOL, bits, check_dispatch, dev, host64, rel_err
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# name: (d, F, rows per expert (k = 1), weight layout blocked16)
CASES = {
    "ms10_mix": (256, 448, [150, 144, 145, 73], False),
    "multi_tile": (128, 320, [330, 320, 161, 0, 49, 16, 10, 10], True),
    "tails_blocked": (256, 320, [96, 130, 150, 60], True),
    "one_expert_long": (128, 192, [700, 20, 10, 5, 5, 0], False),
    "ragged_f": (192, 256, [50, 159, 144, 1, 100], False),
    "mean_150": (128, 320, [150, 160, 149, 141], False),   # every tile past 144 rows but one
}


def _inputs(name):
    d, F, counts, blocked = CASES[name]
    E, T = len(counts), sum(counts)
    wl = get_workload("mixtral_t512", T=T, d=d, E=E, k=1, F=F)
    inp = make_inputs(wl, 0)
    rng = np.random.default_rng(5)
    ids = rng.permutation(np.repeat(np.arange(E, dtype=np.int32), counts)).reshape(T, 1)
    w = np.ones((T, 1), dtype=np.float32)
    return wl, inp, ids, w, blocked


def _shape(wl, capacity, blocked):
    import grouped_gemm_gemv_amd as M
    return M.Shape(wl.T, wl.d, wl.E, 1, wl.F, capacity, torch.bfloat16, 160,
                   M.LAYOUT_BLOCKED16 if blocked else M.LAYOUT_ROWS)


@pytest.mark.parametrize("name", sorted(CASES))
def test_two_width_gate_up(name):
    import grouped_gemm_gemv_amd as M
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl, inp, ids, w, blocked = _inputs(name)
    print(f"\n[gpu wide] {name}: T={wl.T} d={wl.d} F={wl.F} rows per expert {CASES[name][2]}", flush=True)
    mean = -(-wl.T // wl.E)
    assert 48 <= mean <= 160  # the rows per expert for which moe_forward takes the two-width kernel
    x = dev(inp.x)
    wg, wu, wd = dev(inp.wg), dev(inp.wu), dev(inp.wd)
    if blocked:
        wg, wu, wd = M.moe_pack_blocked16(wg), M.moe_pack_blocked16(wu), M.moe_pack_blocked16(wd)
    ids_d, w_d = dev(ids), dev(w)
    shape = _shape(wl, 0, blocked)
    q = M.query(shape)
    assert q.tile_rows == 160
    ws = M.workspace(q.forward_ws_bytes)
    out = torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device="cuda")
    v = M.moe_forward(shape, x, None, None, ids_d, w_d, wg, wu, wd, out, ws)
    torch.cuda.synchronize()
    ref_disp = O.dispatch(ids, wl.E, 0, 160)
    check_dispatch(v.disp.arrays(), ref_disp, wl.E)
    # h on every live row of every expert
    worst = 0.0
    for e in range(wl.E):
        rows, h_ref, _ = O.expert_rows(inp.x, inp.wg, inp.wu, inp.wd, "bf16", ref_disp, e)
        if rows.size == 0:
            continue
        worst = max(worst, rel_err(host64(v.h[torch.from_numpy(rows).cuda()]), h_ref))
    ref = O.forward(inp.x, inp.wr, inp.wg, inp.wu, inp.wd, 1, "bf16", topk_ids=ids, topk_w=w)["out"]
    err = rel_err(host64(out), ref)
    print(f"[gpu wide] {name}: h rel err (worst expert) {worst:.3e}, layer rel err {err:.3e}", flush=True)
    assert worst <= TOL["bf16"] and err <= TOL["bf16"]
    # the one-width kernel (both capacity passes in one launch) gives the same bits
    cshape = _shape(wl, wl.T, blocked)
    cws = M.workspace(M.query(cshape).forward_ws_bytes)
    out1 = torch.empty_like(out)
    M.moe_forward(cshape, x, None, None, ids_d, w_d, wg, wu, wd, out1, cws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(out1))
    # the gathered x_perm through moe_ffn_gate_up gives the same h as the folded gather
    xp = torch.empty((q.rows, wl.d), dtype=torch.bfloat16, device="cuda")
    pws = M.workspace(q.permute_ws_bytes)
    M.moe_permute(shape, x, ids_d, v.disp, xp, pws)
    h2 = torch.empty_like(v.h)
    M.moe_ffn_gate_up(shape, xp, wg, wu, v.disp, 0, h2)
    torch.cuda.synchronize()
    live = torch.from_numpy(np.nonzero(ref_disp["token_of"] >= 0)[0]).cuda()
    assert np.array_equal(bits(h2[live]), bits(v.h[live]))


# K-split down GEMM (bf16, 160-row tile map, at least 80 mean rows per
# expert): name -> (d, F, rows per expert (k = 1), capacity)
SPLIT = {
    "odd_k_steps": (256, 192, [150, 60, 100, 160], 0),      # 3 K steps: ranges of 2 and 1
    "multi_tile": (512, 448, [330, 0, 161, 49, 100], 0),
    "capacity": (256, 320, [200, 40, 120, 80], 100),          # both passes in one launch
}


@pytest.mark.parametrize("name", sorted(SPLIT))
def test_split_k_down(name):
    import grouped_gemm_gemv_amd as M
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d, F, counts, C = SPLIT[name]
    E, T = len(counts), sum(counts)
    assert -(-T // E) >= 80 and (not C or min(-(-T // E), C) >= 80)
    wl = get_workload("mixtral_t512", T=T, d=d, E=E, k=1, F=F)
    inp = make_inputs(wl, 0)
    rng = np.random.default_rng(6)
    ids = rng.permutation(np.repeat(np.arange(E, dtype=np.int32), counts)).reshape(T, 1)
    w = np.ones((T, 1), dtype=np.float32)
    print(f"\n[gpu split-k] {name}: T={T} d={d} F={F} rows per expert {counts} C={C}", flush=True)
    shape = M.Shape(T, d, E, 1, F, C, torch.bfloat16, 160)
    q = M.query(shape)
    x, wg, wu, wd, ids_d, w_d = dev(inp.x), dev(inp.wg), dev(inp.wu), dev(inp.wd), dev(ids), dev(w)
    ws = M.workspace(q.forward_ws_bytes)
    out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    v = M.moe_forward(shape, x, None, None, ids_d, w_d, wg, wu, wd, out, ws)
    torch.cuda.synchronize()
    assert v.disp.c.kpart  # the shape splits the down GEMM's K loop
    ref_disp = O.dispatch(ids, E, C, 160)
    check_dispatch(v.disp.arrays(), ref_disp, E)
    worst = 0.0
    for e in range(E):
        rows, _, y_ref = O.expert_rows(inp.x, inp.wg, inp.wu, inp.wd, "bf16", ref_disp, e)
        if rows.size:
            worst = max(worst, rel_err(host64(v.y_perm[torch.from_numpy(rows).cuda()]), y_ref))
    ref = O.forward(inp.x, inp.wr, inp.wg, inp.wu, inp.wd, 1, "bf16", topk_ids=ids, topk_w=w, capacity=C)["out"]
    err = rel_err(host64(out), ref)
    print(f"[gpu split-k] {name}: y_perm rel err (worst expert) {worst:.3e}, layer rel err {err:.3e}", flush=True)
    assert worst <= TOL["bf16"] and err <= TOL["bf16"]
    # repeated down launches and whole layers give the same bits
    y0 = v.y_perm.clone()
    ps = M.PASS_BOTH if C else 0
    for _ in range(3):
        M.moe_ffn_down(shape, v.h, wd, v.disp, ps, v.y_perm)
    out2 = torch.empty_like(out)
    M.moe_forward(shape, x, None, None, ids_d, w_d, wg, wu, wd, out2, ws)
    torch.cuda.synchronize()
    live = torch.from_numpy(np.nonzero(ref_disp["token_of"] >= 0)[0]).cuda()
    assert np.array_equal(bits(v.y_perm[live]), bits(y0[live]))
    assert np.array_equal(bits(out2), bits(out))
    # moe_forward forms y inside its combine (combine_split_kernel); the
    # separate steps (down GEMM + k_split_finish, then moe_combine) give the
    # same y and the same output bits
    M.moe_ffn_down(shape, v.h, wd, v.disp, ps, v.y_perm)
    out3 = torch.empty_like(out)
    M.moe_combine(shape, v.y_perm, w_d, v.disp, out3)
    torch.cuda.synchronize()
    assert np.array_equal(bits(v.y_perm[live]), bits(y0[live]))
    assert np.array_equal(bits(out3), bits(out))
