"""GPU parity of the ping-pong main loop of the grouped GEMMs (bf16): gate+up
on 192- and 384-row tiles (prefetch depth 3 and 2), down on the 192-row
pieces of 384-row tiles (depth 3).

Routing is set explicitly so that tiles have full, partial and empty pieces
and experts have no rows; d and F give K loops whose length is and is not a
multiple of the prefetch depth (the last nit mod PF iterations issue no
loads).  h is compared with the oracle on every live row of every expert and
the layer output on every token; and since every output element sums the
same MFMA products in the same K order as in the shared main loop, the
output and h must equal, bitwise, those of 128-row tiles (which take the
shared loop for both GEMMs).
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.gpu_helpers import TOL, bits, check_dispatch, dev, host64, rel_err
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# name: (tile rows, d, F, rows per expert (k = 1), blocked weights)
# gate+up K steps = d / 64, down K steps = F / 64
CASES = {
    "bm384_tails": (384, 192, 320, [400, 384, 129, 0, 1, 700], False),    # 3 and 5 steps: tails of 1 and 2
    "bm384_even": (384, 256, 384, [385, 128, 256, 17], True),             # 4 and 6 steps: no tail
    "bm384_down_tail1": (384, 128, 448, [900, 30, 383], False),          # 2 and 7 steps
    "bm384_short_k": (384, 64, 128, [300, 5, 0, 129], False),            # 1 and 2 steps: fewer than the depth
    "bm192_tail3": (192, 448, 192, [192, 193, 50, 0, 400], True),        # gate+up 7 steps at depth 3: tail 1
    "bm192_tail1": (192, 320, 256, [10, 191, 384, 77], False),           # gate+up 5 steps: tail 2
    "bm192_short_k": (192, 128, 128, [200, 3, 0, 190], False),           # gate+up 2 steps: fewer than the depth
}


def _run(M, wl, shape, x, wg, wu, wd, ids_d, w_d):
    q = M.query(shape)
    ws = M.workspace(q.forward_ws_bytes)
    out = torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device="cuda")
    v = M.moe_forward(shape, x, None, None, ids_d, w_d, wg, wu, wd, out, ws)
    torch.cuda.synchronize()
    return q, v, out, ws


@pytest.mark.parametrize("name", sorted(CASES))
def test_pingpong_loop(name):
    import grouped_gemm_gemv_amd as M
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bm, d, F, counts, blocked = CASES[name]
    E, T = len(counts), sum(counts)
    wl = get_workload("mixtral_t512", T=T, d=d, E=E, k=1, F=F)
    inp = make_inputs(wl, 0)
    rng = np.random.default_rng(11)
    ids = rng.permutation(np.repeat(np.arange(E, dtype=np.int32), counts)).reshape(T, 1)
    w = np.ones((T, 1), dtype=np.float32)
    print(f"\n[gpu ping-pong] {name}: tile rows {bm}, T={T} d={d} F={F} rows per expert {counts}", flush=True)
    layout = M.LAYOUT_BLOCKED16 if blocked else M.LAYOUT_ROWS
    x = dev(inp.x)
    wg, wu, wd = dev(inp.wg), dev(inp.wu), dev(inp.wd)
    if blocked:
        wg, wu, wd = M.moe_pack_blocked16(wg), M.moe_pack_blocked16(wu), M.moe_pack_blocked16(wd)
    ids_d, w_d = dev(ids), dev(w)
    shape = M.Shape(T, d, E, 1, F, 0, torch.bfloat16, bm, layout)
    q, v, out, _ws = _run(M, wl, shape, x, wg, wu, wd, ids_d, w_d)
    assert q.tile_rows == bm
    ref_disp = O.dispatch(ids, E, 0, bm)
    check_dispatch(v.disp.arrays(), ref_disp, E)
    worst = 0.0
    for e in range(E):
        rows, h_ref, _ = O.expert_rows(inp.x, inp.wg, inp.wu, inp.wd, "bf16", ref_disp, e)
        if rows.size == 0:
            continue
        worst = max(worst, rel_err(host64(v.h[torch.from_numpy(rows).cuda()]), h_ref))
    ref = O.forward(inp.x, inp.wr, inp.wg, inp.wu, inp.wd, 1, "bf16", topk_ids=ids, topk_w=w)["out"]
    err = rel_err(host64(out), ref)
    print(f"[gpu ping-pong] {name}: h rel err (worst expert) {worst:.3e}, layer rel err {err:.3e}", flush=True)
    assert worst <= TOL["bf16"] and err <= TOL["bf16"]
    # 128-row tiles run the shared main loop for both GEMMs: same bits
    shape128 = M.Shape(T, d, E, 1, F, 0, torch.bfloat16, 128, layout)
    q128, v128, out128, _ws128 = _run(M, wl, shape128, x, wg, wu, wd, ids_d, w_d)
    assert q128.tile_rows == 128
    assert np.array_equal(bits(out), bits(out128))
    d128 = O.dispatch(ids, E, 0, 128)
    for e in range(E):
        r1, _, _ = O.expert_rows(inp.x, inp.wg, inp.wu, inp.wd, "bf16", ref_disp, e)
        r2, _, _ = O.expert_rows(inp.x, inp.wg, inp.wu, inp.wd, "bf16", d128, e)
        if r1.size == 0:
            continue
        h1 = v.h[torch.from_numpy(r1).cuda()]
        h2 = v128.h[torch.from_numpy(r2).cuda()]
        assert np.array_equal(bits(h1), bits(h2)), f"expert {e}: h differs from the shared loop's"
