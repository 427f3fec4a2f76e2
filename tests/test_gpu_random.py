"""Seeded randomized parity sweep: moe_forward (and moe_forward_fp8) against
the oracle on shapes drawn at random — odd token counts, expert counts that
are not powers of two, narrow and wide d/F, capacity on and off, both
weight layouts, fp32/bf16/E4M3, automatic and forced tile heights.  Each
case is small enough for the oracle; the draw is fixed by the case index.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.gpu_helpers import TOL, bits, check_dispatch, dev, host64, rel_err, torch_dtype
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

N_CASES = 96
TILES = (0, 0, 0, 16, 32, 48, 64, 96, 128, 160, 192)


def draw(i, seed_base=1000, tiles=TILES):
    rng = np.random.default_rng(seed_base + i)
    E = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 31, 64, 100, 256]))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([1, 2, 7, 15, 16, 17, 63, 100, 257, 600]))
    d = int(64 * rng.integers(1, 9))
    F = int(64 * rng.integers(1, 9))
    kind = rng.choice(["bf16", "bf16", "f32", "fp8"])
    cap = 0
    if rng.random() < 0.35:
        cap = int(rng.integers(1, max(2, T * k // max(E, 1)) + 2))
    bm = int(rng.choice(tiles))
    layout = int(rng.integers(0, 2))
    return dict(E=E, k=k, T=T, d=d, F=F, kind=str(kind), capacity=cap, bm=bm, layout=layout)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_parity(i):
    _run_case(i, draw(i))


@pytest.mark.parametrize("i", range(24))
def test_random_shape_parity_384_row_tiles(i):
    """384-row tiles: each tile of the map is worked in pieces (three of 128
    rows by gate+up, two of 192 by down), some of them empty or ragged."""
    _run_case(100 + i, draw(i, seed_base=2000, tiles=(384,)))


def _run_case(i, c):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_gemm_gemv_amd as M
    print(f"\n[gpu random] case {i}: {c}", flush=True)
    base = {"bf16": "mixtral_t512", "f32": "tiny_f32", "fp8": "mixtral_t512_fp8"}[c["kind"]]
    over = dict(T=c["T"], d=c["d"], E=c["E"], k=c["k"], F=c["F"], capacity=c["capacity"])
    if c["kind"] == "f32":
        over.update(wr_std=1.0 / np.sqrt(c["d"]), w_std=1.0 / np.sqrt(c["d"]))
    wl = get_workload(base, **over)
    inp = make_inputs(wl, i)
    dt = torch_dtype(wl.dtype)
    fp8 = wl.weights == "e4m3"
    shape = M.Shape(wl.T, wl.d, wl.E, wl.k, wl.F, wl.capacity, dt, c["bm"], c["layout"])
    q = M.query(shape)
    names = ("wg", "wu", "wd", "sg", "su", "sd") if fp8 else ("wg", "wu", "wd")
    w = [dev(getattr(inp, n)) for n in names]
    if c["layout"]:
        w = [M.moe_pack_blocked16(t) if t.dim() == 3 else t for t in w]
    ws = M.workspace(q.forward_ws_bytes)
    out = torch.empty((wl.T, wl.d), dtype=dt, device="cuda")
    fwd = M.moe_forward_fp8 if fp8 else M.moe_forward
    v = fwd(shape, dev(inp.x), dev(inp.wr), None, None, None, *w, out, ws)
    torch.cuda.synchronize()
    ids = v.topk_ids.cpu().numpy()
    # routing: the GPU's ids must be a valid top-k of the oracle's logits (near-ties aside)
    lg = O.router_logits(inp.x, inp.wr, wl.dtype)
    o_ids, _ = O.route_from_logits(lg, wl.k)
    gap = O.topk_gap(lg, wl.k)
    differ = [t for t in range(wl.T) if not np.array_equal(ids[t], o_ids[t])]
    assert all(gap[t] < 1e-4 for t in differ), (differ, gap[differ])
    m = lg.max(axis=1, keepdims=True)
    p = np.exp(lg - m)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    w_ref = sel / sel.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(v.topk_w.cpu().numpy(), w_ref, atol=2e-6)
    disp = O.dispatch(ids, wl.E, wl.capacity, q.tile_rows)
    check_dispatch(v.disp.arrays(), disp, wl.E)
    ow = (O.Fp8Weights(inp.wg, inp.sg), O.Fp8Weights(inp.wu, inp.su), O.Fp8Weights(inp.wd, inp.sd)) if fp8 \
        else (inp.wg, inp.wu, inp.wd)
    ref = O.forward(inp.x, inp.wr, *ow, wl.k, wl.dtype, topk_ids=ids, topk_w=w_ref, capacity=wl.capacity,
                    tile_rows=q.tile_rows)
    err = rel_err(host64(out), ref["out"])
    print(f"[gpu random] case {i}: tile rows {q.tile_rows}, rel err {err:.2e}")
    assert err <= TOL[wl.dtype]
