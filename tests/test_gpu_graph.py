"""moe_forward captured in a hipGraph: capture succeeds (no host sync, no
allocation inside the call) and every replay equals an eager run bitwise,
with eager work, synchronisations and input changes between replays."""
import numpy as np
import pytest

from tests.gpu_helpers import bits, dev, torch_dtype
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("base,over,bm", [
    ("mixtral_t512", dict(T=200, d=256, F=320), 0),
    ("capacity_gini0.30", dict(T=300, d=128, E=16, k=4, F=192, capacity=40), 0),
    ("e64_zipf_a1.2", dict(T=96, d=192, F=128), 0),
    # 384-row tiles worked in pieces; the two inputs route differently
    ("mixtral_t512", dict(T=900, d=128, E=2, k=1, F=192), 384),
])
def test_graph_replays_match_eager(base, over, bm):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_gemm_gemv_amd as M
    wl = get_workload(base, **over)
    print(f"\n[gpu graph] {base} {over} tile rows {bm}", flush=True)
    inp = make_inputs(wl, 0)
    inp2 = make_inputs(wl, 1, experts=False)
    dt = torch_dtype(wl.dtype)
    shape = M.Shape(wl.T, wl.d, wl.E, wl.k, wl.F, wl.capacity, dt, bm)
    q = M.query(shape)
    x = dev(inp.x)
    xs = [dev(inp.x), dev(inp2.x)]
    wr, bias = dev(inp.wr), dev(inp.bias)
    ids, w = dev(inp.topk_ids), dev(inp.topk_w)
    wg, wu, wd = dev(inp.wg), dev(inp.wu), dev(inp.wd)
    ws = M.workspace(q.forward_ws_bytes)
    out = torch.empty((wl.T, wl.d), dtype=dt, device="cuda")

    def step():
        M.moe_forward(shape, x, wr, bias, ids, w, wg, wu, wd, out, ws)

    # eager references for both inputs (separate workspace and output)
    ws_e = M.workspace(q.forward_ws_bytes)
    refs = []
    for xi in xs:
        o = torch.empty_like(out)
        M.moe_forward(shape, xi, wr, bias, ids, w, wg, wu, wd, o, ws_e)
        torch.cuda.synchronize()
        refs.append(bits(o))
    assert not np.array_equal(refs[0], refs[1])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(6):
        which = rep % 2
        x.copy_(xs[which])
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), refs[which]), f"replay {rep} differs"
        # unrelated eager work between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)


def test_graph_replays_match_eager_fp8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_gemm_gemv_amd as M
    wl = get_workload("mixtral_t512_fp8", T=200, d=256, F=320)
    inp = make_inputs(wl, 0)
    inp2 = make_inputs(wl, 1, experts=False)
    shape = M.Shape(wl.T, wl.d, wl.E, wl.k, wl.F, 0, torch.bfloat16)
    q = M.query(shape)
    x = dev(inp.x)
    xs = [dev(inp.x), dev(inp2.x)]
    wr = dev(inp.wr)
    wts = [dev(getattr(inp, n)) for n in ("wg", "wu", "wd", "sg", "su", "sd")]
    ws = M.workspace(q.forward_ws_bytes)
    out = torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device="cuda")
    ws_e = M.workspace(q.forward_ws_bytes)
    refs = []
    for xi in xs:
        o = torch.empty_like(out)
        M.moe_forward_fp8(shape, xi, wr, None, None, None, *wts, o, ws_e)
        torch.cuda.synchronize()
        refs.append(bits(o))

    def step():
        M.moe_forward_fp8(shape, x, wr, None, None, None, *wts, out, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        which = rep % 2
        x.copy_(xs[which])
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), refs[which]), f"replay {rep} differs"
