"""moe_forward_noalloc through the C ABI: the whole layer with the library's
own device scratch array instead of a workspace.  Its output must equal
moe_forward's bitwise (same kernels, same shape) and the oracle's within the
layer tolerance, on consecutive calls whose inputs shrink, so each call finds
the previous call's data in the shared array."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.gpu_helpers import TOL, bits, dev, host64, rel_err, torch_dtype
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# (base workload, overrides): each case smaller than the one before
CALLS = [
    ("mixtral_t512", dict(T=200, d=256, F=320)),                                  # bf16, router routing
    ("tiny_f32", dict(T=37, d=128, F=192)),                                       # fp32, smaller
    ("capacity_gini0.30", dict(T=24, d=128, E=8, k=2, F=128, capacity=5)),        # bf16, overflow pass
]


def _layer(M, wl, inp, noalloc):
    dt = torch_dtype(wl.dtype)
    shape = M.Shape(wl.T, wl.d, wl.E, wl.k, wl.F, wl.capacity, dt)
    out = torch.full((wl.T, wl.d), float("nan"), dtype=dt, device="cuda")
    args = (shape, dev(inp.x), dev(inp.wr), dev(inp.bias), dev(inp.topk_ids), dev(inp.topk_w), dev(inp.wg),
            dev(inp.wu), dev(inp.wd), out)
    if noalloc:
        M.moe_forward_noalloc(*args)
        ids = None
    else:
        ws = M.workspace(M.workspace_size(shape))
        v = M.moe_forward(*args, ws)
        ids = v.topk_ids
    torch.cuda.synchronize()
    return out, ids


def test_noalloc_matches_forward_on_shrinking_calls():
    import grouped_gemm_gemv_amd as M
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for base, over in CALLS:
        wl = get_workload(base, **over)
        print(f"\n[gpu noalloc] {base} {over}", flush=True)
        inp = make_inputs(wl, 0)
        got, _ = _layer(M, wl, inp, noalloc=True)
        ref, ids = _layer(M, wl, inp, noalloc=False)
        assert np.array_equal(bits(got), bits(ref))
        ids = ids.cpu().numpy()
        if inp.topk_ids is None:
            lg = O.router_logits(inp.x, inp.wr, wl.dtype, inp.bias)
            p = np.exp(lg - lg.max(axis=1, keepdims=True))
            sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
            w = sel / sel.sum(axis=1, keepdims=True)
        else:
            w = inp.topk_w
        o = O.forward(inp.x, inp.wr, inp.wg, inp.wu, inp.wd, wl.k, wl.dtype, topk_ids=ids, topk_w=w,
                      capacity=wl.capacity)["out"]
        err = rel_err(host64(got), o)
        print(f"[gpu noalloc] {base}: bitwise equal to moe_forward, rel err vs oracle {err:.3e}", flush=True)
        assert err <= TOL[wl.dtype]


def test_noalloc_rejects_shapes_past_the_scratch_size():
    import grouped_gemm_gemv_amd as M
    from grouped_gemm_gemv_amd._lib import NOALLOC_SCRATCH_BYTES, MoeError
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    shape = M.Shape(512, 4096, 8, 2, 14336 * 4, 0, torch.bfloat16)
    assert M.workspace_size(shape) > NOALLOC_SCRATCH_BYTES
    x = torch.zeros((512, 4096), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda")  # never read: rejected before any launch
    with pytest.raises(MoeError, match="WORKSPACE_TOO_SMALL"):
        M.moe_forward_noalloc(shape, x, w, None, None, None, w, w, w, x)
