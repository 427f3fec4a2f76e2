"""Blocked 16-row weight storage (MOE_LAYOUT_BLOCKED16).

moe_pack_blocked16 must equal the layout's definition byte for byte, and
every layer computed from blocked weights must be bitwise equal to the same
layer from row-major weights (the GEMMs read the same values into the same
MFMA operands; only the addresses change), across tile families, dtypes,
fp8 weights, capacity mode and the full Mixtral-shaped layer.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.gpu_helpers import bits, dev, torch_dtype
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("shape,dt", [((1, 16, 64), np.uint8), ((3, 48, 192), np.uint8), ((2, 32, 320), np.int16),
                                      ((5, 64, 96), np.float32), ((1, 14336 // 16 * 16, 4096), np.int16)])
def test_pack_matches_definition(shape, dt):
    _need_gpu()
    import grouped_gemm_gemv_amd as M
    print(f"\n[gpu layout] pack {shape} {dt.__name__}", flush=True)
    rng = np.random.default_rng(sum(shape))
    a = rng.integers(-100, 100, size=shape).astype(dt)
    out = M.moe_pack_blocked16(torch.from_numpy(a).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), O.blocked16(a))


CASES = {
    "bf16_auto": ("mixtral_t512", dict(T=200, d=256, F=320), 0),
    "bf16_bm16": ("mixtral_t512", dict(T=24, d=256, F=320), 16),
    "bf16_bm48": ("mixtral_t512", dict(T=152, d=128, F=128), 48),
    "bf16_bm96": ("mixtral_t512", dict(T=256, d=128, F=192), 96),
    "bf16_bm160": ("mixtral_t512", dict(T=512, d=256, F=128), 160),
    "bf16_bm192": ("mixtral_t512", dict(T=512, d=128, E=4, F=192), 192),
    "bf16_capacity": ("capacity_gini0.30", dict(T=300, d=128, E=16, k=4, F=192, capacity=40), 0),
    "bf16_zipf2": ("e64_zipf_a2.0", dict(T=160, d=128, F=192), 0),
    "f32_tiny": ("tiny_f32", {}, 0),
    "fp8_auto": ("mixtral_t512_fp8", dict(T=200, d=256, F=320), 0),
    "fp8_bm16": ("mixtral_t512_fp8", dict(T=24, d=256, F=320), 16),
    "fp8_capacity": ("capacity_gini0.30", dict(T=300, d=128, E=16, k=4, F=192, capacity=40, weights="e4m3"), 0),
}


def _forward(M, wl, inp, shape, w, ws, out):
    d = {n: dev(getattr(inp, n)) for n in ("x", "wr", "bias", "topk_ids", "topk_w")}
    if wl.weights == "e4m3":
        M.moe_forward_fp8(shape, d["x"], d["wr"], d["bias"], d["topk_ids"], d["topk_w"], *w, out, ws)
    else:
        M.moe_forward(shape, d["x"], d["wr"], d["bias"], d["topk_ids"], d["topk_w"], *w, out, ws)
    torch.cuda.synchronize()
    return bits(out)


def _compare(wl, inp, bm):
    import grouped_gemm_gemv_amd as M
    dt = torch_dtype(wl.dtype)
    names = ("wg", "wu", "wd", "sg", "su", "sd") if wl.weights == "e4m3" else ("wg", "wu", "wd")
    w_rows = [dev(getattr(inp, n)) for n in names]
    w_blk = [M.moe_pack_blocked16(t) if t.dim() == 3 else t for t in w_rows]
    res = []
    for layout, w in ((0, w_rows), (1, w_blk)):
        shape = M.Shape(wl.T, wl.d, wl.E, wl.k, wl.F, wl.capacity, dt, bm, layout)
        ws = M.workspace(M.query(shape).forward_ws_bytes)
        out = torch.empty((wl.T, wl.d), dtype=dt, device="cuda")
        res.append(_forward(M, wl, inp, shape, w, ws, out))
    return res


@pytest.mark.parametrize("case", sorted(CASES))
def test_blocked_forward_equals_row_major(case):
    _need_gpu()
    base, over, bm = CASES[case]
    wl = get_workload(base, **over)
    print(f"\n[gpu layout] {case}", flush=True)
    a, b = _compare(wl, make_inputs(wl, 0), bm)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["mixtral_t512", "mixtral_t512_fp8"])
def test_blocked_fullsize_equals_row_major(name):
    _need_gpu()
    wl = get_workload(name)
    print(f"\n[gpu layout] full size {name}", flush=True)
    a, b = _compare(wl, make_inputs(wl, 0), 0)
    assert np.array_equal(a, b)
