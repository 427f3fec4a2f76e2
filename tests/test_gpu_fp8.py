"""GPU parity of the fp8-weight path (OCP E4M3 codes, one fp32 scale per
output channel, bf16 activations) against the oracle's dequantised weights.

Small cases span several row and column tiles, ragged tails, every tile
height family (split-K short tiles, 96, the 112-column 160 tile, 192, 384),
capacity mode and skewed routing; full-size cases check every token, and h
and y_perm on every row of the busiest expert.
Tolerance: max|gpu - oracle| / max|oracle| <= 2e-2 (bf16 activations; the
oracle uses the same quantised weights, so quantisation error is not part
of the comparison).
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.gpu_helpers import TOL, bits, check_dispatch, check_routing, dev, host64, rel_err
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# name: (base workload, overrides, tile rows (0 = automatic))
CASES = {
    "fp8_ragged": ("mixtral_t512_fp8", dict(T=200, d=256, F=320), 0),
    "fp8_bm16": ("mixtral_t512_fp8", dict(T=24, d=256, F=320), 16),
    "fp8_bm48": ("mixtral_t512_fp8", dict(T=152, d=128, F=128), 48),
    "fp8_bm96": ("mixtral_t512_fp8", dict(T=256, d=128, F=192), 96),
    "fp8_bm160": ("mixtral_t512_fp8", dict(T=512, d=256, F=128), 160),
    "fp8_bm192": ("mixtral_t512_fp8", dict(T=512, d=128, E=4, F=192), 192),
    "fp8_t1": ("mixtral_t512_fp8", dict(T=1, d=256, F=320), 0),  # the combine inside the down GEMM
    # ping-pong main loops: gate+up on 192-row tiles with a K loop longer than
    # its prefetch depth, and both GEMMs on 384-row tiles (K loops of 3 and 5
    # steps: tails of 1 and 2 past whole rounds)
    "fp8_bm192_long_k": ("mixtral_t512_fp8", dict(T=700, d=320, E=3, F=192), 192),
    "fp8_bm384": ("mixtral_t512_fp8", dict(T=900, d=192, E=2, F=320), 384),
    "fp8_capacity": ("capacity_gini0.30", dict(T=300, d=128, E=16, k=4, F=192, capacity=40, weights="e4m3"), 0),
    "fp8_e64_zipf2": ("e64_zipf_a2.0", dict(T=160, d=128, F=192, weights="e4m3"), 0),
}


def _fp8(inp):
    return (O.Fp8Weights(inp.wg, inp.sg), O.Fp8Weights(inp.wu, inp.su), O.Fp8Weights(inp.wd, inp.sd))


class Run:
    def __init__(self, case):
        import grouped_gemm_gemv_amd as M
        base, over, bm = CASES[case]
        wl = get_workload(base, **over)
        assert wl.weights == "e4m3" and wl.dtype == "bf16"
        self.wl = wl
        self.inp = inp = make_inputs(wl, 0)
        self.shape = M.Shape(wl.T, wl.d, wl.E, wl.k, wl.F, wl.capacity, torch.bfloat16, bm)
        self.q = M.query(self.shape)
        d = {n: dev(getattr(inp, n)) for n in ("x", "wr", "bias", "wg", "wu", "wd", "sg", "su", "sd",
                                               "topk_ids", "topk_w")}
        self.d = d
        ws = M.workspace(self.q.forward_ws_bytes)
        self.out = torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device="cuda")
        self.v = M.moe_forward_fp8(self.shape, d["x"], d["wr"], d["bias"], d["topk_ids"], d["topk_w"], d["wg"],
                                   d["wu"], d["wd"], d["sg"], d["su"], d["sd"], self.out, ws)
        torch.cuda.synchronize()
        self.ws = ws
        self.gpu_ids = self.v.topk_ids.cpu().numpy()
        self.gpu_w = self.v.topk_w.cpu().numpy().astype(np.float64)
        self.ref_disp = O.dispatch(self.gpu_ids, wl.E, wl.capacity, self.q.tile_rows)
        self.y_gpu = host64(self.v.y_perm)


@pytest.fixture(scope="module")
def runs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cache = {}

    def get(case):
        if case not in cache:
            print(f"\n[gpu fp8] case {case} {CASES[case]}", flush=True)
            cache[case] = Run(case)
        return cache[case]
    return get


@pytest.mark.parametrize("case", sorted(CASES))
def test_fp8_layer_output(runs, case):
    r = runs(case)
    wl = r.wl
    check_dispatch(r.v.disp.arrays(), r.ref_disp, wl.E)
    wg, wu, wd = _fp8(r.inp)
    ref = O.forward(r.inp.x, r.inp.wr, wg, wu, wd, wl.k, wl.dtype, r.inp.bias, topk_ids=r.gpu_ids,
                    topk_w=r.gpu_w, capacity=wl.capacity, tile_rows=r.q.tile_rows)
    live = r.ref_disp["token_of"] >= 0
    ey = rel_err(r.y_gpu[live], ref["y"][live])
    eo = rel_err(host64(r.out), ref["out"])
    print(f"[gpu fp8] {case}: tile rows {r.q.tile_rows}, y rel err {ey:.2e}, out rel err {eo:.2e}")
    assert ey <= TOL["bf16"] and eo <= TOL["bf16"]


@pytest.mark.parametrize("case", ["fp8_ragged", "fp8_capacity", "fp8_bm16", "fp8_t1"])
def test_fp8_forward_equals_steps_and_repeats(runs, case):
    import grouped_gemm_gemv_amd as M
    r = runs(case)
    wl, d = r.wl, r.d
    R = r.q.rows
    h = torch.zeros((R, wl.F), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((R, wl.d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(r.out)
    for p in range(r.q.n_passes):
        M.moe_ffn_gate_up_fp8(r.shape, d["x"], d["wg"], d["wu"], d["sg"], d["su"], r.v.disp, p, h)
        M.moe_ffn_down_fp8(r.shape, h, d["wd"], d["sd"], r.v.disp, p, y)
    M.moe_combine(r.shape, y, r.v.topk_w, r.v.disp, out)
    out2 = torch.empty_like(r.out)
    ws2 = M.workspace(r.q.forward_ws_bytes)
    M.moe_forward_fp8(r.shape, d["x"], d["wr"], d["bias"], d["topk_ids"], d["topk_w"], d["wg"], d["wu"], d["wd"],
                      d["sg"], d["su"], d["sd"], out2, ws2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(r.out))
    assert np.array_equal(bits(out2), bits(r.out))


def test_fp8_rejects_f32_activations():
    import grouped_gemm_gemv_amd as M
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    shape = M.Shape(8, 64, 4, 2, 64, 0, torch.float32)
    x = torch.zeros((8, 64), device="cuda")
    c = torch.zeros((4, 64, 64), dtype=torch.uint8, device="cuda")
    s = torch.ones((4, 64), device="cuda")
    ws = M.workspace(M.query(shape).forward_ws_bytes)
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        M.moe_forward_fp8(shape, x, None, None, torch.zeros((8, 2), dtype=torch.int32, device="cuda"),
                          torch.ones((8, 2), device="cuda"), c, c, c, s, s, s, torch.empty_like(x), ws)


FULL = ["mixtral_t512_fp8", "mixtral_decode_t1_fp8", "mixtral_decode_t8_fp8", "mixtral_decode_t32_fp8",
        "mixtral_decode_t128_fp8", "mixtral_decode_t256_fp8"]


@pytest.fixture(scope="module")
def full_weights():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = get_workload("mixtral_t512_fp8")
    inp = make_inputs(wl, 0)
    return inp, tuple(dev(getattr(inp, n)) for n in ("wg", "wu", "wd", "sg", "su", "sd"))


@pytest.mark.parametrize("name", FULL)
def test_fp8_fullsize(full_weights, name):
    import grouped_gemm_gemv_amd as M
    wl = get_workload(name)
    print(f"\n[gpu fp8 fullsize] {name}: T={wl.T}", flush=True)
    winp, dw = full_weights
    inp = make_inputs(wl, 0, experts=False)
    shape = M.Shape(wl.T, wl.d, wl.E, wl.k, wl.F, 0, torch.bfloat16)
    q = M.query(shape)
    ws = M.workspace(q.forward_ws_bytes)
    out = torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device="cuda")
    v = M.moe_forward_fp8(shape, dev(inp.x), dev(inp.wr), None, None, None, *dw, out, ws)
    torch.cuda.synchronize()
    ids = v.topk_ids.cpu().numpy()
    w = v.topk_w.cpu().numpy().astype(np.float64)
    differ = check_routing(ids, w, O.router_logits(inp.x, inp.wr, wl.dtype), wl.k)
    assert differ <= max(1, wl.T // 200), differ
    ref_disp = O.dispatch(ids, wl.E, 0, q.tile_rows)
    check_dispatch(v.disp.arrays(), ref_disp, wl.E)
    ow = _fp8(winp)
    e = int(np.argmax(ref_disp["counts"]))
    rows, h_ref, y_ref = O.expert_rows(inp.x, *ow, wl.dtype, ref_disp, e)
    idx = torch.from_numpy(rows).cuda()
    eh, ey = rel_err(host64(v.h[idx]), h_ref), rel_err(host64(v.y_perm[idx]), y_ref)
    print(f"[gpu fp8 fullsize] {name}: expert {e}, {rows.size} rows: h rel err {eh:.3e}, y_perm {ey:.3e}",
          flush=True)
    assert eh <= TOL["bf16"] and ey <= TOL["bf16"], (eh, ey)
    ref = O.forward(inp.x, inp.wr, *ow, wl.k, wl.dtype, topk_ids=ids, topk_w=w)["out"]
    err = rel_err(host64(out), ref)
    print(f"[gpu fp8 fullsize] {name}: all {wl.T} tokens rel err {err:.3e}, tile rows {q.tile_rows}", flush=True)
    assert err <= TOL["bf16"]
