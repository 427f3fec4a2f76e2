"""Shared helpers of the GPU tests: moving seeded inputs to the device and
comparing GPU results with the oracle under the stated tolerances."""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as O

# Layer-output tolerance: max|gpu - oracle| / max|oracle|.
TOL = {"bf16": 2e-2, "f32": 1e-4}
# Routing: ids may differ only where the oracle's logits are within this gap.
NEAR_TIE = 1e-4


def torch_dtype(dt: str):
    import torch
    return torch.bfloat16 if dt == "bf16" else torch.float32


def dev(a: np.ndarray, dt: str = None):
    """numpy (bf16 bits as uint16, or fp32/int32) -> contiguous device tensor."""
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bits(t) -> np.ndarray:
    """Raw bit patterns of a device tensor (for bitwise comparisons)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy()
    return t.cpu().numpy()


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    den = np.abs(ref).max()
    return float(np.abs(gpu - ref).max() / (den if den > 0 else 1.0))


def check_routing(gpu_ids: np.ndarray, gpu_w: np.ndarray, logits: np.ndarray, k: int):
    """GPU top-k agrees with the oracle's logits except at near-ties; weights
    equal the renormalised softmax at the GPU's ids.  Returns #tokens whose
    ids differ from the oracle's selection."""
    T, E = logits.shape
    o_ids, _ = O.route_from_logits(logits, k)
    differ = 0
    for t in range(T):
        g = gpu_ids[t]
        assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < E, (t, g)
        lg = logits[t]
        sel = lg[g]
        # slot order: non-increasing up to near-ties
        assert (np.diff(sel) <= NEAR_TIE).all(), (t, sel)
        rest = np.setdiff1d(np.arange(E), g)
        if rest.size:
            assert sel.min() >= lg[rest].max() - NEAR_TIE, (t, sel, lg[rest].max())
        if not np.array_equal(g, o_ids[t]):
            differ += 1
    # weights at the GPU's ids
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    sel = np.take_along_axis(p, gpu_ids.astype(np.int64), axis=1)
    w_ref = sel / sel.sum(axis=1, keepdims=True)
    assert np.abs(gpu_w - w_ref).max() <= 2e-6, np.abs(gpu_w - w_ref).max()
    return differ


def check_dispatch(arr: dict, ref: dict, E: int):
    """Integer dispatch outputs must be bit-exact."""
    for key in ("counts", "offsets", "spill_counts", "spill_offsets", "row_of", "token_of"):
        g = arr[key].cpu().numpy()
        assert np.array_equal(g, ref[key]), key
    n_tiles = arr["n_tiles"].cpu().numpy()
    assert np.array_equal(n_tiles, ref["n_tiles"]), (n_tiles, ref["n_tiles"])
    tile_off = arr["tile_off"].cpu().numpy()
    tile_map = arr["tile_map"].cpu().numpy()
    for p in (0, 1):
        assert np.array_equal(tile_off[p], ref["tile_off"][p]), p
        assert np.array_equal(tile_map[p][:n_tiles[p]], ref["tile_map"][p]), p
    assert int(arr["err_flags"].cpu().numpy()[0]) == 0
