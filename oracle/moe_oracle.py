"""CPU oracle for the single-GPU MoE layer forward pass.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct
reference the GPU library is checked against.  Only the test suite, the
package smoke check and the CPU-baseline leg of the benchmark may import it;
the library itself never does, and nothing here is shared with the GPU path.

Everything is computed in float64 from the plain definition of a top-k routed
SwiGLU mixture-of-experts layer:

* router scoring, permutation, expert GEMMs and weighted unpermutation are the
  five stages named in the TritonMoE review (pith.science verdict for arXiv
  2605.23911, referee summary and desk-editor letter); the expert FFN is the
  SwiGLU form (SiLU on the gate projection, product with the up projection,
  then the down projection) named in that review's key machinery;
* the capacity-bounded dispatch with an overflow ("spill") pass follows the
  Cap-and-Spill critique (juhe.plus blog, section "Cap-and-Spill"): a first
  pass of at most C tokens per expert, the overflow compacted into one
  contiguous buffer whose size is bounded in advance, and no token dropped;
* the tile map is the block schedule of the TritonMoE review (Algorithm 1,
  section 3.2): fixed-size row blocks mapped to (expert, row offset) pairs.

Where the pages leave a step open, the reading taken is stated at the
function that takes it.  Every function here is pinned by the CPU tests
against closed forms, textbook values, special cases and a scalar
brute-force re-implementation (oracle/brute.py).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# Input decoding
# ----------------------------------------------------------------------------

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of the stored input to float64.

    dtype "bf16": `a` holds bf16 bit patterns (uint16); a bf16 value is the
    fp32 value whose upper 16 bits are those bits and lower 16 bits are zero.
    dtype "f32": `a` holds fp32 values.
    """
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Value of OCP 8-bit floating point E4M3 codes, from the format's definition.

    Bit 7 is the sign, bits 6..3 the exponent field E (bias 7), bits 2..0 the
    mantissa M.  E = 0: subnormal, (M / 8) * 2^-6.  E >= 1: (1 + M / 8) *
    2^(E - 7).  E = 15 with M = 7 (0x7F, 0xFF) is NaN; there is no infinity, so
    the largest finite magnitude is (1 + 6/8) * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = sign * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


_E4M3_VALUES = e4m3_to_f64(np.arange(256, dtype=np.uint8))


class Fp8Weights:
    """Expert weights stored as E4M3 codes with one scale per output channel.

    codes [E, N, K] uint8 and scales [E, N] fp32 stand for the matrices
    W[e, n, i] = scales[e, n] * e4m3(codes[e, n, i]).  The pages name an fp8
    grouped GEMM (TEMPO review, referee summary) without fixing the format or
    the scale granularity; per-output-channel scaling is the reading taken.
    """

    def __init__(self, codes: np.ndarray, scales: np.ndarray):
        self.codes = np.asarray(codes, dtype=np.uint8)
        self.scales = np.asarray(scales, dtype=np.float32)
        assert self.codes.ndim == 3 and self.scales.shape == self.codes.shape[:2]

    @property
    def shape(self):
        return self.codes.shape

    def expert(self, e: int) -> np.ndarray:
        """W[e] in float64 (every product of a code value and an fp32 scale is exact).

        The codes are looked up in the values of all 256 codes, each from
        e4m3_to_f64: the same definition, evaluated once per code value."""
        return self.scales[e].astype(np.float64)[:, None] * _E4M3_VALUES[self.codes[e]]


def widen_expert(w, e: int, dtype: str) -> np.ndarray:
    """Weights of expert e in float64: stored values of `dtype`, or dequantised fp8."""
    if isinstance(w, Fp8Weights):
        return w.expert(e)
    return to_f64(w[e], dtype)


def blocked16(a: np.ndarray) -> np.ndarray:
    """Reference of the library's blocked 16-row weight storage order.

    Not a step of the layer: a byte order the GPU library accepts for its
    expert weights.  For every matrix [rows, row_bytes] (rows % 16 == 0,
    row_bytes % 64 == 0) the rows are taken in groups of 16 and each group is
    written as consecutive 1024-byte blocks, block c holding bytes
    [64c, 64c + 64) of the group's 16 rows in row order.  `a` is any array
    whose last two axes are (rows, K); the result has the same shape and
    dtype and holds the reordered bytes.
    """
    a = np.ascontiguousarray(a)
    b = a.view(np.uint8).reshape(-1, a.shape[-2], a.shape[-1] * a.itemsize)
    m, rows, rb = b.shape
    out = b.reshape(m, rows // 16, 16, rb // 64, 64).transpose(0, 1, 3, 2, 4)
    return np.ascontiguousarray(out).reshape(-1).view(a.dtype).reshape(a.shape)


# ----------------------------------------------------------------------------
# Step 1: routing
# ----------------------------------------------------------------------------

def router_logits(x: np.ndarray, wr: np.ndarray, dtype: str,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """logits[t, e] = sum_i x[t, i] * Wr[e, i] (+ bias[e]), in float64."""
    lg = to_f64(x, dtype) @ to_f64(wr, dtype).T
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return lg


def route_from_logits(logits: np.ndarray, k: int):
    """Top-k softmax routing of one batch of router logits.

    Reading taken (the TritonMoE review names only "router scoring"):
    probabilities are a softmax over all E experts; each token keeps the k
    experts with the largest logits (equal logits: the lower expert index
    first); slot j holds the j-th largest; the kept probabilities are
    renormalised to sum to one.  Selecting on logits or on probabilities picks
    the same experts (softmax is increasing); logits avoid ties created by
    rounding in exp.

    Returns ids [T, k] int32 and weights [T, k] float64.
    """
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # stable sort of -logit: equal logits keep ascending expert index.
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids, axis=1)
    w = sel / sel.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w


def route(x, wr, k: int, dtype: str, bias=None):
    """Router scoring followed by top-k softmax routing (see route_from_logits)."""
    lg = router_logits(x, wr, dtype, bias)
    ids, w = route_from_logits(lg, k)
    return ids, w, lg


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token: (k-th largest logit) - ((k+1)-th largest logit); +inf if k == E."""
    T, E = logits.shape
    s = -np.sort(-logits, axis=1)
    if k >= E:
        return np.full(T, np.inf)
    return s[:, k - 1] - s[:, k]


# ----------------------------------------------------------------------------
# Steps 2-4: count, exclusive scan, stable permutation, capacity split, tiles
# ----------------------------------------------------------------------------

def spill_rows_bound(T: int, k: int, capacity: int) -> int:
    """Rows reserved for the overflow region in capacity mode: max(0, T*k - C).

    Bound: if no expert exceeds C the overflow is empty.  Otherwise, with
    n_e the per-expert counts (sum n_e = T*k) and S the experts with n_e > C,
    sum_e max(0, n_e - C) = sum_{e in S} n_e - C*|S| <= T*k - C*|S| <= T*k - C.
    """
    return max(0, T * k - capacity)


def row_space(T: int, k: int, E: int, capacity: int) -> int:
    """Number of rows of the permuted buffers: T*k uncapped, E*C + spill bound with capacity C."""
    if capacity <= 0:
        return T * k
    return E * capacity + spill_rows_bound(T, k, capacity)


def max_tiles(T: int, k: int, E: int, capacity: int, tile_rows: int, pass_idx: int) -> int:
    """Upper bound on the number of row tiles of one pass (sizes the static grid).

    A pass covering R_p rows over at most E_p non-empty experts has
    sum_e ceil(r_e / BM) <= (R_p + E_p * (BM - 1)) / BM tiles.
    """
    BM = tile_rows
    Tk = T * k
    if capacity <= 0:
        if pass_idx == 1:
            return 0
        Rp, Ep = Tk, min(E, Tk)
        return (Rp + Ep * (BM - 1)) // BM
    C = capacity
    if pass_idx == 0:
        Rp, Ep = min(Tk, E * C), min(E, Tk)
        return min((Rp + Ep * (BM - 1)) // BM, E * ((C + BM - 1) // BM))
    Rp = spill_rows_bound(T, k, C)
    Ep = min(E, Tk // (C + 1))  # an overflowing expert holds at least C+1 entries
    return (Rp + Ep * (BM - 1)) // BM


def dispatch(ids: np.ndarray, E: int, capacity: int = 0, tile_rows: int = 16) -> Dict[str, np.ndarray]:
    """Count, scan, stable permutation, capacity split and tile map.

    Flat index f = t*k + j names slot j of token t.

    * counts[e] = number of f with ids[f] == e; offsets = exclusive scan.
    * Stable order (reading of "stable permutation"): within each expert the
      entries are kept in ascending f, i.e. ascending token.  rank(f) is the
      position of f inside its expert in that order.
    * Uncapped: row_of[f] = offsets[e] + rank(f).
    * Capacity C > 0 (Cap-and-Spill critique): the first C entries of an
      expert in stable order go to the fixed region, row e*C + rank; the rest,
      in the same order, go to the overflow region, compacted across experts:
      row E*C + spill_offsets[e] + (rank - C), where spill_offsets is the
      exclusive scan of o_e = max(0, n_e - C).  Reading taken: "the first C"
      means the first C in stable order (the critique's "top 16 tokens" does
      not say by what).  Nothing is dropped.
    * token_of[row] = f div k for live rows, -1 for rows no entry maps to.
    * Tile map, per pass (pass 0: uncapped rows or fixed region; pass 1:
      overflow region): expert e's rows of that pass are cut into
      ceil(r_e / BM) tiles of BM rows; tiles are listed expert by expert;
      entry = (expert, first row, rows in tile, tile index within expert);
      tile_off is the exclusive scan of tiles per expert.

    Ids outside [0, E) are a precondition violation and raise.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    Tk = flat.size
    T, k = np.asarray(ids).shape
    if Tk and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    C = int(capacity)
    counts = np.zeros(E, dtype=np.int64)
    for f in range(Tk):
        counts[flat[f]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    # stable order: a stable sort of the flat ids keeps ascending f per expert
    order = np.argsort(flat, kind="stable")
    rank = np.empty(Tk, dtype=np.int64)
    rank[order] = np.arange(Tk) - offsets[flat[order]]
    if C > 0:
        spill = np.maximum(counts - C, 0)
        kept = np.minimum(counts, C)
    else:
        spill = np.zeros(E, dtype=np.int64)
        kept = counts.copy()
    spill_off = np.zeros(E + 1, dtype=np.int64)
    spill_off[1:] = np.cumsum(spill)
    R = row_space(T, k, E, C)
    if C > 0:
        assert spill_off[E] <= spill_rows_bound(T, k, C)
        in_fixed = rank < C
        row_of = np.where(in_fixed, flat * C + rank, E * C + spill_off[flat] + (rank - C))
        base = [np.arange(E) * C, E * C + spill_off[:E]]
        rows = [kept, spill]
    else:
        row_of = offsets[flat] + rank
        base = [offsets[:E], np.zeros(E, dtype=np.int64)]
        rows = [counts, np.zeros(E, dtype=np.int64)]
    token_of = np.full(R, -1, dtype=np.int64)
    token_of[row_of] = np.arange(Tk) // k
    BM = int(tile_rows)
    tile_off = np.zeros((2, E + 1), dtype=np.int64)
    tile_map = []
    for p in range(2):
        tiles = []
        for e in range(E):
            nt = -(-int(rows[p][e]) // BM)
            for i in range(nt):
                r0 = int(base[p][e]) + i * BM
                tiles.append((e, r0, min(BM, int(rows[p][e]) - i * BM), i))
            tile_off[p, e + 1] = tile_off[p, e] + nt
        tile_map.append(np.array(tiles, dtype=np.int64).reshape(-1, 4))
    return {
        "counts": counts, "offsets": offsets, "spill_counts": spill,
        "spill_offsets": spill_off, "kept_counts": kept,
        "rank": rank, "row_of": row_of, "token_of": token_of, "R": R,
        "pass_base": np.stack(base), "pass_rows": np.stack(rows),
        "tile_off": tile_off, "tile_map": tile_map,
        "n_tiles": np.array([len(tile_map[0]), len(tile_map[1])]),
    }


def gather(x: np.ndarray, disp: Dict[str, np.ndarray]) -> np.ndarray:
    """x_perm[row] = x[token_of[row]] for live rows; dead rows stay zero (values copied, not rounded)."""
    tok = disp["token_of"]
    out = np.zeros((disp["R"],) + x.shape[1:], dtype=x.dtype)
    live = tok >= 0
    out[live] = x[tok[live]]
    return out


# ----------------------------------------------------------------------------
# Steps 5-6: expert FFN (SwiGLU) on the rows of each expert
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)) (written in the overflow-free split form)."""
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def swiglu_hidden(X: np.ndarray, wg: np.ndarray, wu: np.ndarray) -> np.ndarray:
    """One expert's SwiGLU intermediate: h = silu(Wg . x) * (Wu . x) for every row x of X.

    X [n, d], wg/wu [F, d], all float64.  No biases.
    """
    G = X @ wg.T
    U = X @ wu.T
    return silu(G) * U


def swiglu_ffn(X: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """One expert: y = Wd . (silu(Wg . x) * (Wu . x)) for every row x of X.

    X [n, d], wg/wu [F, d], wd [d, F], all float64.  No biases.
    """
    return swiglu_hidden(X, wg, wu) @ wd.T


def expert_rows(x, wg, wu, wd, dtype: str, disp, e: int):
    """Every live row of expert e with its intermediate and output.

    Returns (rows, h, y): the rows of the row space that expert e's entries
    occupy, in stable order (its fixed-region rows, then its overflow rows in
    capacity mode), h[i] = silu(Wg[e] . x) * (Wu[e] . x) and y[i] = Wd[e] . h[i]
    for x the token of rows[i], in float64 (no intermediate rounding).
    """
    tok = np.asarray(disp["token_of"])
    base, nrows = disp["pass_base"], disp["pass_rows"]
    rows = np.concatenate([base[p][e] + np.arange(nrows[p][e]) for p in range(2)]).astype(np.int64)
    X = to_f64(np.asarray(x)[tok[rows]], dtype)
    h = swiglu_hidden(X, widen_expert(wg, e, dtype), widen_expert(wu, e, dtype))
    return rows, h, h @ widen_expert(wd, e, dtype).T


def expert_outputs(x, wg, wu, wd, dtype: str, disp, ids) -> np.ndarray:
    """y[row] for every live row: the FFN of the row's expert applied to its token.

    The result of a (token, expert) pair does not depend on which region or
    pass holds its row: each expert's rows are evaluated together, in stable
    order, whatever the capacity.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    k = np.asarray(ids).shape[1]
    x64 = to_f64(x, dtype)
    d = x64.shape[1]
    y = np.zeros((disp["R"], d), dtype=np.float64)
    order = np.argsort(flat, kind="stable")
    off = disp["offsets"]
    for e in range(len(off) - 1):
        fs = order[off[e]:off[e + 1]]
        if fs.size == 0:
            continue
        X = x64[fs // k]
        Y = swiglu_ffn(X, widen_expert(wg, e, dtype), widen_expert(wu, e, dtype), widen_expert(wd, e, dtype))
        y[disp["row_of"][fs]] = Y
    return y


# ----------------------------------------------------------------------------
# Step 7: weighted combine
# ----------------------------------------------------------------------------

def combine(y: np.ndarray, w: np.ndarray, row_of: np.ndarray) -> np.ndarray:
    """out[t] = sum_{j=0..k-1} w[t, j] * y[row_of[t*k + j]], slots in ascending j."""
    T, k = w.shape
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    r = np.asarray(row_of).reshape(T, k)
    w64 = np.asarray(w, dtype=np.float64)
    for j in range(k):
        out += w64[:, j:j + 1] * y[r[:, j]]
    return out


# ----------------------------------------------------------------------------
# The whole layer
# ----------------------------------------------------------------------------

def forward(x, wr, wg, wu, wd, k: int, dtype: str, bias=None, topk_ids=None, topk_w=None,
            capacity: int = 0, tile_rows: int = 16) -> Dict[str, np.ndarray]:
    """Route (unless ids/weights are supplied), dispatch, expert FFN, combine.

    Returns a dict with the layer output "out" [T, d] float64 and every
    intermediate (ids, w, logits, dispatch arrays, y rows).
    """
    res: Dict[str, np.ndarray] = {}
    if topk_ids is None:
        ids, w, lg = route(x, wr, k, dtype, bias)
        res["logits"] = lg
    else:
        ids = np.asarray(topk_ids, dtype=np.int32)
        w = np.asarray(topk_w, dtype=np.float64)  # fp32 inputs widen exactly
    E = np.asarray(wr).shape[0]
    disp = dispatch(ids, E, capacity, tile_rows)
    y = expert_outputs(x, wg, wu, wd, dtype, disp, ids)
    res.update(ids=ids, w=w, disp=disp, y=y, out=combine(y, w, disp["row_of"]))
    return res


def forward_tokens(x, wg, wu, wd, dtype: str, ids, w, tokens: Sequence[int]) -> np.ndarray:
    """Layer output for a sample of tokens only, given their routing.

    out[t] = sum_j w[t, j] * FFN_{ids[t, j]}(x[t]) for t in `tokens`; used to
    check full-size runs one output row at a time.  Each expert's weights are
    widened once for all sampled (token, slot) pairs routed to it.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    ids = np.asarray(ids)
    w64 = np.asarray(w, dtype=np.float64)
    x64 = to_f64(np.asarray(x)[tokens], dtype)
    out = np.zeros((tokens.size, x64.shape[1]), dtype=np.float64)
    k = ids.shape[1]
    for e in np.unique(ids[tokens]):
        sel = [(i, j) for i, t in enumerate(tokens) for j in range(k) if ids[t, j] == e]
        if not sel:
            continue
        X = np.stack([x64[i] for i, _ in sel])
        Y = swiglu_ffn(X, widen_expert(wg, e, dtype), widen_expert(wu, e, dtype), widen_expert(wd, e, dtype))
        for (i, j), yrow in zip(sel, Y):
            out[i] += w64[tokens[i], j] * yrow
    return out


def gini(counts: np.ndarray) -> float:
    """Gini coefficient of per-expert counts: sum_i sum_j |n_i - n_j| / (2 E^2 mean(n)).

    Reading taken: the DODOCO abstract (fugumt.com summary of arXiv
    2605.20982) reports a "routing Gini" without defining it; this is the
    standard Gini of the E per-expert token counts.
    """
    n = np.asarray(counts, dtype=np.float64)
    E = n.size
    mu = n.mean()
    if mu == 0:
        return 0.0
    return float(np.abs(n[:, None] - n[None, :]).sum() / (2.0 * E * E * mu))
