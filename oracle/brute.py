"""Scalar brute-force MoE layer for tiny inputs (test infrastructure only).

A second, independent statement of the same definition as moe_oracle, written
with plain Python loops and scalar arithmetic, so that the vectorised oracle
can be pinned against it on small shapes.  Inputs are float64 nested lists or
arrays; bf16 decoding is done by the caller.
"""
from __future__ import annotations

import math
from typing import Dict, List


def route(x, wr, k: int, bias=None):
    """Router logits by explicit dot products; k rounds of argmax (strictly
    greater wins, scanning experts in ascending order, so the lowest index
    wins a tie); softmax over all experts; renormalise the k kept values."""
    T, E, d = len(x), len(wr), len(wr[0])
    ids: List[List[int]] = []
    ws: List[List[float]] = []
    for t in range(T):
        lg = []
        for e in range(E):
            s = 0.0
            for i in range(d):
                s += float(x[t][i]) * float(wr[e][i])
            if bias is not None:
                s += float(bias[e])
            lg.append(s)
        taken = [False] * E
        sel = []
        for _ in range(k):
            best = -1
            for e in range(E):
                if not taken[e] and (best < 0 or lg[e] > lg[best]):
                    best = e
            taken[best] = True
            sel.append(best)
        mx = max(lg)
        z = sum(math.exp(v - mx) for v in lg)
        p = [math.exp(lg[e] - mx) / z for e in sel]
        sp = sum(p)
        ids.append(sel)
        ws.append([v / sp for v in p])
    return ids, ws


def dispatch(ids, E: int, capacity: int, tile_rows: int) -> Dict[str, list]:
    """Counts, offsets and stable ranks by scanning; capacity split; tile lists."""
    T, k = len(ids), len(ids[0])
    flat = [int(ids[t][j]) for t in range(T) for j in range(k)]
    Tk = len(flat)
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + counts[e])
    rank = []
    for f in range(Tk):
        rank.append(sum(1 for g in range(f) if flat[g] == flat[f]))
    C = capacity
    if C > 0:
        spill = [max(0, counts[e] - C) for e in range(E)]
    else:
        spill = [0] * E
    spill_off = [0]
    for e in range(E):
        spill_off.append(spill_off[-1] + spill[e])
    if C > 0:
        R = E * C + max(0, Tk - C)
        row_of = []
        for f in range(Tk):
            e, q = flat[f], rank[f]
            row_of.append(e * C + q if q < C else E * C + spill_off[e] + q - C)
        bases = [[e * C for e in range(E)], [E * C + spill_off[e] for e in range(E)]]
        rows = [[min(counts[e], C) for e in range(E)], spill]
    else:
        R = Tk
        row_of = [offsets[flat[f]] + rank[f] for f in range(Tk)]
        bases = [offsets[:E], [0] * E]
        rows = [counts, [0] * E]
    token_of = [-1] * R
    for f in range(Tk):
        token_of[row_of[f]] = f // k
    tile_off = [[0], [0]]
    tile_map = [[], []]
    for p in range(2):
        for e in range(E):
            r0, left, i = bases[p][e], rows[p][e], 0
            while left > 0:
                n = min(tile_rows, left)
                tile_map[p].append((e, r0, n, i))
                r0 += n
                left -= n
                i += 1
            tile_off[p].append(len(tile_map[p]))
    return {"counts": counts, "offsets": offsets, "spill_counts": spill,
            "spill_offsets": spill_off, "rank": rank, "row_of": row_of,
            "token_of": token_of, "R": R, "tile_off": tile_off, "tile_map": tile_map}


def hidden(xrow, wg, wu):
    """The SwiGLU intermediate of one token for one expert, with explicit loops."""
    F, d = len(wg), len(xrow)
    h = []
    for n in range(F):
        g = 0.0
        u = 0.0
        for i in range(d):
            g += float(wg[n][i]) * float(xrow[i])
            u += float(wu[n][i]) * float(xrow[i])
        h.append(g / (1.0 + math.exp(-g)) * u)
    return h


def expert(xrow, wg, wu, wd):
    """One token through one SwiGLU expert with explicit loops."""
    F = len(wg)
    h = hidden(xrow, wg, wu)
    y = []
    for o in range(len(wd)):
        s = 0.0
        for n in range(F):
            s += float(wd[o][n]) * h[n]
        y.append(s)
    return y


def forward(x, wr, wg, wu, wd, k: int, bias=None, ids=None, w=None,
            capacity: int = 0, tile_rows: int = 16):
    """Whole layer; every (token, slot) pair is evaluated on its own."""
    if ids is None:
        ids, w = route(x, wr, k, bias)
    E = len(wr)
    disp = dispatch(ids, E, capacity, tile_rows)
    T, d = len(x), len(x[0])
    out = [[0.0] * d for _ in range(T)]
    for t in range(T):
        for j in range(k):
            y = expert(x[t], wg[ids[t][j]], wu[ids[t][j]], wd[ids[t][j]])
            for i in range(d):
                out[t][i] += float(w[t][j]) * y[i]
    return {"ids": ids, "w": w, "disp": disp, "out": out}
