"""Seeded generators for the MoE-layer inputs.

Every array has its own PCG64 stream, keyed by (seed, tag, expert), so any
subset of the inputs can be drawn without drawing the rest and the draws can
run in parallel threads.  Values are drawn in fp32; bf16 inputs are the
round-to-nearest-even bf16 encodings of those fp32 draws, carried as uint16
bit patterns so that the oracle and the GPU see identical bits.

Nothing here computes any step of the MoE layer.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

from .configs import Workload

_TAG_X, _TAG_WR, _TAG_WG, _TAG_WU, _TAG_WD, _TAG_BIAS, _TAG_ROUTE, _TAG_PERM = range(1, 9)


def _rng(seed: int, tag: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tag, sub)))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits.

    Finite inputs only (the generators never draw inf/nan).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).copy()
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(seed: int, tag: int, sub: int, shape, std: float, dtype: str) -> np.ndarray:
    a = _rng(seed, tag, sub).standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    a = a.reshape(shape)
    return bf16_bits_from_f32(a) if dtype == "bf16" else a


@dataclasses.dataclass
class Inputs:
    """Host arrays for one layer call.  bf16 tensors are uint16 bit patterns."""
    x: np.ndarray                      # [T, d]
    wr: np.ndarray                     # [E, d]
    bias: Optional[np.ndarray]         # [E] fp32, or None
    wg: Optional[np.ndarray]           # [E, F, d]
    wu: Optional[np.ndarray]           # [E, F, d]
    wd: Optional[np.ndarray]           # [E, d, F]
    topk_ids: Optional[np.ndarray]     # [T, k] int32 (supplied routing), or None
    topk_w: Optional[np.ndarray]       # [T, k] fp32 (supplied routing), or None
    sg: Optional[np.ndarray] = None    # [E, F] fp32 channel scales of wg (E4M3 weights), else None
    su: Optional[np.ndarray] = None    # [E, F]
    sd: Optional[np.ndarray] = None    # [E, d]


def e4m3_codes_from_f32(v: np.ndarray) -> np.ndarray:
    """OCP E4M3 codes of fp32 values: round to nearest, ties to even, saturating at +-448.

    E4M3: sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
    holds the subnormals m * 2^-9.  Used to synthesise fp8 weight inputs (a
    quantised checkpoint); the layer itself only reads codes.  Normal range:
    the fp32 mantissa is rounded to 3 bits on the bit pattern (adding
    0x7FFFF plus the lowest kept bit, then truncating, carries into the
    exponent when the rounding does); subnormal range: m = rint(|v| * 512).
    """
    v = np.asarray(v, dtype=np.float32)
    sign = ((v.view(np.uint32) >> np.uint32(24)) & np.uint32(0x80)).astype(np.int32)
    a = np.abs(v)
    au = a.view(np.uint32)
    r = au + np.uint32(0x7FFFF) + ((au >> np.uint32(20)) & np.uint32(1))
    normal = (((r >> np.uint32(23)).astype(np.int32) - 120) << 3) | ((r >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    sub = np.rint(np.minimum(a, np.float32(1.0)) * np.float32(512.0)).astype(np.int32)
    code = np.where(au < np.uint32(0x3C800000), sub, normal)  # 0x3C800000 = 2^-6
    return (np.minimum(code, 0x7E) | sign).astype(np.uint8)


def quantize_rows_e4m3(w: np.ndarray, block: int = 512):
    """Per-row (output channel) E4M3 quantisation of an fp32 matrix [N, K]:
    scale[n] = max_i |w[n, i]| / 448 (fp32), codes = E4M3(w / scale)."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = np.empty(w.shape, dtype=np.uint8)
    for r0 in range(0, w.shape[0], block):
        codes[r0:r0 + block] = e4m3_codes_from_f32(w[r0:r0 + block] / scale[r0:r0 + block, None])
    return codes, scale


def zipf_routing(T: int, E: int, k: int, alpha: float, seed: int):
    """Expert ids drawn per token without replacement from a Zipf(alpha) law
    over a seeded permutation of the experts, plus gate weights.

    Rank r (1-based) has mass proportional to r**-alpha.  Successive draws
    without replacement, each renormalising the mass that is left, are
    generated with the Gumbel-top-k equivalence: the order of the keys
    log(mass_r) + Gumbel_r, largest first, is distributed exactly as the
    successive draws.  Slot j holds the j-th draw.  Gate weights are a softmax
    of k standard-normal scores taken in draw order.
    """
    if k > E:
        raise ValueError("k > E")
    perm = _rng(seed, _TAG_PERM).permutation(E)
    r = _rng(seed, _TAG_ROUTE, 0)
    logmass = -alpha * np.log(np.arange(1, E + 1, dtype=np.float64))
    keys = logmass[None, :] + r.gumbel(size=(T, E))
    order = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    ids = perm[order].astype(np.int32)
    scores = _rng(seed, _TAG_ROUTE, 1).standard_normal((T, k))
    scores -= scores.max(axis=1, keepdims=True)
    ew = np.exp(scores)
    w = (ew / ew.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def make_inputs(wl: Workload, seed: int = 0, experts: bool = True,
                threads: Optional[int] = None, T: Optional[int] = None) -> Inputs:
    """Draw the inputs of workload `wl` at `seed`.

    experts=False skips the expert weights (routing-only uses).  `T` overrides
    the token count (the first T' rows of x are not a prefix of the T rows:
    each T draws its own x).
    """
    T = wl.T if T is None else T
    dt = wl.dtype
    x = _normal(seed, _TAG_X, T, (T, wl.d), wl.x_std, dt)
    wr = _normal(seed, _TAG_WR, 0, (wl.E, wl.d), wl.wr_std, dt)
    bias = None
    if wl.routing == "router_bias":
        z = _rng(seed, _TAG_BIAS).standard_normal(wl.E)
        bias = np.exp(wl.bias_sigma * z).astype(np.float32)
    ids = w = None
    if wl.routing == "zipf":
        ids, w = zipf_routing(T, wl.E, wl.k, wl.zipf_alpha, seed)
    wg = wu = wd = None
    sg = su = sd = None
    if experts and wl.weights == "e4m3":
        nthr = threads or min(16, os.cpu_count() or 1)
        wg = np.empty((wl.E, wl.F, wl.d), dtype=np.uint8)
        wu = np.empty((wl.E, wl.F, wl.d), dtype=np.uint8)
        wd = np.empty((wl.E, wl.d, wl.F), dtype=np.uint8)
        sg = np.empty((wl.E, wl.F), dtype=np.float32)
        su = np.empty((wl.E, wl.F), dtype=np.float32)
        sd = np.empty((wl.E, wl.d), dtype=np.float32)
        dst = {_TAG_WG: (wg, sg), _TAG_WU: (wu, su), _TAG_WD: (wd, sd)}

        def run_q(job):
            tag, e, shape = job
            c, sc = quantize_rows_e4m3(_normal(seed, tag, e, shape, wl.w_std, "f32"))
            dst[tag][0][e] = c
            dst[tag][1][e] = sc

        jobs = [(t, e, (wl.d, wl.F) if t == _TAG_WD else (wl.F, wl.d))
                for e in range(wl.E) for t in (_TAG_WG, _TAG_WU, _TAG_WD)]
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(run_q, jobs))
    elif experts:
        nthr = threads or min(16, os.cpu_count() or 1)
        jobs = []
        for e in range(wl.E):
            jobs.append((_TAG_WG, e, (wl.F, wl.d)))
            jobs.append((_TAG_WU, e, (wl.F, wl.d)))
            jobs.append((_TAG_WD, e, (wl.d, wl.F)))
        np_dt = np.uint16 if dt == "bf16" else np.float32
        wg = np.empty((wl.E, wl.F, wl.d), dtype=np_dt)
        wu = np.empty((wl.E, wl.F, wl.d), dtype=np_dt)
        wd = np.empty((wl.E, wl.d, wl.F), dtype=np_dt)
        dst = {_TAG_WG: wg, _TAG_WU: wu, _TAG_WD: wd}

        def run(job):
            tag, e, shape = job
            dst[tag][e] = _normal(seed, tag, e, shape, wl.w_std, dt)

        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(run, jobs))
    return Inputs(x=x, wr=wr, bias=bias, wg=wg, wu=wu, wd=wd, topk_ids=ids, topk_w=w, sg=sg, su=su, sd=sd)
