"""Host-side checks of the C ABI (no GPU): exports, sizing and validation.

Every call here either is host arithmetic (moe_query, moe_dispatch_carve,
moe_status_string) or fails validation, which returns before any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from grouped_gemm_gemv_amd import _lib
from grouped_gemm_gemv_amd._lib import MoeDispatch, MoeForwardViews, MoeShape, MoeSizes
from oracle import moe_oracle as O
from workloads import WORKLOADS, get_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libmoe.so not built")


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status_t|const char\*)\s+(moe_\w+)\s*\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    lib = _lib.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_lib.EXPORTED) == names


def test_status_strings():
    lib = _lib.lib()
    for code, name in _lib.STATUS.items():
        assert lib.moe_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.moe_status_string(99)


def _shape(T=64, d=128, E=8, k=2, F=256, C=0, dt=1, bm=0, layout=0):
    return MoeShape(T, d, E, k, F, C, dt, bm, layout)


def _query(s):
    out = MoeSizes()
    st = _lib.lib().moe_query(ctypes.byref(s), ctypes.byref(out))
    return st, out


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_query_sizes_match_definition(name):
    wl = WORKLOADS[name]
    s = _shape(wl.T, wl.d, wl.E, wl.k, wl.F, wl.capacity, 1 if wl.dtype == "bf16" else 0)
    st, q = _query(s)
    assert st == 0
    assert q.rows == O.row_space(wl.T, wl.k, wl.E, wl.capacity)
    assert q.tile_rows in (16, 32, 48, 64, 96, 128, 160, 192, 384)
    for p in (0, 1):
        assert q.max_tiles >= O.max_tiles(wl.T, wl.k, wl.E, wl.capacity, q.tile_rows, p)
    assert q.n_passes == (2 if wl.capacity else 1)
    eb = 2 if wl.dtype == "bf16" else 4
    assert q.forward_ws_bytes >= q.rows * (wl.d + wl.F) * eb + q.dispatch_bytes


def test_tile_rows_override():
    for bm in (16, 32, 48, 64, 96, 128, 160, 192, 384):
        st, q = _query(_shape(T=300, E=16, k=4, C=40, bm=bm))
        assert st == 0 and q.tile_rows == bm
        for p in (0, 1):
            assert q.max_tiles >= O.max_tiles(300, 4, 16, 40, bm, p)


@pytest.mark.parametrize("name,bm", [
    ("mixtral_t512", 160),        # 8 experts x 32 down column tiles fill the units; 128 rows pad less at 160
    ("mixtral_t4096", 384),       # 1024 rows per expert: 384-row tiles worked in pieces
    ("mixtral_decode_t1", 16),    # 2 active experts: split-K short tiles keep the units up
    ("mixtral_decode_t8", 16),    # two rows per active expert: 16-row split-K tiles
    ("mixtral_decode_t128", 160), # 8 experts x 32 tall down tiles fill the units
    ("e64_zipf_a2.0", 192),       # 64 experts x 14 256-column down tiles
    ("capacity_gini0.10", 192),   # 384 rows: 2 tiles of 192, 64 x 2 x 8 of them
    ("tiny_f32", 32),             # one 128-column down tile per expert: mean 16 -> 1.25x -> 32
])
def test_automatic_tile_rows(name, bm):
    wl = get_workload(name)
    st, q = _query(_shape(T=wl.T, d=wl.d, E=wl.E, k=wl.k, F=wl.F, C=wl.capacity))
    assert st == 0 and q.tile_rows == bm


@pytest.mark.parametrize("T,E,k,d,F,bm", [
    (16, 1, 1, 4096, 14336, 32),    # one expert, 16 rows: split-K 32-row tiles
    (64, 1, 1, 4096, 14336, 64),    # past 32 rows: 64-row split-K tiles
    (128, 1, 1, 4096, 14336, 64),   # 32 tall down tiles only: stay short
    (256, 1, 1, 4096, 14336, 64),   # a lone expert stays short up to 512 rows
    (1024, 1, 1, 4096, 14336, 160), # past 512 rows: tall, too few tiles for 192
    (256, 2, 1, 4096, 14336, 160),  # 128 rows, 64 tall down tiles: tall
    (128, 8, 1, 2048, 1408, 48),    # 16 rows, 8 x 32 64-column tiles fill the chip
    (256, 8, 2, 3584, 2560, 160),   # 224 tall down tiles >= 192; 8 x 14 tiles of 192 rows too few
    (1024, 32, 2, 3584, 2560, 192), # 32 x 14 = 448 tiles of 192 rows
    (1536, 8, 1, 3584, 2560, 192),  # 192 rows: one 192-row tile beats 160 + 32
    (2048, 8, 1, 2048, 1408, 128),  # 256 rows: two balanced 128-row tiles
    (1792, 8, 1, 4096, 14336, 128), # 224 rows: two balanced 128-row tiles
    (1600, 8, 1, 4096, 14336, 128), # 200 rows: 128 + 72 rather than 192 + 8
    (1536, 8, 1, 4096, 14336, 192), # 192 rows: one 192-row tile
    (3584, 8, 1, 2048, 1408, 192),  # 448 rows, 8 x 3 x 8 tiles of 192 rows
    (8192, 8, 1, 2048, 1408, 384),  # 1024 rows per expert
    (3584, 8, 1, 4096, 14336, 384), # 448 rows of large experts (d * F >= 2^25): 384-row tiles
    (3072, 8, 1, 4096, 14336, 192), # 384 rows of large experts: two 192-row tiles
    (6144, 8, 1, 4096, 14336, 384), # 768 rows of large experts
    (24576, 32, 1, 3584, 2560, 192),# 768 rows of d * F = 9.2M: 192
    (4096, 1, 1, 4096, 14336, 384), # one expert of 4096 rows: 22 x 16 tiles of 192 rows, then 384
])
def test_tile_rows_rule_shapes(T, E, k, d, F, bm):
    st, q = _query(_shape(T=T, d=d, E=E, k=k, F=F))
    assert st == 0 and q.tile_rows == bm


def test_capacity_rows_example():
    st, q = _query(_shape(T=4096, d=2048, E=64, k=6, F=1408, C=384))
    assert st == 0 and q.rows == 64 * 384 + (4096 * 6 - 384)


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), 1), (dict(E=0), 1), (dict(E=257), 1), (dict(k=0), 1), (dict(k=9, E=8), 1),
    (dict(k=65, E=100), 1), (dict(C=-1), 1), (dict(dt=7), 1), (dict(d=100), 4), (dict(F=96), 4),
    (dict(d=32), 1), (dict(T=2**30, k=8), 1), (dict(bm=40), 4), (dict(bm=256), 4),
])
def test_query_rejects_bad_shapes(kw, code):
    st, _ = _query(_shape(**kw))
    assert st == code


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workspace_size_is_the_forward_workspace(name):
    wl = WORKLOADS[name]
    s = _shape(wl.T, wl.d, wl.E, wl.k, wl.F, wl.capacity, 1 if wl.dtype == "bf16" else 0)
    st, q = _query(s)
    n = ctypes.c_size_t()
    assert st == 0 and _lib.lib().moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0
    assert n.value == q.forward_ws_bytes


def test_workspace_size_errors():
    lib = _lib.lib()
    n = ctypes.c_size_t(7)
    assert lib.moe_workspace_size(None, ctypes.byref(n)) == 2
    assert lib.moe_workspace_size(ctypes.byref(_shape()), None) == 2
    assert lib.moe_workspace_size(ctypes.byref(_shape(T=0)), ctypes.byref(n)) == 1
    assert lib.moe_workspace_size(ctypes.byref(_shape(d=100)), ctypes.byref(n)) == 4
    assert n.value == 7  # untouched on error


@pytest.mark.parametrize("kw", [dict(d=(1 << 19) + 64), dict(F=(1 << 19) + 64),
                                dict(d=(1 << 18) + 64, dt=0), dict(F=(1 << 18) + 64, dt=0)])
def test_rows_past_one_mib_are_unsupported(kw):
    # a weight or activation row above 1 MiB would leave the kernels' 32-bit offsets
    st, _ = _query(_shape(**kw))
    assert st == 4
    ok = {k: (v - 64 if k in ("d", "F") else v) for k, v in kw.items()}
    st, _ = _query(_shape(**ok))
    assert st == 0


@pytest.mark.parametrize("T,d,dt,code", [
    (262144, 4096, 0, 4),    # fp32 x of 4 GiB
    (262144, 4096, 1, 4),    # bf16 x of 2 GiB
    (262016, 4096, 1, 2),    # 0x7ff00000 bytes: accepted (then the null pointers are reported)
])
def test_x_past_the_gather_offset_range_is_unsupported(T, d, dt, code):
    # moe_forward and the gather-folded gate+up address x with 32-bit offsets
    lib = _lib.lib()
    s = _shape(T=T, d=d, E=8, k=2, F=256, dt=dt)
    st, q = _query(s)
    assert st == 0
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_forward(ctypes.byref(s), None, fake, None, None, None, fake, fake, fake, fake, fake,
                           1 << 62, None, None) == code
    assert lib.moe_ffn_gate_up_gather(ctypes.byref(s), None, fake, fake, None, 0, fake, None) == code
    if dt == 1:
        assert lib.moe_forward_fp8(ctypes.byref(s), None, fake, None, None, None, fake, fake, fake, fake, fake,
                                   fake, fake, fake, 1 << 62, None, None) == code
        assert lib.moe_ffn_gate_up_fp8(ctypes.byref(s), None, fake, fake, fake, fake, None, 0, fake, None) == code


def test_noalloc_size_and_argument_checks_return_before_any_hip_call():
    # the scratch size check and the argument checks come before the first
    # HIP call (taking the scratch array's device address)
    lib = _lib.lib()
    fake = ctypes.c_void_p(0x1000)
    big = _shape(T=512, d=4096, E=8, k=2, F=57344)
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 0 and n.value > _lib.NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(ctypes.byref(big), fake, fake, None, None, None, fake, fake, fake, fake,
                                   None, None) == 3
    s = _shape()
    assert lib.moe_forward_noalloc(ctypes.byref(s), None, fake, None, None, None, fake, fake, fake, fake,
                                   None, None) == 2
    assert lib.moe_forward_noalloc(ctypes.byref(s), fake, fake, None, fake, None, fake, fake, fake, fake,
                                   None, None) == 1
    assert lib.moe_forward_noalloc(ctypes.byref(_shape(T=0)), fake, fake, None, None, None, fake, fake, fake,
                                   fake, None, None) == 1


def test_null_pointers_rejected_before_gpu():
    lib = _lib.lib()
    s = _shape()
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_query(None, ctypes.byref(MoeSizes())) == 2
    assert lib.moe_query(ctypes.byref(s), None) == 2
    assert lib.moe_route(ctypes.byref(s), None, fake, None, fake, fake, None) == 2
    assert lib.moe_route(ctypes.byref(s), fake, fake, None, None, fake, None) == 2
    d = MoeDispatch()
    assert lib.moe_permute(ctypes.byref(s), fake, fake, ctypes.byref(d), fake, fake, 1 << 20, None) == 2
    assert lib.moe_permute(ctypes.byref(s), fake, fake, None, fake, fake, 1 << 20, None) == 2
    assert lib.moe_combine(ctypes.byref(s), fake, fake, None, fake, None) == 2
    assert lib.moe_forward(ctypes.byref(s), fake, fake, None, None, None, fake, fake, fake, fake, None, 0,
                           None, None) == 2
    # ids without weights (or the reverse) is an argument error
    assert lib.moe_forward(ctypes.byref(s), fake, fake, None, fake, None, fake, fake, fake, fake, fake,
                           1 << 40, None, None) == 1


def test_carve_and_workspace_checks():
    lib = _lib.lib()
    s = _shape(T=100, E=16, k=4, C=10)
    st, q = _query(s)
    d = MoeDispatch()
    base = 0x100000
    assert lib.moe_dispatch_carve(ctypes.byref(s), base, q.dispatch_bytes - 1, ctypes.byref(d)) == 3
    assert lib.moe_dispatch_carve(ctypes.byref(s), base + 4, q.dispatch_bytes, ctypes.byref(d)) == 1
    assert lib.moe_dispatch_carve(ctypes.byref(s), base, q.dispatch_bytes, ctypes.byref(d)) == 0
    assert d.kpart is None  # 40 rows per expert: the down GEMM does not split K
    ptrs = [getattr(d, n) for n in _lib.DISPATCH_ARRAYS if n != "kpart"]
    assert all(p % 256 == 0 and base <= p < base + q.dispatch_bytes for p in ptrs)
    assert len(set(ptrs)) == len(ptrs)
    # a shape whose down GEMM splits K (bf16, 160-row tiles, 128 rows per expert) carves the two
    # [R][d] fp32 planes of partial sums
    s2 = _shape(T=512, d=512, E=8, k=2, F=256, bm=160)
    st, q2 = _query(s2)
    d2 = MoeDispatch()
    assert st == 0 and lib.moe_dispatch_carve(ctypes.byref(s2), base, q2.dispatch_bytes, ctypes.byref(d2)) == 0
    assert d2.kpart is not None and d2.kpart % 256 == 0
    assert d2.kpart + 2 * q2.rows * 512 * 4 <= base + q2.dispatch_bytes
    assert d.tile_rows == q.tile_rows and d.max_tiles == q.max_tiles
    fake = ctypes.c_void_p(0x1000)
    # permute workspace too small
    assert lib.moe_permute(ctypes.byref(s), fake, fake, ctypes.byref(d), fake, fake, q.permute_ws_bytes - 1,
                           None) == 3
    # forward workspace too small / misaligned
    assert lib.moe_forward(ctypes.byref(s), fake, fake, None, None, None, fake, fake, fake, fake,
                           ctypes.c_void_p(0x100000), q.forward_ws_bytes - 1, None, None) == 3
    assert lib.moe_forward(ctypes.byref(s), fake, fake, None, None, None, fake, fake, fake, fake,
                           ctypes.c_void_p(0x100010), q.forward_ws_bytes, None, None) == 1
    # unsupported tile height, undersized tile map
    d2 = MoeDispatch.from_buffer_copy(d)
    d2.tile_rows = 40
    assert lib.moe_ffn_gate_up(ctypes.byref(s), fake, fake, fake, ctypes.byref(d2), 0, fake, None) == 4
    d2 = MoeDispatch.from_buffer_copy(d)
    d2.max_tiles = 0
    assert lib.moe_ffn_down(ctypes.byref(s), fake, fake, ctypes.byref(d2), 0, fake, None) == 1
    # pass: 0, 1 or MOE_PASS_BOTH (2); anything else is rejected before any launch
    for bad in (-1, 3):
        assert lib.moe_ffn_down(ctypes.byref(s), fake, fake, ctypes.byref(d), bad, fake, None) == 1
        assert lib.moe_ffn_gate_up(ctypes.byref(s), fake, fake, fake, ctypes.byref(d), bad, fake, None) == 1


def test_views_struct_layout():
    # the Python mirror of moe_forward_views_t: a dispatch struct and 5 pointers
    assert ctypes.sizeof(MoeDispatch) == 11 * 8 + 8
    assert ctypes.sizeof(MoeShape) == 9 * 4
    assert ctypes.sizeof(MoeForwardViews) == ctypes.sizeof(MoeDispatch) + 5 * 8
    assert ctypes.sizeof(MoeSizes) == 8 + 4 * 4 + 3 * 8


def test_weight_layout_field_is_validated():
    for layout, code in ((0, 0), (1, 0), (2, 1), (-1, 1)):
        st, _ = _query(_shape(layout=layout))
        assert st == code


@pytest.mark.parametrize("args,code", [
    ((0, 4096, 1, 16, 64), 2),            # null src
    ((4096, 0, 1, 16, 64), 2),            # null dst
    ((4096, 1 << 20, 0, 16, 64), 1),      # no matrices
    ((4096, 1 << 20, 1, 24, 64), 1),      # rows not a multiple of 16
    ((4096, 1 << 20, 1, 16, 96), 1),      # row bytes not a multiple of 64
    ((4096, 4096 + 512, 1, 16, 64), 1),   # dst overlaps src (1024 bytes each)
    ((4104, 1 << 20, 1, 16, 64), 1),      # src not 16-byte aligned
])
def test_pack_blocked16_validation(args, code):
    # validation returns before any HIP call, so fake addresses are safe here
    lib = _lib.lib()
    src, dst, m, rows, rb = args
    assert lib.moe_pack_blocked16(src or None, dst or None, m, rows, rb, None) == code


def test_query_random_and_extreme_shapes():
    """moe_query on random and extreme shapes: either a clean validation error
    or sizes that agree with the definitions (no overflow, no crash)."""
    rng = np.random.default_rng(77)
    shapes = []
    for _ in range(400):
        E = int(rng.integers(1, 257))
        shapes.append(dict(T=int(rng.choice([1, 7, 512, 4096, 1 << 16, 1 << 20, (1 << 31) - 1])),
                           d=int(64 * rng.integers(1, 256)), E=E, k=int(rng.integers(1, min(E, 64) + 1)),
                           F=int(64 * rng.integers(1, 512)),
                           C=int(rng.choice([0, 1, 384, 1 << 20, (1 << 31) - 1])),
                           bm=int(rng.choice([0, 0, 16, 192]))))
    shapes += [dict(T=1, d=64, E=256, k=64, F=64, C=0, bm=0),
               dict(T=(1 << 31) - 1, d=64, E=256, k=64, F=64, C=0, bm=0),
               dict(T=1 << 24, d=64, E=256, k=64, F=64, C=(1 << 31) - 1, bm=0)]
    ok = 0
    for sh in shapes:
        st, q = _query(_shape(T=sh["T"], d=sh["d"], E=sh["E"], k=sh["k"], F=sh["F"], C=sh["C"], bm=sh["bm"]))
        assert st in (0, 1), (sh, st)
        if st != 0:
            # errors only where a count or index would not fit in int32
            Tk = sh["T"] * sh["k"]
            R = O.row_space(sh["T"], sh["k"], sh["E"], sh["C"])
            assert Tk >= 2 ** 31 - 1 or R >= 2 ** 31 - 1 or sh["E"] * sh["C"] >= 2 ** 31 - 1, sh
            continue
        ok += 1
        assert q.rows == O.row_space(sh["T"], sh["k"], sh["E"], sh["C"])
        for p in (0, 1):
            assert q.max_tiles >= O.max_tiles(sh["T"], sh["k"], sh["E"], sh["C"], q.tile_rows, p)
        assert q.forward_ws_bytes >= q.rows * (sh["d"] + sh["F"]) * 2 + q.dispatch_bytes
        assert q.forward_ws_bytes < 2 ** 62
    assert ok > 100


# ---- measurement probes (libmoe_peaks) ----

PEAKS_HEADER = os.path.join(ROOT, "include", "moe_peaks.h")


def test_every_declared_probe_is_exported():
    from grouped_gemm_gemv_amd import peaks as P
    if not os.path.exists(P.LIB_PATH):
        pytest.skip("libmoe_peaks.so not built")
    names = sorted(set(re.findall(r"^\s*int\s+(moe_\w+)\s*\(", open(PEAKS_HEADER).read(), re.M)))
    assert names == sorted(P.EXPORTED)
    lib = P.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_probe_argument_checks_return_before_any_launch():
    from grouped_gemm_gemv_amd import peaks as P
    if not os.path.exists(P.LIB_PATH):
        pytest.skip("libmoe_peaks.so not built")
    lib = P.lib()
    fake = 1 << 20  # never dereferenced: every call below fails validation first
    assert lib.moe_peak_read(None, 1024, fake, 1, 0, None) == 1
    assert lib.moe_peak_read(fake, 1000, fake, 1, 0, None) == 1      # not a multiple of 1 KB
    assert lib.moe_peak_read(fake, 0, fake, 1, 0, None) == 1
    assert lib.moe_peak_read(fake, 1024, fake, 0, 0, None) == 1      # no workgroups
    assert lib.moe_peak_read(fake + 8, 1024, fake, 1, 0, None) == 1  # misaligned
    assert lib.moe_peak_read(fake, 1024, fake, 1, 4, None) == 1      # unknown flags
    assert lib.moe_peak_read(fake, 1024, fake, 1, -1, None) == 1
    assert lib.moe_peak_copy(fake, fake + 512, 1024, 1, 0, None) == 1  # overlapping
    assert lib.moe_peak_copy(fake, None, 1024, 1, 0, None) == 1
    assert lib.moe_peak_copy(fake, fake + 4096, 1024, 1, 7, None) == 1
    assert lib.moe_peak_mfma(1.0, 1.0, 0, fake, 1, None) == 1
    assert lib.moe_peak_mfma(1.0, 1.0, 1, None, 1, None) == 1


# ---- measurement build (libmoe_phases) ----

PHASES_HEADER = os.path.join(ROOT, "include", "moe_phases.h")
PHASES_LIB = os.path.join(ROOT, "grouped_gemm_gemv_amd", "libmoe_phases.so")


def test_phase_build_exports_the_layer_and_its_readers_only_there():
    """libmoe_phases.so exports every moe.h symbol plus the two phase readers
    of moe_phases.h; the product library libmoe.so has no phase reader."""
    import ctypes
    if not os.path.exists(PHASES_LIB):
        pytest.skip("libmoe_phases.so not built")
    readers = sorted(set(re.findall(r"^\s*int\s+(moe_\w+)\s*\(", open(PHASES_HEADER).read(), re.M)))
    assert readers == ["moe_loop_phases_down", "moe_loop_phases_gateup"]
    ph = ctypes.CDLL(PHASES_LIB)
    for n in declared_functions() + readers:
        assert hasattr(ph, n), n
    prod = _lib.lib()
    for n in readers:
        assert not hasattr(prod, n), n
