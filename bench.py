"""Benchmark of the MoE layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K=200] [--warmup W=150] [--workload mixtral_t512]

A step is one whole layer (routing, count/scan, permutation, fused gate+up
SwiGLU grouped GEMM, down grouped GEMM, combine) over one batch of seeded
synthetic input, replayed from a hipGraph with every input already resident
in HBM.  Before the W warm-up replays the graph is replayed for --settle-ms
of wall time (reported as `clock_settle`): the GPU raises its clocks over the
first tens of milliseconds of load, and the requested warm-up alone may be
too short for that.  The K timed replays each sit between two HIP events;
`ms_per_step` is the median of those K single-replay times and `value` is T
over it (tokens/s).  Prints one JSON line with that throughput, the
grouped-GEMM MFMA and HBM fractions, the roofline of the dominant kernel
(the fused gate+up GEMM, timed with HIP events on the stream it runs on) and
the CPU oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s @Mixtral shape T=512; grouped-GEMM % MFMA / % HBM peak"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
PEAK_F32_TFLOPS = 157.3      # MI355X fp32 vector/matrix, TFLOP/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvent:
    """A HIP event created with hipEventDisableSystemFence, recorded on a given
    stream.  A default event record also writes back and invalidates the
    caches at system scope, work that lands inside the interval the event
    bounds; HIP documents this flag for events used only as timing marks.
    The HIP runtime is the one torch loaded (same shared object), so torch's
    stream handles are valid here."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes

            import torch  # noqa: F401  (loads the HIP runtime first)
            h = ctypes.CDLL("libamdhip64.so.7")
            vp = ctypes.c_void_p
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            h.hipEventRecord.argtypes = [vp, vp]
            h.hipEventSynchronize.argtypes = [vp]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            h.hipEventDestroy.argtypes = [vp]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        if self.hip().hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        import ctypes
        if self.hip().hipEventRecord(self._ev, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def synchronize(self):
        if self.hip().hipEventSynchronize(self._ev) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        import ctypes
        ms = ctypes.c_float()
        if self.hip().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        if self._hip is not None and getattr(self, "_ev", None):
            self._hip.hipEventDestroy(self._ev)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="wall time of graph replays run before the warm-up so the clocks reach their "
                         "loaded level (reported as clock_settle; 0 disables)")
    ap.add_argument("--workload", default="mixtral_t512")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak probes (streaming read / copy, bf16 MFMA loop)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens of the workload the CPU oracle runs (0: all)")
    ap.add_argument("--kernel-iters", type=int, default=40)
    ap.add_argument("--weight-layout", choices=("blocked16", "rows"), default="blocked16",
                    help="storage order of the expert weights (re-stored once before timing)")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="first copy 256 MiB device to device 3 times (reference for PMC byte counters)")
    ap.add_argument("--summarize", metavar="DB", help="print a text summary of a rocprofv3 result database and exit")
    ap.add_argument("--kernel-table", nargs=3, metavar=("FETCH_DB", "WRITE_DB", "TRACE_DB"),
                    help="per kernel: HBM bytes per dispatch from a FETCH_SIZE and a WRITE_SIZE run (both with "
                         "--pmc-calibration), median duration from a kernel trace, achieved GB/s; then exit")
    ap.add_argument("--cost-curve", action="store_true",
                    help="per-expert cost curve: time the grouped GEMMs with every expert given n rows, "
                         "for n from 1 to 1024, fit t = max(a, c + b*n) and exit")
    ap.add_argument("--cost-experts", type=int, default=8, help="experts per launch for --cost-curve")
    ap.add_argument("--cost-tile-rows", type=int, default=0, help="tile height for --cost-curve (0: automatic)")
    ap.add_argument("--stall-summary", nargs="+", metavar="DB",
                    help="per grouped-GEMM kernel: TA/TD busy and stall cycles and matrix-core busy cycles as a "
                         "fraction of the kernel's cycles, from PMC runs that together hold GRBM_GUI_ACTIVE, "
                         "TA_TA_BUSY_sum, TD_TD_BUSY_sum, TD_TC_STALL_sum, TCP_PENDING_STALL_CYCLES_sum, "
                         "TA_ADDR_STALLED_BY_TC_CYCLES_sum and SQ_VALU_MFMA_BUSY_CYCLES; then exit")
    ap.add_argument("--cold-read", metavar="MB", default=None,
                    help="comma-separated sizes: time one streaming read (libmoe_peaks) of each size right after a "
                         "1 GiB read that evicts it from the caches, best over workgroup counts and cache policies "
                         "(the single-launch ceiling of a GEMM that streams that many weight bytes); then exit")
    ap.add_argument("--loop-phases", action="store_true",
                    help="run the workload's layer on libmoe_phases.so (the bf16 grouped GEMMs built with main-loop "
                         "phase timing) and print, per GEMM, the share of each wavefront's loop cycles spent waiting "
                         "for its loads, at the workgroup barrier, issuing activation loads + MFMAs, and issuing "
                         "weight loads; then exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="print the grouped-GEMM HBM traffic from a FETCH_SIZE and a WRITE_SIZE run "
                         "(both with --pmc-calibration) and exit")
    return ap.parse_args()


GEMM_SOURCES = ["grouped_gemm.hpp", "gemm_tiles.hpp", "device_common.hpp"]
def pmc_summary_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"gateup_{workload}_pmc.txt")


def gemm_source_hash() -> str:
    """Hash of the grouped-GEMM sources, comments and blank lines left out: PMC
    traffic figures are only valid for this code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "grouped_gemm_gemv_amd", "csrc", f), encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        code = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
        h.update("\n".join(line for line in code if line.strip()).encode())
    return h.hexdigest()[:16]


def gemm_role(kernel_name: str):
    """'gateup' or 'down' for a grouped-GEMM kernel name (its sixth template
    argument is the gated flag; the two-width kernel is gate+up only), else None."""
    if "grouped_gemm_wide_kernel<" in kernel_name:
        return "gateup"
    key = "grouped_gemm_kernel<"
    if key not in kernel_name:
        return None
    args = kernel_name.split(key, 1)[1].split(">(", 1)[0].split(", ")
    return "gateup" if args[5].strip() == "true" else "down"


def measured_traffic(workload: str):
    """HBM bytes per launch of the fused gate+up GEMM from the committed PMC summary,
    if it was taken on the current GEMM sources and this workload; else None."""
    path = pmc_summary_path(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha") != gemm_source_hash() or kv.get("workload") != workload:
        return None
    try:
        return float(kv["gateup_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def summarize(db_path: str):
    """Per-kernel summary of a rocprofv3 database: dispatch count and average
    duration (kernel trace), or average counter values (PMC runs)."""
    import collections
    import sqlite3
    db = sqlite3.connect(db_path)
    views = {r[0] for r in db.execute("select name from sqlite_master where type in ('view','table')")}
    if "pmc_events" in views and db.execute("select count(*) from pmc_events").fetchone()[0]:
        rows = db.execute("select name, dispatch_id, counter_name, counter_value from pmc_events").fetchall()
        per = collections.defaultdict(float)  # a counter may come as several rows (one per SE) per dispatch
        for name, did, cn, cv in rows:
            per[(name, cn, did)] += cv
        acc = collections.defaultdict(list)
        for (name, cn, _), v in per.items():
            acc[(name, cn)].append(v)
        print(f"# PMC summary of {os.path.basename(db_path)}: kernel | counter | dispatches | mean value per dispatch")
        for (name, cn), vals in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
            print(f"{name[:110]} | {cn} | {len(vals)} | {sum(vals) / len(vals):.1f}")
    else:
        acc = collections.defaultdict(list)
        for name, dur in db.execute("select name, end - start from kernels"):
            acc[name].append(dur / 1000)
        print(f"# kernel trace summary of {os.path.basename(db_path)}: "
              "kernel | dispatches | avg us | median us | total us")
        for name, d in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
            d = sorted(d)
            med = d[len(d) // 2] if len(d) % 2 else (d[len(d) // 2 - 1] + d[len(d) // 2]) / 2
            print(f"{name[:110]} | {len(d)} | {sum(d) / len(d):.2f} | {med:.2f} | {sum(d):.1f}")


def pmc_summary(fetch_db: str, write_db: str, workload: str):
    """HBM bytes per launch of the two grouped GEMMs from rocprofv3 PMC runs.

    Each run starts with three 256 MiB device-to-device copies (--pmc-calibration);
    their counter readings give the factor from counter KiB to bytes moved."""
    import sqlite3
    calib = 256 * 1024 * 1024 / 1024  # KiB copied
    out = {}
    for db_path, counter in ((fetch_db, "FETCH_SIZE"), (write_db, "WRITE_SIZE")):
        db = sqlite3.connect(db_path)
        rows = db.execute("select name, dispatch_id, counter_value from pmc_events where counter_name = ? "
                          "order by dispatch_id", (counter,)).fetchall()
        copies = [v for n, _, v in rows if "copyBuffer" in n][:3]
        if len(copies) < 3:
            raise SystemExit(f"{db_path}: fewer than 3 calibration copies")
        copy_kib = sum(copies) / 3
        scale = calib / copy_kib
        out[counter] = (copy_kib, scale)
        for key in ("gateup", "down"):
            vals = [v for n, _, v in rows if gemm_role(n) == key]
            out[(key, counter)] = (sum(vals) / max(1, len(vals)), len(vals))
    (cf, sf), (cw, sw) = out["FETCH_SIZE"], out["WRITE_SIZE"]
    print(f"copy_fetch_kib_per_256MiB: {cf:.1f}  (mean of the 3 calibration copies)")
    print(f"copy_write_kib_per_256MiB: {cw:.1f}")
    print(f"fetch_scale: {sf:.4f}")
    print(f"write_scale: {sw:.4f}")
    for key in ("gateup", "down"):
        f, nf = out[(key, "FETCH_SIZE")]
        w, _ = out[(key, "WRITE_SIZE")]
        print(f"{key}_fetch_kib_per_launch: {f:.1f}  (dispatches {nf})")
        print(f"{key}_write_kib_per_launch: {w:.1f}")
    print(f"workload: {workload}")
    print(f"gemm_source_sha: {gemm_source_hash()}")
    for key in ("gateup", "down"):
        f, _ = out[(key, "FETCH_SIZE")]
        w, _ = out[(key, "WRITE_SIZE")]
        print(f"{key}_hbm_bytes_per_launch: {round((f * sf + w * sw) * 1024)}")


def stall_summary(dbs):
    """Busy and stall fractions of the grouped-GEMM kernels from PMC runs.

    Counter values are summed over the instances the profiler reports and
    averaged over dispatches: GRBM_GUI_ACTIVE counts cycles of each of the 8
    XCDs, the TA/TD/TCP counters cycles of each of the 256 compute units, and
    SQ_VALU_MFMA_BUSY_CYCLES cycles of each of the 1024 SIMDs, so each ratio
    below is a per-unit fraction of the kernel's cycles."""
    import collections
    import sqlite3
    vals = collections.defaultdict(list)
    for db_path in dbs:
        db = sqlite3.connect(db_path)
        per = collections.defaultdict(float)
        for name, did, cn, cv in db.execute("select name, dispatch_id, counter_name, counter_value from pmc_events"):
            role = gemm_role(name)
            if role is not None:
                per[(role, cn, did)] += cv
        for (role, cn, _), v in per.items():
            vals[(role, cn)].append(v)
    mean = {k: sum(v) / len(v) for k, v in vals.items()}
    print("# kernel | cycles per XCD | TA busy | TD busy | TD stalled on L1 | L1 stalled on L2 | TA address "
          "stalled on L1 | matrix cores busy (per SIMD) | dispatches")
    for role in ("gateup", "down"):
        if (role, "GRBM_GUI_ACTIVE") not in mean:
            continue
        cyc = mean[(role, "GRBM_GUI_ACTIVE")] / 8

        def f(counter, units=256):
            v = mean.get((role, counter))
            return "n/a" if v is None else f"{v / units / cyc * 100:.0f} %"
        print(f"{role} | {cyc:,.0f} | {f('TA_TA_BUSY_sum')} | {f('TD_TD_BUSY_sum')} | {f('TD_TC_STALL_sum')} | "
              f"{f('TCP_PENDING_STALL_CYCLES_sum')} | {f('TA_ADDR_STALLED_BY_TC_CYCLES_sum')} | "
              f"{f('SQ_VALU_MFMA_BUSY_CYCLES', 1024)} | {len(vals[(role, 'GRBM_GUI_ACTIVE')])}")


def kernel_table(fetch_db: str, write_db: str, trace_db: str):
    """Achieved HBM bandwidth of every kernel: counter bytes per dispatch
    (scaled by the calibration copies, as in pmc_summary) over the median
    duration of the same kernel in a kernel-trace run of the same command."""
    import collections
    import sqlite3

    def counter(db_path, name):
        db = sqlite3.connect(db_path)
        rows = db.execute("select name, dispatch_id, counter_value from pmc_events where counter_name = ? "
                          "order by dispatch_id", (name,)).fetchall()
        copies = [v for n, _, v in rows if "copyBuffer" in n][:3]
        scale = (256 * 1024 * 1024 / 1024) / (sum(copies) / 3)
        acc = collections.defaultdict(list)
        for n, _, v in rows[3:] if len(copies) == 3 else rows:
            acc[n].append(v * scale * 1024)
        return {n: sum(v) / len(v) for n, v in acc.items()}

    fetch = counter(fetch_db, "FETCH_SIZE")
    write = counter(write_db, "WRITE_SIZE")
    db = sqlite3.connect(trace_db)
    dur = collections.defaultdict(list)
    for n, d in db.execute("select name, end - start from kernels"):
        dur[n].append(d)
    print("# kernel | HBM read MB | HBM write MB | median us (trace) | GB/s")
    for n in sorted(fetch, key=lambda k: -(fetch[k] + write.get(k, 0))):
        if n not in dur or "copyBuffer" in n:
            continue
        d = sorted(dur[n])[len(dur[n]) // 2] / 1000  # median us
        rd, wr = fetch[n] / 1e6, write.get(n, 0) / 1e6
        print(f"{n[:100]} | {rd:.2f} | {wr:.2f} | {d:.2f} | {(rd + wr) * 1e3 / d:.0f}")


def fit_knee(n, t):
    """Least-squares fit of t = max(a, c + b*n): flat up to a knee, then linear.
    Returns (a, c, b, n_star) with n_star = (a - c) / b, the knee."""
    n = np.asarray(n, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    best = None
    for i in range(1, len(n) - 1):
        a = float(np.mean(t[:i]))
        b, c = np.polyfit(n[i:], t[i:], 1)
        if b <= 0:
            continue
        sse = float(np.sum((np.maximum(a, c + b * n) - t) ** 2))
        if best is None or sse < best[0]:
            best = (sse, a, float(c), float(b))
    if best is None:
        return None
    _, a, c, b = best
    return a, c, b, (a - c) / b


def cost_curve(args):
    """Time one pass of the two grouped GEMMs when each of `--cost-experts`
    experts holds exactly n rows, for n = 1 ... 1024, at the workload's d and F.

    The cost of an expert's GEMMs is flat in n while its weight stream bounds
    it and grows linearly once the matrix cores do (the TEMPO review, per-expert
    cost model); the fitted knee n* is where the layer leaves the
    weight-streaming regime on this GPU."""
    import torch

    import grouped_gemm_gemv_amd as M
    from workloads import get_workload

    wl = get_workload(args.workload)
    Eg = args.cost_experts
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dt_bytes = 2 if wl.dtype == "bf16" else 4
    peak_f = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    g = torch.Generator(device="cuda").manual_seed(args.seed)
    wg = (torch.randn((Eg, wl.F, wl.d), device="cuda", generator=g) * 0.02).to(dt)
    wu = (torch.randn((Eg, wl.F, wl.d), device="cuda", generator=g) * 0.02).to(dt)
    wd = (torch.randn((Eg, wl.d, wl.F), device="cuda", generator=g) * 0.02).to(dt)
    blocked = args.weight_layout == "blocked16"
    if blocked:
        wg, wu, wd = M.moe_pack_blocked16(wg), M.moe_pack_blocked16(wu), M.moe_pack_blocked16(wd)
    cur = torch.cuda.current_stream()
    rows = [1, 2, 4, 8, 16, 24, 32, 48, 64, 80, 96, 128, 160, 192, 224, 256, 320, 384, 448, 512, 640, 768, 1024]
    res = []
    print(f"# per-expert cost curve: {Eg} experts x n rows, d={wl.d}, F={wl.F}, {wl.dtype}, "
          f"{args.weight_layout} weights; one gate+up and one down launch, HIP events, median of 5 runs of "
          f"{args.kernel_iters} calls")
    print("# n | tile rows | gate+up us | down us | total us | us per expert | TFLOP/s | weight TB/s")
    for n in rows:
        T = n * Eg
        shape = M.Shape(T, wl.d, Eg, 1, wl.F, 0, dt, args.cost_tile_rows,
                        M.LAYOUT_BLOCKED16 if blocked else M.LAYOUT_ROWS)
        q = M.query(shape)
        x = (torch.randn((T, wl.d), device="cuda", generator=g)).to(dt)
        ids = (torch.arange(T, device="cuda", dtype=torch.int32) // n).reshape(T, 1).contiguous()
        w = torch.ones((T, 1), device="cuda", dtype=torch.float32)
        ws = M.workspace(q.forward_ws_bytes)
        out = torch.empty((T, wl.d), dtype=dt, device="cuda")
        v = M.moe_forward(shape, x, None, None, ids, w, wg, wu, wd, out, ws)
        torch.cuda.synchronize()

        def timed(fn):
            for _ in range(3):
                fn()
            meas = []
            for _ in range(5):
                a, b = HipEvent(), HipEvent()
                a.record(cur)
                for _ in range(args.kernel_iters):
                    fn()
                b.record(cur)
                b.synchronize()
                meas.append(a.elapsed_time(b) / args.kernel_iters * 1e3)
            return float(np.median(meas))

        t_gu = timed(lambda: M.moe_ffn_gate_up_gather(shape, x, wg, wu, v.disp, 0, v.h))
        t_dn = timed(lambda: M.moe_ffn_down(shape, v.h, wd, v.disp, 0, v.y_perm))
        tot = t_gu + t_dn
        flops = 2.0 * T * 3 * wl.d * wl.F
        wbytes = 3.0 * Eg * wl.d * wl.F * dt_bytes
        res.append((n, q.tile_rows, t_gu, t_dn, tot))
        print(f"{n} | {q.tile_rows} | {t_gu:.1f} | {t_dn:.1f} | {tot:.1f} | {tot / Eg:.2f} | "
              f"{flops / tot / 1e6:.1f} | {wbytes / tot / 1e6:.2f}", flush=True)
        del x, ids, w, ws, out, v
    n_arr = [r[0] for r in res]
    fit = fit_knee(n_arr, [r[4] for r in res])
    hbm_eff = 3.0 * Eg * wl.d * wl.F * dt_bytes / (res[0][4] * 1e-6) / (PEAK_HBM_GBS * 1e9)
    mfma_eff = 2.0 * res[-1][0] * Eg * 3 * wl.d * wl.F / (res[-1][4] * 1e-6) / (peak_f * 1e12)
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9) * (dt_bytes / 2)
    summary = {"experts": Eg, "d": wl.d, "F": wl.F, "dtype": wl.dtype,
               "hbm_eff_at_n1": round(hbm_eff, 4), "mfma_eff_at_nmax": round(mfma_eff, 4),
               "ridge_rows_datasheet": round(ridge, 1),
               "ridge_rows_measured_eff": round(ridge * mfma_eff / hbm_eff, 1)}
    if fit is not None:
        a, c, b, nstar = fit
        summary.update({"fit_flat_us": round(a, 2), "fit_intercept_us": round(c, 2),
                        "fit_us_per_row": round(b, 4), "n_star": round(nstar, 1)})
    print("# fit of total us = max(a, c + b*n) and ridge estimates:")
    print(json.dumps(summary), flush=True)


def gemm_work(wl, counts, dt_bytes, spill_counts=None):
    """Algorithmic FLOPs and HBM bytes of the two grouped GEMMs (all passes):
    every active expert's weights once, plus once more for every expert with
    rows in the overflow pass (capacity mode; that re-streaming is the method's
    own cost), E4M3 codes at 1 byte per element plus one fp32 scale per output
    channel; activation rows read once per slot, outputs written once."""
    Tk = wl.T * wl.k
    active = int((counts > 0).sum())
    streams = active + (int((spill_counts > 0).sum()) if spill_counts is not None else 0)
    gu_flops = 4.0 * Tk * wl.d * wl.F
    dn_flops = 2.0 * Tk * wl.d * wl.F
    if wl.weights == "e4m3":
        wgu = streams * (2.0 * wl.F * wl.d + 2.0 * wl.F * 4)
        wdn = streams * (1.0 * wl.F * wl.d + wl.d * 4)
    else:
        wgu = streams * 2.0 * wl.F * wl.d * dt_bytes
        wdn = streams * 1.0 * wl.F * wl.d * dt_bytes
    gu_bytes = wgu + (Tk * wl.d + Tk * wl.F) * dt_bytes
    dn_bytes = wdn + (Tk * wl.F + Tk * wl.d) * dt_bytes
    return gu_flops, gu_bytes, dn_flops, dn_bytes, active


def measured_peaks():
    """Achievable ceilings on this device, from the probes of libmoe_peaks
    (include/moe_peaks.h): a streaming read of 4 GiB, a copy of 1 GiB and a
    loop of independent bf16 MFMAs, each the best over several workgroup
    counts (and, for read and copy, chunk orders and cache policies), each
    timed with HIP events on the stream it runs on.  The copy and the MFMA
    results are checked exactly."""
    import torch

    from grouped_gemm_gemv_amd import peaks as P
    cur = torch.cuda.current_stream()

    def seconds(fn, n=10):
        fn()
        fn()
        a, b = HipEvent(), HipEvent()
        cur.synchronize()
        a.record(cur)
        for _ in range(n):
            fn()
        b.record(cur)
        b.synchronize()
        return a.elapsed_time(b) / n * 1e-3

    nb = 4 << 30
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    sweep = [(blk, fl) for fl in range(4) for blk in (256, 512, 1024, 2048)]
    read = max(nb / seconds(lambda: P.moe_peak_read(buf, sink, blk, fl)) / 1e9 for blk, fl in sweep)
    del buf
    half = 1 << 30
    src = torch.empty(half, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.zeros_like(src)
    copy = max(2 * half / seconds(lambda: P.moe_peak_copy(src, dst, blk, fl)) / 1e9 for blk, fl in sweep)
    assert torch.equal(src, dst), "copy probe: wrong result"
    del src, dst
    iters = 8192
    fs = torch.empty(4 * 2048, dtype=torch.float32, device="cuda")
    mfma = 0.0
    for blk in (512, 1024, 2048):
        fl = float(blk) * P.MFMA_WAVES * P.MFMA_CHAINS * iters * P.MFMA_FLOPS
        t = seconds(lambda: P.moe_peak_mfma(1.0, 1.0, iters, fs, blk))
        assert bool((fs[:4 * blk] == 256.0 * iters).all()), "mfma probe: wrong result"
        mfma = max(mfma, fl / t / 1e12)
    torch.cuda.synchronize()
    return {"hbm_read_GBps": round(read, 1), "hbm_copy_GBps": round(copy, 1), "mfma_bf16_TFLOPs": round(mfma, 1),
            "probes": "libmoe_peaks: streaming read of 4 GiB and copy of 1 GiB (read + written bytes), best "
                      "over 256-2048 workgroups, strided or per-wavefront chunk order, default or non-temporal "
                      "cache policy; 8 independent bf16 16x16x32 MFMA chains per wavefront, best over "
                      "512-2048 workgroups"}


def host_cpu() -> dict:
    """The host CPU the oracle runs on: model name, os.cpu_count(), the CPUs
    this process may run on, and the CPU quota of its control group (None if
    it sets none)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()[:2]
            if q != "max":
                quota = float(q) / float(period)
    except (OSError, ValueError):
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"model": model, "os_cpu_count": os.cpu_count(), "affinity": affinity, "cgroup_cpu_quota": quota}


def oracle_threads(cpu: dict) -> int:
    """BLAS threads for the oracle: os.cpu_count(), unless the process may use
    fewer CPUs (affinity mask or control-group quota), then that many."""
    n = cpu["os_cpu_count"] or 1
    n = min(n, cpu["affinity"])
    if cpu["cgroup_cpu_quota"]:
        n = min(n, max(1, int(cpu["cgroup_cpu_quota"])))
    return n


def cpu_baseline(wl, inp, sample_tokens):
    """The oracle as it stands on the workload (or its first `sample_tokens`
    tokens), repeated until about 12 s of CPU time have been spent."""
    from threadpoolctl import threadpool_limits

    from oracle import moe_oracle as O
    n = wl.T if sample_tokens <= 0 else min(wl.T, sample_tokens)
    wg, wu, wd = inp.wg, inp.wu, inp.wd
    if wl.weights == "e4m3":
        wg, wu, wd = O.Fp8Weights(inp.wg, inp.sg), O.Fp8Weights(inp.wu, inp.su), O.Fp8Weights(inp.wd, inp.sd)
    cpu = host_cpu()
    cores = oracle_threads(cpu)
    reps, total = 0, 0.0
    with threadpool_limits(limits=cores):
        while reps == 0 or (total < 12.0 and reps < 10):
            t0 = time.perf_counter()
            if inp.topk_ids is None:
                O.forward(inp.x[:n], inp.wr, wg, wu, wd, wl.k, wl.dtype, bias=inp.bias,
                          capacity=wl.capacity)
            else:
                O.forward(inp.x[:n], inp.wr, wg, wu, wd, wl.k, wl.dtype,
                          topk_ids=inp.topk_ids[:n], topk_w=inp.topk_w[:n], capacity=wl.capacity)
            total += time.perf_counter() - t0
            reps += 1
    return {"value": n * reps / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu["model"], "os_cpu_count": cpu["os_cpu_count"], "cpu_affinity": cpu["affinity"],
            "cgroup_cpu_quota": cpu["cgroup_cpu_quota"],
            "sample": f"{n} of {wl.T} tokens of {wl.name} (seed 0), whole layer in float64, "
                      f"{reps} run(s), {total:.1f} s, {cores} BLAS threads"}


def loop_phases(args):
    """Main-loop phase shares of the bf16 grouped GEMMs (see --loop-phases):
    the layer runs on libmoe_phases.so, whose GEMM kernels are the product's
    with shader-clock reads around each phase of every main-loop iteration."""
    import ctypes

    import torch

    from grouped_gemm_gemv_amd import _lib
    _lib.LIB_PATH = os.path.join(ROOT, "grouped_gemm_gemv_amd", "libmoe_phases.so")
    import grouped_gemm_gemv_amd as M
    from workloads import get_workload, make_inputs

    wl = get_workload(args.workload)
    if wl.dtype != "bf16":
        print("--loop-phases times the bf16 GEMM kernels", file=sys.stderr)
        sys.exit(2)
    inp = make_inputs(wl, args.seed)

    def dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, wr, bias = dev(inp.x), dev(inp.wr), dev(inp.bias)
    wg, wu, wd = dev(inp.wg), dev(inp.wu), dev(inp.wd)
    if args.weight_layout == "blocked16":
        wg, wu, wd = M.moe_pack_blocked16(wg), M.moe_pack_blocked16(wu), M.moe_pack_blocked16(wd)
    ids, w = dev(inp.topk_ids), dev(inp.topk_w)
    shape = M.Shape(wl.T, wl.d, wl.E, wl.k, wl.F, wl.capacity, torch.bfloat16, 0,
                    M.LAYOUT_BLOCKED16 if args.weight_layout == "blocked16" else M.LAYOUT_ROWS)
    q = M.query(shape)
    ws = M.workspace(q.forward_ws_bytes)
    out = torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device="cuda")
    step = lambda: M.moe_forward(shape, x, wr, bias, ids, w, wg, wu, wd, out, ws)  # noqa: E731
    v = step()
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    lib = _lib.lib()
    slots = 1 << 17
    buf = np.zeros(slots * 8, dtype=np.uint64)
    ps = M.PASS_BOTH if q.n_passes == 2 else 0
    print(f"# main-loop phases of the bf16 grouped GEMMs, workload {wl.name} (T={wl.T}, d={wl.d}, E={wl.E}, "
          f"k={wl.k}, F={wl.F}), tile rows {q.tile_rows}, {args.weight_layout} weights; one launch each after "
          f"{max(args.warmup, 1)} layers; shares of the summed loop cycles of every wavefront")
    print("# gemm | wavefronts | iterations per wavefront | loop cycles per wavefront | wait for loads | barrier | "
          "activation loads + MFMAs | weight loads | other | shader clock GHz over the loops")
    for name, fn, reader in (
            ("gate+up", lambda: M.moe_ffn_gate_up_gather(shape, x, wg, wu, v.disp, ps, v.h), lib.moe_loop_phases_gateup),
            ("down", lambda: M.moe_ffn_down(shape, v.h, wd, v.disp, ps, v.y_perm), lib.moe_loop_phases_down)):
        reader.argtypes = [ctypes.c_void_p, ctypes.c_int]
        reader.restype = ctypes.c_int
        step()
        torch.cuda.synchronize()
        if reader(None, 1) != 0:
            raise RuntimeError("clearing the phase buffer failed")
        fn()
        torch.cuda.synchronize()
        if reader(buf.ctypes.data_as(ctypes.c_void_p), 0) != 0:
            raise RuntimeError("reading the phase buffer failed")
        r = buf.reshape(-1, 8)
        r = r[r[:, 7] == 1].astype(np.float64)
        if len(r) == 0:
            print(f"{name} | 0 | - | - | (no WK = 1 main loop in this launch)")
            continue
        tot = r[:, 4].sum()
        sh = r[:, :4].sum(axis=0) / tot
        ghz = tot / max(r[:, 6].sum(), 1.0) * 0.1  # cycles per 100 MHz tick / 10
        print(f"{name} | {len(r)} | {r[:, 5].mean():.1f} | {r[:, 4].mean():.0f} | {sh[0]:.3f} | {sh[1]:.3f} | "
              f"{sh[2]:.3f} | {sh[3]:.3f} | {1 - sh.sum():.3f} | {ghz:.2f}", flush=True)


def cold_read(sizes_mb):
    """Single-launch streaming-read ceilings at the given sizes: each timed
    launch reads a buffer that a 1 GiB read just evicted from L2 and the
    last-level cache, as a layer's GEMM finds its weights; median of 10
    launches per (workgroups, cache policy), best of those."""
    import torch

    from grouped_gemm_gemv_amd import peaks as P
    cur = torch.cuda.current_stream()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    print("# cold single-launch streaming read (libmoe_peaks moe_peak_read), each launch after a 1 GiB read; "
          "median of 10 per setting, best setting")
    print("# bytes | us | GB/s | workgroups | flags (1 non-temporal, 2 per-wavefront regions)")
    for mb in sizes_mb:
        nb = (int(mb * 1e6) // 65536) * 65536
        buf = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(2)
        best = None
        for blk in (512, 1024, 2048, 4096):
            for fl in range(4):
                ts = []
                for _ in range(10):
                    P.moe_peak_read(flush, sink, 1024, 0)
                    a, b = HipEvent(), HipEvent()
                    a.record(cur)
                    P.moe_peak_read(buf, sink, blk, fl)
                    b.record(cur)
                    b.synchronize()
                    ts.append(a.elapsed_time(b) * 1e3)
                t = float(np.median(ts))
                if best is None or t < best[0]:
                    best = (t, blk, fl)
        print(f"{nb} | {best[0]:.1f} | {nb / best[0] / 1e3:.0f} | {best[1]} | {best[2]}", flush=True)
        del buf


def main():
    args = parse()
    if args.cold_read:
        cold_read([float(v) for v in args.cold_read.split(",")])
        return
    if args.loop_phases:
        loop_phases(args)
        return
    if args.summarize:
        summarize(args.summarize)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload)
        return
    if args.kernel_table:
        kernel_table(*args.kernel_table)
        return
    if args.stall_summary:
        stall_summary(args.stall_summary)
        return
    if args.cost_curve:
        if args.gpus != 1:
            print("the cost curve runs on one GPU", file=sys.stderr)
            sys.exit(2)
        cost_curve(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested); "
              "the layer runs on one GPU; it is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)
    import torch

    import grouped_gemm_gemv_amd as M
    from workloads import get_workload, make_inputs

    if args.pmc_calibration:
        n = 256 * 1024 * 1024 // 4
        ca = torch.ones(n, device="cuda")
        cb = torch.empty_like(ca)
        for _ in range(3):
            cb.copy_(ca)
        torch.cuda.synchronize()
        del ca, cb
    wl = get_workload(args.workload)
    log(f"workload {wl.name}: generating inputs (seed {args.seed})")
    t0 = time.time()
    inp = make_inputs(wl, args.seed)
    log(f"inputs ready in {time.time() - t0:.1f} s")
    torch.cuda.set_device(0)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dt_bytes = 2 if wl.dtype == "bf16" else 4

    def dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, wr, bias = dev(inp.x), dev(inp.wr), dev(inp.bias)
    wg, wu, wd = dev(inp.wg), dev(inp.wu), dev(inp.wd)
    fp8 = wl.weights == "e4m3"
    sg, su, sd = dev(inp.sg), dev(inp.su), dev(inp.sd)
    ids_in, w_in = dev(inp.topk_ids), dev(inp.topk_w)
    blocked = args.weight_layout == "blocked16"
    if blocked:
        # weights are re-stored once, as a loader would; not part of a step
        wg, wu, wd = M.moe_pack_blocked16(wg), M.moe_pack_blocked16(wu), M.moe_pack_blocked16(wd)
        torch.cuda.synchronize()
    shape = M.Shape(wl.T, wl.d, wl.E, wl.k, wl.F, wl.capacity, dt, 0,
                    M.LAYOUT_BLOCKED16 if blocked else M.LAYOUT_ROWS)
    q = M.query(shape)
    ws = M.workspace(q.forward_ws_bytes)
    out = torch.empty((wl.T, wl.d), dtype=dt, device="cuda")

    def step():
        if fp8:
            return M.moe_forward_fp8(shape, x, wr, bias, ids_in, w_in, wg, wu, wd, sg, su, sd, out, ws)
        return M.moe_forward(shape, x, wr, bias, ids_in, w_in, wg, wu, wd, out, ws)

    views = step()
    torch.cuda.synchronize()
    counts = views.disp.arrays()["counts"].cpu().numpy()
    spill_counts = views.disp.arrays()["spill_counts"].cpu().numpy() if wl.capacity else None
    log(f"eager forward ok; tile rows {q.tile_rows}, counts {counts.tolist()[:16]}")

    # graph capture of the whole layer (no host sync, no allocation inside)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    # clock settling: replays for --settle-ms of wall time, before the warm-up
    settle_n, t_settle = 0, time.perf_counter()
    while args.settle_ms > 0 and (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(20):
            g.replay()
        torch.cuda.synchronize()
        settle_n += 20
    settle = {"replays": settle_n, "ms": round((time.perf_counter() - t_settle) * 1e3, 1)}
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    # the timed region: exactly K replays, each between two HIP events
    cur = torch.cuda.current_stream()
    evs = [(HipEvent(), HipEvent()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for a, b in evs:
        a.record(cur)
        g.replay()
        b.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    per = np.array([a.elapsed_time(b) for a, b in evs])
    ms = float(np.median(per))
    spread = {"p10": round(float(np.percentile(per, 10)), 4), "p50": round(ms, 4),
              "p90": round(float(np.percentile(per, 90)), 4), "mean": round(float(per.mean()), 4),
              "wall_mean": round(wall * 1e3 / args.steps, 4)}
    log(f"clock settling: {settle['replays']} replays in {settle['ms']} ms; {args.steps} timed graph replays: "
        f"median {ms * 1e3:.1f} us, mean {per.mean() * 1e3:.1f} us, wall {wall * 1e6 / args.steps:.1f} us per step")

    # per-call times (HIP events on the stream the kernels run on)
    cur = torch.cuda.current_stream()
    disp = views.disp
    h, y = views.h, views.y_perm
    xp = torch.empty((q.rows, wl.d), dtype=dt, device="cuda")
    pws = M.workspace(q.permute_ws_bytes)
    ids = views.topk_ids
    wts = views.topk_w

    def timed(fn, iters):
        """Mean duration of one call of fn in microseconds, each call timed on
        its own (two HIP events on the stream it runs on) right after a graph
        replay of the whole layer, so it runs in the clock and cache state of
        the timed layer."""
        for _ in range(3):
            g.replay()
            fn()
        evs = [(HipEvent(), HipEvent()) for _ in range(iters)]
        cur.synchronize()
        for a, b in evs:
            g.replay()
            a.record(cur)
            fn()
            b.record(cur)
        cur.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3  # us

    it = args.kernel_iters
    # the GEMM launches exactly as moe_forward runs them: the gather folded
    # into the gate+up loads, and in capacity mode both passes in one launch
    ps = M.PASS_BOTH if q.n_passes == 2 else 0
    if fp8:
        t_gu = timed(lambda: M.moe_ffn_gate_up_fp8(shape, x, wg, wu, sg, su, disp, ps, h), it)
        t_dn = timed(lambda: M.moe_ffn_down_fp8(shape, h, wd, sd, disp, ps, y), it)
    else:
        t_gu = timed(lambda: M.moe_ffn_gate_up_gather(shape, x, wg, wu, disp, ps, h), it)
        t_dn = timed(lambda: M.moe_ffn_down(shape, h, wd, disp, ps, y), it)
    t_perm = timed(lambda: M.moe_permute(shape, x, ids, disp, xp, pws), it)
    t_comb = timed(lambda: M.moe_combine(shape, y, wts, disp, out), it)
    t_route = 0.0
    if ids_in is None:
        rid = torch.empty_like(ids)
        rw = torch.empty_like(wts)
        t_route = timed(lambda: M.moe_route(shape, x, wr, bias, rid, rw), it)
    log(f"per call (us): route {t_route:.1f} permute {t_perm:.1f} gate_up {t_gu:.1f} down {t_dn:.1f} "
        f"combine {t_comb:.1f}")
    peaks = None if args.no_peaks else measured_peaks()

    gu_flops, gu_bytes, dn_flops, dn_bytes, active = gemm_work(wl, counts, dt_bytes, spill_counts)
    peak_f = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    if gu_flops / gu_bytes < ridge:
        ach = gu_bytes / (t_gu * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic(wl.name)}
    else:
        ach = gu_flops / (t_gu * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak_f, "unit": "TFLOP/s",
                "frac": round(ach / peak_f, 4), "traffic": measured_traffic(wl.name)}
    roof["kernel"] = "grouped_gemm_kernel (fused gate+up SwiGLU%s)" % (", E4M3 weights" if fp8 else "")
    roof["gemm_source_sha"] = gemm_source_hash()
    roof["us_per_launch"] = round(t_gu, 2)  # one launch (both passes in capacity mode)
    roof["algorithmic_bytes"] = gu_bytes
    roof["algorithmic_flops"] = gu_flops
    if peaks is not None:
        # the same kernel against the ceiling measured on this device
        ach_peak = peaks["hbm_read_GBps"] if roof["bound"] == "hbm" else (
            peaks["mfma_bf16_TFLOPs"] if wl.dtype == "bf16" else None)
        if ach_peak:
            roof["achievable_peak"] = ach_peak
            roof["frac_of_achievable"] = round(ach / ach_peak, 4)
    t_gemm = (t_gu + t_dn) * 1e-6
    gemm_flops = gu_flops + dn_flops
    gemm_bytes = gu_bytes + dn_bytes
    gg = {
        "us": round(t_gu + t_dn, 1),
        "tflops": round(gemm_flops / t_gemm / 1e12, 1),
        "mfma_frac": round(gemm_flops / t_gemm / 1e12 / peak_f, 4),
        "gbps": round(gemm_bytes / t_gemm / 1e9, 1),
        "hbm_frac": round(gemm_bytes / t_gemm / 1e9 / PEAK_HBM_GBS, 4),
        "roofline_frac": round(max(gemm_flops / (peak_f * 1e12), gemm_bytes / (PEAK_HBM_GBS * 1e9)) / t_gemm, 4),
        "active_experts": active,
    }
    if peaks is not None:
        gg["hbm_frac_of_achievable"] = round(gemm_bytes / t_gemm / 1e9 / peaks["hbm_read_GBps"], 4)
        if wl.dtype == "bf16":
            gg["mfma_frac_of_achievable"] = round(gemm_flops / t_gemm / 1e12 / peaks["mfma_bf16_TFLOPs"], 4)
    tokens_per_s = wl.T / (ms * 1e-3)
    res = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_stats": spread,
        "clock_settle": settle,
        "timer": "HIP events (hipEventDisableSystemFence) recorded on the launch stream",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded normal draws, random-init weights)",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "E": wl.E, "k": wl.k, "F": wl.F,
                   "capacity": wl.capacity, "seed": args.seed, "graph": True,
                   "expert_weights": "e4m3 codes + fp32 channel scales" if fp8 else wl.dtype,
                   "weight_layout": args.weight_layout},
        "grouped_gemm": gg,
        "per_call_us": {"route": round(t_route, 1), "permute": round(t_perm, 1), "gate_up": round(t_gu, 1),
                        "down": round(t_dn, 1), "combine": round(t_comb, 1)},
        "roofline": roof,
    }
    if peaks is not None:
        res["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_sample_tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
