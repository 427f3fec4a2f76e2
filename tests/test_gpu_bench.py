"""bench.py's output contract on the GPU: one JSON line with the metric, the
throughput, the roofline of the dominant kernel (with the HBM traffic from
the committed counter summary when the GEMM sources match it) and the
measured ceilings.  A short run: few steps, no CPU baseline."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_json_line_with_the_contract_keys():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "10", "--warmup", "10", "--no-cpu-baseline",
           "--kernel-iters", "5", "--settle-ms", "50"]
    print("\n[gpu bench] " + " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "measured_peaks"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 10 and d["warmup"] == 10 and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "mixtral_t512"
    assert d["value"] > 0 and abs(d["value"] - 512 / (d["ms_per_step"] * 1e-3)) / d["value"] < 1e-3
    # ms_per_step is the median of the K single-replay times; the clock-settling
    # replays before the warm-up are reported on their own
    st = d["ms_per_step_stats"]
    assert st["p10"] <= d["ms_per_step"] == st["p50"] <= st["p90"]
    assert d["clock_settle"]["replays"] > 0 and d["clock_settle"]["ms"] >= 50
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert 0 < roof["frac"] < 1
    # traffic: the committed counter summary's figure when it was taken on these
    # GEMM sources (weights read once: at least the algorithmic bytes), else null
    import bench
    committed = bench.measured_traffic("mixtral_t512")
    assert roof["traffic"] == committed
    if committed is not None:
        assert committed >= 0.99 * roof["algorithmic_bytes"]
    peaks = d["measured_peaks"]
    assert 0 < peaks["hbm_read_GBps"] < 8000 * 1.05
    assert 0 < peaks["mfma_bf16_TFLOPs"] < 2500 * 1.05
    assert "cpu_baseline" not in d
