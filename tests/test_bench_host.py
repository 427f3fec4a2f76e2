"""Host-side behaviour of bench.py: which launches are the gate+up and down
GEMMs (the traffic and trace summaries depend on it), the source hash that
ties a committed traffic summary to the kernels it was taken on, and the
refusal of more than one GPU."""
import os
import shutil

import bench

GATE = "void moe::gemm::grouped_gemm_kernel<moe::TBF16, 160, 16, 7, 1, true, 4, 4, {wq}, {rs}>(moe::GemmArgs)"
DOWN = "void moe::gemm::grouped_gemm_kernel<moe::TBF16, 192, 32, 8, 1, false, 2, 4, {wq}, {rs}>(moe::GemmArgs)"


def test_gemm_role_reads_the_gated_argument():
    for wq in ("false", "true"):       # bf16 or E4M3 weights: the flag after NTMS
        for rs in (1, 2, 3):           # pieces per tile
            assert bench.gemm_role(GATE.format(wq=wq, rs=rs)) == "gateup"
            assert bench.gemm_role(DOWN.format(wq=wq, rs=rs)) == "down"
    wide = ("void moe::gemm::grouped_gemm_wide_kernel<moe::TBF16, moe::TileShape<144, 32, 7, 1, 2, 9, 1, 0>, "
            "moe::TileShape<160, 16, 7, 1, 4, 4, 1, 0> >(moe::GemmArgs)")
    assert bench.gemm_role(wide) == "gateup"
    f32 = "void moe::gemm::grouped_gemm_kernel<moe::TF32, 16, 16, 1, 4, false, 4, 1, false, 1>(moe::GemmArgs)"
    assert bench.gemm_role(f32) == "down"
    for other in ("moe::(anonymous namespace)::dispatch_small_kernel(moe::SmallDispatchArgs)",
                  "void moe::(anonymous namespace)::route_kernel<moe::TBF16, 1, 16, 8, 4>(moe::TBF16::T const*)",
                  "__amd_rocclr_copyBuffer"):
        assert bench.gemm_role(other) is None


def test_gemm_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = os.path.join(bench.ROOT, "grouped_gemm_gemv_amd", "csrc")
    dst = tmp_path / "grouped_gemm_gemv_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in bench.GEMM_SOURCES:
        shutil.copy(os.path.join(src, f), dst / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.gemm_source_hash()
    tiles = dst / "gemm_tiles.hpp"
    text = tiles.read_text()
    tiles.write_text("// a new comment line\n\n" + text.replace("namespace moe {", "namespace moe {  /* note */", 1))
    assert bench.gemm_source_hash() == h0
    tiles.write_text(text.replace("TileShape<160, 16, 7, 1, 4, 4>", "TileShape<160, 16, 7, 1, 5, 4>", 1))
    assert bench.gemm_source_hash() != h0


def test_more_than_one_gpu_is_refused_with_a_message():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
