"""CPU tests of bench.py's host-side logic: the one-GPU guard, the traffic
summary's source-hash gate, and the round-trip error report."""
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_rejects_empty_timed_region():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "0"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2 and r.stdout == ""


def test_traffic_summary_hash_gate(tmp_path):
    good = tmp_path / "good.md"
    good.write_text(f"# x\n\nhbm_bytes_per_launch: 356015025\nkernel_sources_sha256: {bench.kernel_source_hash()}\n")
    assert bench.measured_traffic(str(good)) == 356015025.0
    both = tmp_path / "both.md"
    both.write_text("hbm_bytes_per_launch: 356015025\nhbm_bytes_per_launch[k_block128_flat]: 396706335\n"
                    f"kernel_sources_sha256: {bench.kernel_source_hash()}\n")
    assert bench.measured_traffic(str(both), kernel="k_block128_flat") == 396706335.0
    assert bench.measured_traffic(str(both)) == 356015025.0
    assert bench.measured_traffic(str(good), kernel="k_block128_flat") is None
    stale = tmp_path / "stale.md"
    stale.write_text("hbm_bytes_per_launch: 356015025\nkernel_sources_sha256: " + "0" * 64 + "\n")
    assert bench.measured_traffic(str(stale)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.md")) is None
    # the committed summary, whatever its state, parses to a number or None
    v = bench.measured_traffic()
    assert v is None or abs(v / 355991552 - 1) < 0.01
    vb = bench.measured_traffic(kernel="k_block128_flat")
    assert vb is None or abs(vb / (18432 * 7168 * 3 + 144 * 56 * 4) - 1) < 0.01


def test_roundtrip_error_report():
    x = torch.tensor([1.0, 1.0625, -3.0, 1e-9], dtype=torch.float64)
    y = torch.tensor([1.0, 1.0, -3.0, 0.0], dtype=torch.float64)
    r = bench._roundtrip_err(torch, x, y, torch.tensor([1.0]), "e4m3fn")
    # 1e-9 is below the e4m3fn normal range after scaling: excluded
    assert r["elements_checked"] == 3 and r["elements"] == 4
    assert abs(r["max_rel_err"] - 0.0625 / 1.0625) < 1e-12
    assert r["tolerance"] == 2.0 ** -4 and r["within"]
    r2 = bench._roundtrip_err(torch, x, y * 1.5, torch.tensor([1.0]), "e5m2", out_rounding="bf16")
    assert not r2["within"] and r2["tolerance"] == 2.0 ** -3 and "tolerance_with_output_rounding" in r2
