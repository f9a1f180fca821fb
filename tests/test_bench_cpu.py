"""bench.py host logic, without a GPU: one GPU only, the roofline constants,
and the traffic figure read from a profile summary only while that summary
was taken on the current kernel source."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_peaks():
    assert abs(bench.BF16_PEAK_TFLOPS - 256 * 2.4e9 * 4096 / 1e12) < 0.1
    assert bench.FP8_PEAK_TFLOPS == 2 * bench.BF16_PEAK_TFLOPS
    # fp8 queries: both products on the E4M3 matrix cores
    assert bench.FP8Q_PEAK_TFLOPS == bench.FP8_PEAK_TFLOPS
    assert bench.HBM_PEAK_GBS == 8000.0


def test_traffic_needs_the_current_kernel_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.read_traffic("w") is None
    p = tmp_path / "w_counters.md"
    p.write_text("kernel_sha: %s\nhbm_bytes_per_launch: 1.5e+09\n" % bench.kernel_sha())
    assert bench.read_traffic("w") == 1.5e9
    p.write_text("kernel_sha: 0000000000000000\nhbm_bytes_per_launch: 1.5e+09\n")
    assert bench.read_traffic("w") is None


def test_kernel_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }  // one\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    h = bench.kernel_sha()
    src.write_text("/* a comment */\nint f() {\n  return 1;  // two\n}\n")
    assert bench.kernel_sha() == h
    src.write_text("int f() { return 2; }\n")
    assert bench.kernel_sha() != h


def test_sq_figures_need_the_current_kernel_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.read_counters("w") == {"traffic": None, "mfma_busy_pct": None,
                                        "lds_bank_conflicts_per_access": None}
    (tmp_path / "w_sq_counters.md").write_text(
        "kernel_sha: %s\nmfma_busy_pct: 39.80\nlds_bank_conflicts_per_access: 0.4760\n" % bench.kernel_sha())
    c = bench.read_counters("w")
    assert c["mfma_busy_pct"] == 39.8 and c["lds_bank_conflicts_per_access"] == 0.476
    assert c["traffic"] is None
    (tmp_path / "w_sq_counters.md").write_text("kernel_sha: 0000000000000000\nmfma_busy_pct: 39.80\n")
    assert bench.read_counters("w")["mfma_busy_pct"] is None
