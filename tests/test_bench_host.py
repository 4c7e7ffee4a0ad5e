"""Host-side checks of bench.py (no GPU): the multi-GPU refusal, the
algorithmic byte and FLOP accounting, and that measured profile figures are
reported only while the profile was taken with the current kernel sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_kernel_bytes_add_up_to_the_path():
    d, th, BH, T = 128, 65536 * 96, 96, 65536
    state = BH * d * d * 4
    intra = bench.kernel_bytes("intra", th, d, BH, T)
    scan = bench.kernel_bytes("scan", th, d, BH, T)
    assert intra + scan - state == th * 1538            # q, k, z, beta | v, gate, y
    assert bench.kernel_bytes("fused", th, d, BH, T) == th * 1538 + 2 * state
    with pytest.raises(KeyError):
        bench.kernel_bytes("decode", th, d, BH, T)
    assert abs(bench.path_flops_per_token_head(128) - 1.51e5) < 0.01e5


def _write_profile(tmp_path, name, sha, lines):
    prof = tmp_path / "profiles"
    prof.mkdir(exist_ok=True)
    (prof / name).write_text("# test profile\n" + f"source_sha256: {sha}\n" + "\n".join(lines) + "\n")


def test_profile_figures_follow_the_source_hash(tmp_path, monkeypatch):
    sha = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: sha)
    assert bench.profiled_traffic("scan", "w") is None and bench.profiled_counters("w") is None   # no file
    _write_profile(tmp_path, "hbm_traffic_w.txt", sha, ["scan_hbm_bytes_per_launch: 1234"])
    assert bench.profiled_traffic("scan", "w") == 1234.0
    assert bench.profiled_traffic("intra", "w") is None
    (tmp_path / "profiles" / "counters_w.txt").write_text(
        f"# source_sha256: {sha}\n[scan] x\nscan_mfma_busy_own_cus: 0.5\nscan_mfma_tflops: 400\n")
    c = bench.profiled_counters("w")
    assert c["scan_mfma_busy_own_cus"] == 0.5 and c["scan_mfma_tflops"] == 400.0
    # taken with other sources: not reported
    _write_profile(tmp_path, "hbm_traffic_w.txt", "0" * 64, ["scan_hbm_bytes_per_launch: 1234"])
    (tmp_path / "profiles" / "counters_w.txt").write_text("# source_sha256: " + "0" * 64 + "\nscan_mfma_tflops: 1\n")
    assert bench.profiled_traffic("scan", "w") is None and bench.profiled_counters("w") is None


def test_path_bytes_and_headline_roofline_definition():
    """The headline roofline credits the dominant launch with the path's
    algorithmic bytes of every token-head it processes: 1,538 B per token-head
    at d = 128 (q, k, z, v, gate in and y out at 2 d bytes, beta 2 bytes)."""
    assert bench.path_bytes_per_token_head(128) == 1538
    assert bench.path_bytes_per_token_head(64) == 6 * 128 + 2


def test_cpu_model_is_a_string():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
