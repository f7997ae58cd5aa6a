"""CPU checks of bench.py's contract that need no GPU: the one-GPU refusal and
the counter-derived roofline traffic, which is reported only for the kernel
source the counters were taken on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_traffic_only_for_the_profiled_source(monkeypatch, tmp_path):
    import bench

    prof = tmp_path / "counters.md"
    cur = bench._source_hash(*bench.GEMM_SOURCES)
    prof.write_text(f"- gemm_source_sha256_16: `{cur}`\n- hbm_bytes_per_launch: `1.25e+09`\n")
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(prof))
    assert bench._traffic_from_profile() == 1.25e9
    prof.write_text("- gemm_source_sha256_16: `0000000000000000`\n- hbm_bytes_per_launch: `1.25e+09`\n")
    assert bench._traffic_from_profile() is None
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(tmp_path / "missing.md"))
    assert bench._traffic_from_profile() is None


def test_committed_counter_profile_parses():
    import bench

    v = bench._traffic_from_profile()
    assert v is None or v > 0  # None once the GEMM source changed after the counters were taken
