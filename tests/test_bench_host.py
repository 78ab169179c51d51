"""Host-side logic of the benchmark (CPU only): the lookup of the committed
HBM byte counters and the refusal of more than one GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _record(h, first, steps, traffic, mix="routed"):
    return (f"kernel_source_sha256: {h}\nlaunch_mix: {mix}\nfirst_step: {first}\n"
            f"stride: {bench.PROFILE_STRIDE}\nsteps: {steps}\ntraffic_bytes_per_launch: {traffic}\n")


def test_traffic_record_matches_only_its_own_launches(tmp_path, monkeypatch):
    f = tmp_path / "traffic.md"
    f.write_text("# summary\n\n| a | b |\n\n" + _record("abc", 32, 480, 111) + "\n## short run\n\n" +
                 _record("abc", 21, 20, 222) + "\n" + _record("old", 40, 8, 333))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic("abc", "drift", 32, 480) == 111.0
    assert bench.read_traffic("abc", "drift", 21, 20) == 222.0
    assert bench.read_traffic("abc", "drift", 32, 64) is None        # another step count, another mix
    assert bench.read_traffic("abc", "drift", 40, 8) is None         # taken on other kernel sources
    assert bench.read_traffic("abc", "hqekv", 32, 480) is None       # another workload
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.read_traffic("abc", "drift", 32, 480) is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr
    assert not r.stdout.strip()
