"""Host-side behaviour of bench.py that needs no GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    # the library measures one GPU; a request for more exits with a message
    # and status 2 before touching a device
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_keyed_to_the_kernel_sources(tmp_path, monkeypatch):
    # the HBM-bytes figure is reported only while the profile's source hash
    # matches the kernel sources; any other hash gives None
    sys.path.insert(0, ROOT)
    import bench

    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
    good = tmp_path / "good.md"
    good.write_text(f"kernel_source_sha256_16: {h}\nhbm_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(good))
    assert bench.measured_traffic() == 12345.0
    stale = tmp_path / "stale.md"
    stale.write_text("kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(stale))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None
