"""bench.py's command-line contract that needs no GPU: more than one GPU is refused with
exit status 2 and a message, and a profile summary's traffic figure is reported only
while the kernel source still has the sha256 recorded beside it."""
import hashlib
import os
import subprocess
import sys

from conftest import ROOT


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_recorded_traffic_follows_the_source_sha(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "p.md").write_text(f"x\ntraffic_per_launch: read_bytes=1000 write_bytes=24 "
                               f"source_sha256={sha}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("p.md", "k.hip") == 1024
    src.write_text("kernel source, edited\n")
    assert bench.recorded_traffic("p.md", "k.hip") is None
    assert bench.recorded_traffic("missing.md", "k.hip") is None
