"""Host-side parts of the benchmark's contract (no GPU needed): more than one
GPU is refused with a message, and the HBM-traffic figure is read from the
committed counter summary only while the kernel sources it was taken from are
unchanged."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_only_for_unchanged_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    row = "| bwd_dkdv | 16 | 4000 | 100 | 1.00..2.00 | 500 | 123456789 |"
    body = "# x\n\nkernel sources sha256: `{}`\n\n| kernel | a | b | c | d | e | f |\n|---|---|---|---|---|---|---|\n" + row + "\n"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the hash is taken over the kernel sources under ROOT: mirror them
    for rel in bench.TRAFFIC_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    sha = bench.kernel_sources_sha256()
    (prof / "hbm_traffic_w.md").write_text(body.format(sha))
    assert bench.measured_traffic("bwd_dkdv", "w") == 123456789
    assert bench.measured_traffic("fwd_step", "w") is None
    (prof / "hbm_traffic_w.md").write_text(body.format("0" * 64))
    assert bench.measured_traffic("bwd_dkdv", "w") is None
    assert bench.measured_traffic("bwd_dkdv", "missing") is None
