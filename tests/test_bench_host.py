"""Host-side pieces of bench.py (no GPU): the one-GPU guard and the lookup of
the committed HBM-traffic summary that fills the roofline's traffic."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _write_profile(root, kernel, sha, workload, hbm):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", "hbm_traffic_%s.txt" % kernel), "w") as f:
        f.write("# comment: not a record\n")
        f.write("kernel: %s\n" % kernel)
        f.write("workload: %s\n" % workload)
        f.write("kernel_source_sha256: %s\n" % sha)
        f.write("hbm_bytes_per_launch: %d\n" % hbm)


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return str(tmp_path)


def test_traffic_is_read_for_the_current_source_and_workload(fake_root):
    _write_profile(fake_root, "k", bench._source_hash(), "mid_192 (C 192->192, ...)", 123456789)
    assert bench.traffic_for("k", "mid_192") == 123456789.0
    assert bench.traffic_for("k") == 123456789.0


def test_traffic_is_null_once_the_source_changed(fake_root):
    _write_profile(fake_root, "k", "0" * 64, "mid_192 (C 192->192, ...)", 123456789)
    assert bench.traffic_for("k", "mid_192") is None


def test_traffic_is_null_for_another_workload_or_kernel(fake_root):
    _write_profile(fake_root, "k", bench._source_hash(), "mid_192 (C 192->192, ...)", 123456789)
    assert bench.traffic_for("k", "mid_192_dt2") is None
    assert bench.traffic_for("other", "mid_192") is None

