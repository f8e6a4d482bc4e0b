"""Host-side pieces of bench.py (no GPU): the one-GPU guard, the clock record
parsed from rocm-smi, and the lookup of
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


K = "bf16_s3_n64_p24x32_g32"


def test_traffic_is_read_for_the_current_source_and_workload(fake_root):
    _write_profile(fake_root, K, bench._source_hash(K), "mid_192 (C 192->192, ...)", 123456789)
    assert bench.traffic_for(K, "mid_192") == 123456789.0
    assert bench.traffic_for(K) == 123456789.0


def test_source_hash_follows_the_kernels_own_files():
    # the group-staged kernel's hash covers its translation unit and the
    # shared headers, not the other kernel families
    files = bench._kernel_sources(K)
    assert "cc3d_k_g32.hip" in files and "cc3d_device.h" in files and "cc3d_k_mfma.hip" not in files
    assert "cc3d_few.inc" in bench._kernel_sources("bf16_s3_few_p15x128")
    assert "cc3d_k_s1.hip" in bench._kernel_sources("bf16_s1_n192_p256_rd")
    assert bench._source_hash(K) != bench._source_hash("bf16_s3_few_p15x128")
    for f in bench._kernel_sources(None):
        assert os.path.exists(os.path.join(bench.CSRC, f))


def test_traffic_is_null_once_the_source_changed(fake_root):
    _write_profile(fake_root, K, "0" * 64, "mid_192 (C 192->192, ...)", 123456789)
    assert bench.traffic_for(K, "mid_192") is None


def test_traffic_is_null_for_another_workload_or_kernel(fake_root):
    _write_profile(fake_root, K, bench._source_hash(K), "mid_192 (C 192->192, ...)", 123456789)
    assert bench.traffic_for(K, "mid_192_dt2") is None
    assert bench.traffic_for("other", "mid_192") is None



def _fake_smi(tmp_path, body, rc=0):
    exe = tmp_path / "rocm-smi"
    exe.write_text("#!/bin/sh\ncat <<'TXT'\n%sTXT\nexit %d\n" % (body, rc))
    exe.chmod(0o755)
    return str(exe)


def _no_gpu(monkeypatch):
    import torch
    monkeypatch.setattr(bench, "run_step", lambda work, stream, packed=True: None)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)


def test_clock_levels_parsed_from_rocm_smi(tmp_path, monkeypatch):
    """The clock record reads each clock's current level from rocm-smi's
    --showclocks text; a failing or missing rocm-smi gives None."""
    import shutil
    _no_gpu(monkeypatch)
    text = ("======== ROCm System Management Interface ========\n"
            "GPU[0]\t\t: fclk clock level: 0: (1200Mhz)\n"
            "GPU[0]\t\t: mclk clock level: 3: (1900Mhz)\n"
            "GPU[0]\t\t: sclk clock level: 1: (2100Mhz)\n")
    exe = _fake_smi(tmp_path, text)
    monkeypatch.setattr(shutil, "which", lambda name: exe)
    assert bench.gpu_clocks_under_load(None, None) == {"fclk": 1200, "mclk": 1900, "sclk": 2100}
    exe = _fake_smi(tmp_path, text, rc=1)
    assert bench.gpu_clocks_under_load(None, None) is None
    monkeypatch.setattr(shutil, "which", lambda name: None)
    monkeypatch.setattr(bench.os.path, "exists", lambda p: False)
    assert bench.gpu_clocks_under_load(None, None) is None
