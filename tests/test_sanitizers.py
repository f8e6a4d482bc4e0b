"""Host sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer) of
the planner and of the CPU oracle, each driven over an exhaustive or random
grid of small shapes by a driver of its own (tests/sanitize/).  The planner
is the library's host code; the device kernels cannot be built with a
sanitizer here, and are covered on the GPU by NaN-poisoned guard bands,
unread frames and bitwise repeatability."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _build_and_run(tmp_path, cmd, exe):
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


def test_planner_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_driver")
    out = _build_and_run(tmp_path, ["g++", "-std=c++17"] + SAN + [
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "causal_conv3d_video_amd", "csrc"),
        os.path.join(ROOT, "causal_conv3d_video_amd", "csrc", "cc3d_plan.cpp"),
        os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"), "-o", exe], exe)
    assert "0 failed checks" in out


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = _build_and_run(tmp_path, ["gcc", "-std=c11", "-ffp-contract=off"] + SAN + [
        os.path.join(ROOT, "oracle", "cc3d_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
        "-o", exe], exe)
    assert "0 failed checks" in out
