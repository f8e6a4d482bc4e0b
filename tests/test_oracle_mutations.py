"""Mutation check of the oracle's pins (CPU only): plausible mistakes are
planted, one at a time, in copies of the oracle's C source (oracle/
cc3d_oracle.c), each copy is built and swapped in for the oracle, and the
pins of test_oracle_pins -- checks against torch conv3d in float64, the
impulse closed form, the bias-once closed form and streaming equivalence --
are run against it.  Every mutant must fail at least one of them; the
unmutated source must pass them all.  The mistakes are the ones a reading of
the lowering section could plausibly produce: a flipped temporal or spatial
kernel, the wrong sign of the effective left pad p_l, the bias added per tap,
an off-by-one input frame, the temporal dilation or the spatial stride
ignored, the padding applied the wrong way."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "cc3d_oracle.c")

MUTATIONS = {
    "temporal taps flipped": ("const int64_t t = o * st + k * dt - pl;",
                              "const int64_t t = o * st + (kt - 1 - k) * dt - pl;"),
    "spatial kernel flipped": ("const int64_t u = i * sh - ph + a * dh;",
                               "const int64_t u = i * sh - ph + (kh - 1 - a) * dh;"),
    "p_l sign": ("const int64_t pl = pbase - tc;\n  const int64_t total", "const int64_t pl = tc - pbase;\n  const int64_t total"),
    "bias per tap": ("if (t < 0 || t >= zt) continue;",
                     "if (t < 0 || t >= zt) continue;\n        for (int64_t c2 = 0; c2 < cout; ++c2)"
                     " acc[c2] += bias ? to_double(bias, c2, in_dtype) : 0.0;"),
    "input frame off by one": ("base = (((nn * tx + (t - tc)) * h + u) * wd + v) * cin;",
                               "base = (((nn * tx + (t > tc ? t - tc - 1 : t - tc)) * h + u) * wd + v) * cin;"),
    "temporal dilation ignored": ("const int64_t t = o * st + k * dt - pl;", "const int64_t t = o * st + k - pl;"),
    "spatial stride ignored": ("const int64_t v = j * sw - pw + c * dw;", "const int64_t v = j - pw + c * dw;"),
    "padding sign": ("const int64_t u = i * sh - ph + a * dh;", "const int64_t u = i * sh + ph + a * dh;"),
}


def _build(src_text, path):
    with open(path + ".c", "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o", path, path + ".c"],
                   check=True, capture_output=True, timeout=120)
    lib = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    lib.cc3d_oracle_conv3d.restype = ctypes.c_int
    lib.cc3d_oracle_conv3d.argtypes = ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p] + [i64] * 19 + [ctypes.c_void_p, i64, ctypes.c_void_p,
                                                                        ctypes.c_int])
    lib.cc3d_oracle_out_shape.restype = ctypes.c_int
    lib.cc3d_oracle_out_shape.argtypes = [i64] * 16 + [ctypes.POINTER(i64)] * 3
    return lib


def _pins():
    """Run the pin battery; returns the names of the pins that failed."""
    failed = []
    checks = [("torch conv3d %d" % i, lambda c=c: pins.test_oracle_matches_torch_conv3d_float64(c))
              for i, c in enumerate(pins.CASES)]
    checks += [("impulse", pins.test_impulse_selects_one_weight_no_flip),
               ("bias once", pins.test_zero_weights_give_bias_exactly_once),
               ("streaming", lambda: pins.test_streaming_with_cache_carry_equals_one_shot_bitwise(
                   [1, 4, 4, 4], 1, 2, (3, 3, 3)))]
    for name, fn in checks:
        try:
            fn()
        except (AssertionError, ValueError):
            failed.append(name)
    return failed


@pytest.fixture
def swap_oracle(monkeypatch, tmp_path):
    def swap(text, tag):
        lib = _build(text, str(tmp_path / ("mut_%s.so" % tag)))
        monkeypatch.setattr(oracle, "_lib", lib)
    return swap


def test_unmutated_source_passes_every_pin(swap_oracle):
    swap_oracle(open(SRC).read(), "none")
    assert _pins() == []


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_each_planted_mistake_fails_a_pin(swap_oracle, name):
    text = open(SRC).read()
    old, new = MUTATIONS[name]
    assert text.count(old) == 1, "mutation site not found once: %s" % name
    swap_oracle(text.replace(old, new), "%d" % list(MUTATIONS).index(name))
    assert _pins(), "no pin caught: %s" % name
