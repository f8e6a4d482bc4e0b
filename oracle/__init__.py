"""TEST INFRASTRUCTURE ONLY -- the CPU oracle for the cached causal Conv3D.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never imports or
links it, and it shares no code with the product library.

The arithmetic lives in ``cc3d_oracle.c`` (plain C, fp64, OpenMP).  It follows
"Cache-Aware Conv3D Lowering Across Embedded World-Model Decoders", lowering
section (the paper's Sec. 4): the source Z joins the temporal cache C ahead of
the input X; the causal left pad is p_l = p_base - |C|; tap k of output frame o
reads source time o*s_t + k*d_t - p_l and a time outside Z contributes zero;
each tap's spatial part is a bias-free PyTorch-convention Conv2D with the
original stride/padding/dilation, and the bias is added once.  This module only
marshals arrays to that C code, plus the cache carry, which is a plain slice of
Z (see ``cache_out``).

Layouts: activations [N][T][H][W][C] (channels last), weights
[Cout][Kt][Kh][Kw][Cin], bias [Cout].  Inputs may be float32 or bfloat16 (numpy
uint16 bit patterns or torch CPU tensors); both convert to float64 exactly.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cc3d_oracle.c")
_LIB = os.path.join(_HERE, "libcc3d_oracle.so")
_lib = None

__all__ = ["build", "out_shape", "conv3d", "cache_out", "pixels_u8", "default_threads"]


def build(force=True):
    """Compile the oracle's C source into ``libcc3d_oracle.so`` (gcc, OpenMP)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([
        "gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
        "-Wall", "-Wextra", "-o", tmp, _SRC])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64 = ctypes.c_int64
        lib.cc3d_oracle_conv3d.restype = ctypes.c_int
        lib.cc3d_oracle_conv3d.argtypes = (
            [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
            + [i64] * 19 + [ctypes.c_void_p, i64, ctypes.c_void_p, ctypes.c_int])
        lib.cc3d_oracle_out_shape.restype = ctypes.c_int
        lib.cc3d_oracle_out_shape.argtypes = [i64] * 16 + [ctypes.POINTER(i64)] * 3
        _lib = lib
    return _lib


def default_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _as_array(t):
    """Return (contiguous numpy array, dtype code): 0 float32, 1 bfloat16 bits."""
    if t is None:
        return None, None
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16), 1
            if t.dtype == torch.float32:
                return t.numpy(), 0
            raise TypeError("oracle inputs must be float32 or bfloat16, got %s" % t.dtype)
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(t)
    if a.dtype == np.float32:
        return a, 0
    if a.dtype == np.uint16:
        return a, 1
    raise TypeError("oracle inputs must be float32 or bfloat16 bits, got %s" % a.dtype)


def out_shape(tx, tc, h, w, kt=3, kh=3, kw=3, st=1, sh=1, sw=1, dt=1, dh=1, dw=1,
              ph=1, pw=1, pbase=2):
    """(To, Ho, Wo) of the cached causal Conv3D, or None when any is < 1."""
    lib = _load()
    r = [ctypes.c_int64() for _ in range(3)]
    bad = lib.cc3d_oracle_out_shape(tx, tc, h, w, kt, kh, kw, st, sh, sw, dt, dh, dw,
                                    ph, pw, pbase, *[ctypes.byref(v) for v in r])
    return None if bad else tuple(v.value for v in r)


def conv3d(x, cache, w, b, *, stride=(1, 1, 1), dilation=(1, 1, 1), padding=(1, 1),
           pbase=2, points=None, nthreads=None):
    """fp64 cached causal Conv3D over Z = [cache; x].

    x: [N][Tx][H][W][Cin]; cache: [N][Tc][H][W][Cin] or None (Tc = 0);
    w: [Cout][Kt][Kh][Kw][Cin]; b: [Cout] or None; stride = (s_t, s_h, s_w);
    dilation = (d_t, d_h, d_w); padding = (p_h, p_w) spatial zero pad;
    pbase = base causal left pad.  points: optional int array [P][4] of
    (n, o, i, j) output positions.  Returns float64 [N][To][Ho][Wo][Cout], or
    [P][Cout] when points is given.
    """
    xa, dx = _as_array(x)
    ca, dc = _as_array(cache)
    wa, dw_ = _as_array(w)
    ba, db = _as_array(b)
    codes = {d for d in (dx, dc, dw_, db) if d is not None}
    if len(codes) != 1:
        raise TypeError("x, cache, w and b must share one dtype")
    code = codes.pop()
    n, tx, h, wd, cin = xa.shape
    tc = 0 if ca is None else ca.shape[1]
    if ca is not None and (ca.shape[0] != n or ca.shape[2:] != (h, wd, cin)):
        raise ValueError("cache shape %s does not match x %s" % (ca.shape, xa.shape))
    if ca is not None and tc == 0:
        ca = None
    cout, kt, kh, kw, wcin = wa.shape
    if wcin != cin:
        raise ValueError("weight C_in %d != input C_in %d" % (wcin, cin))
    if ba is not None and ba.shape != (cout,):
        raise ValueError("bias must be [Cout]")
    st, sh, sw = stride
    dt, dh, dw = dilation
    ph, pw = padding
    shp = out_shape(tx, tc, h, wd, kt, kh, kw, st, sh, sw, dt, dh, dw, ph, pw, pbase)
    if shp is None:
        raise ValueError("empty output for these sizes")
    to, ho, wo = shp
    if points is None:
        pts = None
        out = np.empty((n, to, ho, wo, cout), dtype=np.float64)
        npts = 0
    else:
        pts = np.ascontiguousarray(np.asarray(points, dtype=np.int64).reshape(-1, 4))
        npts = pts.shape[0]
        out = np.empty((npts, cout), dtype=np.float64)
    rc = _load().cc3d_oracle_conv3d(
        xa.ctypes.data, None if ca is None else ca.ctypes.data, code,
        wa.ctypes.data, None if ba is None else ba.ctypes.data,
        n, tx, tc, h, wd, cin, cout, kt, kh, kw, st, sh, sw, dt, dh, dw, ph, pw, pbase,
        None if pts is None else pts.ctypes.data, npts, out.ctypes.data,
        int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected the call (code %d)" % rc)
    return out


def cache_out(x, cache, pbase):
    """The temporal cache carried to the next call: the last min(p_base, |Z|)
    frames of Z = [cache; x] (the cache holds the previous chunk's trailing
    source frames, which the next call's causal taps read).  Returns an array
    of the input's own dtype (torch tensors come back as numpy bit patterns)."""
    xa, _ = _as_array(x)
    ca, _ = _as_array(cache)
    z = xa if ca is None or ca.shape[1] == 0 else np.concatenate([ca, xa], axis=1)
    keep = min(pbase, z.shape[1])
    return z[:, z.shape[1] - keep:].copy()


def pixels_u8(y, scale=0.5, offset=0.5):
    """8-bit pixel codes of decoded frames, following the FastVideo pull
    request "[perf] Quantize frames to uint8 on-device before the post-decode
    D->H copy" (Summary and Correctness sections): the frames are scaled by
    255, clamped to [0, 255] and cast to uint8, and the cast truncates.  The
    page starts from frames in [0, 1]; the head output y is mapped there first
    by y*scale + offset (0.5, 0.5 maps [-1, 1] to [0, 1]; the usual decoder
    convention, not on the pages).

    The decision is taken in fp32, the precision of the frames on that page:
    y is rounded to fp32, y*scale + offset is rounded once to fp32 (a fused
    multiply-add), and the product by 255 is rounded to fp32.  NaN gives 0."""
    y32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    v = (y32.astype(np.float64) * np.float64(np.float32(scale)) + np.float64(np.float32(offset))).astype(np.float32)
    p = v * np.float32(255)
    p = np.where(np.isnan(p), np.float32(0), p)
    return np.trunc(np.clip(p, np.float32(0), np.float32(255))).astype(np.uint8)
