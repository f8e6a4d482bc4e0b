"""Streaming comparison of a full-size GPU output against the fp64 oracle.

TEST INFRASTRUCTURE.  A full-size output (a 720x1280 frame of 96 channels is
708 MB in fp64) is compared output frame by output frame: the oracle computes
one frame at a time (points mode, every pixel of the frame), and the
comparator keeps only running sums -- max |d|, sum r^2, sum d^2, sum |d|,
sum g*r, sum g^2, NaN/Inf counts -- from which the metrics of the paper's
evaluation (max and mean abs, RMSE, cosine, non-finite counts; setup
section) and the bf16 bar (max |d| <= 2e-2 * RMS of the whole oracle output)
follow exactly as if the two tensors had been compared at once."""
import math

import numpy as np
import torch

import oracle
from gpu_util import BF16_REL_TOL, assert_bias_only_exact, bf16_step


class Comparator:
    def __init__(self, what=""):
        self.what = what
        self.n = 0
        self.max_abs = 0.0
        self.sum_abs = 0.0
        self.sum_d2 = 0.0
        self.sum_r2 = 0.0
        self.sum_g2 = 0.0
        self.sum_gr = 0.0
        self.nonfinite_gpu = 0
        self.nonfinite_ref = 0
        self.beyond_step = []  # per block: |d| - bf16 step at r, the largest (for the faithful-rounding bar)

    def add(self, got, ref, exclude=None):
        """Accumulate one block: got (tensor or array) against ref (fp64 array
        of the same number of elements); exclude: optional boolean mask,
        broadcast over channels, of positions left out."""
        g = got.detach().float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else \
            np.asarray(got, dtype=np.float64)
        r = np.asarray(ref, dtype=np.float64)
        g = g.reshape(r.shape)
        if exclude is not None:
            keep = ~np.broadcast_to(exclude, r.shape)
            g, r = g[keep], r[keep]
        self.nonfinite_gpu += int(np.sum(~np.isfinite(g)))
        self.nonfinite_ref += int(np.sum(~np.isfinite(r)))
        d = g - r
        self.n += r.size
        if r.size:
            self.max_abs = max(self.max_abs, float(np.max(np.abs(d))))
        self.sum_abs += float(np.sum(np.abs(d)))
        self.sum_d2 += float(np.sum(d * d))
        self.sum_r2 += float(np.sum(r * r))
        self.sum_g2 += float(np.sum(g * g))
        self.sum_gr += float(np.sum(g * r))
        if r.size:
            self.beyond_step.append(float(np.max(np.abs(d) - bf16_step(r))))

    def metrics(self):
        n = max(self.n, 1)
        denom = math.sqrt(self.sum_g2) * math.sqrt(self.sum_r2)
        return {
            "max_abs": self.max_abs, "mean_abs": self.sum_abs / n, "rmse": math.sqrt(self.sum_d2 / n),
            "rms_ref": math.sqrt(self.sum_r2 / n), "cos": self.sum_gr / denom if denom > 0 else 1.0,
            "nonfinite_gpu": self.nonfinite_gpu, "nonfinite_ref": self.nonfinite_ref, "count": self.n,
        }

    def assert_bf16(self, strict=False):
        """The bar of gpu_util.assert_bf16_close, on the running sums: max |d|
        <= 2e-2 x RMS, or (not strict) every output within one bf16 step of
        its fp64 value plus 1e-4 x RMS."""
        m = self.metrics()
        assert m["nonfinite_gpu"] == 0 and m["nonfinite_ref"] == 0, (self.what, m)
        if m["max_abs"] <= BF16_REL_TOL * m["rms_ref"]:
            return m
        assert not strict, (self.what, m)
        m["beyond_step"] = max(self.beyond_step, default=0.0)
        assert m["beyond_step"] <= 1e-4 * m["rms_ref"], (self.what, m)
        return m


def frame_points(n, o, ho, wo):
    """Every (n, o, i, j) of output frame o of batch item n."""
    i, j = np.meshgrid(np.arange(ho, dtype=np.int64), np.arange(wo, dtype=np.int64), indexing="ij")
    return np.stack([np.full(i.size, n, np.int64), np.full(i.size, o, np.int64), i.ravel(), j.ravel()], 1)


def compare_full(y, x, cache, w, b, what="", mask=None, strict=False, **conv):
    """Every output of y ([N][T_o][H_o][W_o][C_out] on the GPU) against the
    oracle over the same bf16 inputs (moved to the host once), frame by
    frame.  conv: the oracle's keyword arguments (stride, dilation, padding,
    pbase).  mask: optional bias-only mask ([N][T_o][H_o][W_o][1]); those
    outputs are checked bit for bit against the bias and left out of the
    tolerance comparison.  strict: the stated bar alone (no faithful-rounding
    fallback).  Returns the metrics."""
    xc = x.detach().cpu()
    cc = None if cache is None else cache.detach().cpu()
    wc = w.detach().cpu()
    bc = None if b is None else b.detach().cpu()
    n, to, ho, wo, _ = y.shape
    cmp = Comparator(what)
    if mask is not None:
        assert_bias_only_exact(y, b, mask, what)
    for nn in range(n):
        for o in range(to):
            ref = oracle.conv3d(xc, cc, wc, bc, points=frame_points(nn, o, ho, wo), **conv)
            cmp.add(y[nn, o], ref.reshape(ho, wo, -1), None if mask is None else mask[nn, o])
    return cmp.assert_bf16(strict)
