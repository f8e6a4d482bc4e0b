"""Test-side helpers for the GPU parity tests: run the library through its
binding, and compare against the oracle with the stated tolerances."""
import re

import numpy as np
import torch

import causal_conv3d_video_amd as cc3d

BF16_REL_TOL = 2e-2   # max |gpu - oracle| <= 2e-2 * RMS(oracle) for bf16 outputs
F32_ABS_TOL = 1e-4    # max |gpu - oracle| <= 1e-4 for fp32 outputs


def plan_for(x, tc, w, *, k, pad, dt=1, p_base=2, has_bias=True, dtype=torch.bfloat16, variant=None, st=1,
             sst=(1, 1), sdil=(1, 1)):
    n, tx, h, wd, cin = x.shape
    cout = w.shape[0]
    desc = cc3d.make_desc(n, cin, cout, h, wd, tx, tc, k=k, stride=(st,) + tuple(sst), dilation=(dt,) + tuple(sdil),
                          padding=pad, p_base=p_base, has_bias=has_bias, dtype=dtype)
    if variant is not None:
        return cc3d.causal_conv3d_plan_variant(desc, variant)
    return cc3d.causal_conv3d_plan(desc)


def run(x, cache, w, b, *, k=(3, 3, 3), pad=(1, 1), dt=1, p_base=2, want_cache=True, out=None, variant=None, st=1,
        sst=(1, 1), sdil=(1, 1)):
    """GPU forward through the C ABI; returns (out, cache_out, plan).  variant
    pins a kernel variant by name (default: the library's choice)."""
    tc = 0 if cache is None else cache.shape[1]
    plan = plan_for(x, tc, w, k=k, pad=pad, dt=dt, p_base=p_base, has_bias=b is not None, dtype=x.dtype,
                    variant=variant, st=st, sst=sst, sdil=sdil)
    sh = plan.shapes()
    if out is None:
        out = torch.empty(sh["out"], dtype=x.dtype, device=x.device)
    co = torch.empty(sh["cache_out"], dtype=x.dtype, device=x.device) if want_cache else None
    cc3d.causal_conv3d_forward(plan, x, cache, w, b, out, co)
    return out, co, plan


def metrics(got, ref):
    """The comparison metrics of the paper's evaluation: max and mean absolute
    difference, RMSE, cosine similarity (fp64 accumulation), NaN/Inf counts."""
    g = got.detach().float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else got
    r = np.asarray(ref, dtype=np.float64)
    g = g.reshape(r.shape)
    d = g - r
    rms = float(np.sqrt(np.mean(r * r)))
    denom = float(np.linalg.norm(g) * np.linalg.norm(r))
    return {
        "max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
        "mean_abs": float(np.mean(np.abs(d))) if d.size else 0.0,
        "rmse": float(np.sqrt(np.mean(d * d))) if d.size else 0.0,
        "rms_ref": rms,
        "cos": float(np.sum(g * r) / denom) if denom > 0 else 1.0,
        "nonfinite_gpu": int(np.sum(~np.isfinite(g))),
        "nonfinite_ref": int(np.sum(~np.isfinite(r))),
    }


def assert_bf16_close(got, ref, what=""):
    m = metrics(got, ref)
    assert m["nonfinite_gpu"] == 0 and m["nonfinite_ref"] == 0, (what, m)
    assert m["max_abs"] <= BF16_REL_TOL * m["rms_ref"], (what, m)
    return m


def assert_f32_close(got, ref, what=""):
    m = metrics(got, ref)
    assert m["nonfinite_gpu"] == 0, (what, m)
    assert m["max_abs"] <= F32_ABS_TOL, (what, m)
    return m


def tile_of(plan):
    """(rows, columns) of the plan's output tile, from its kernel name
    ("..._p<rows>x<cols>..."); (8, 32) for kernels without one."""
    m = re.search(r"_p(\d+)x(\d+)", plan.info["kernel_name"])
    return (int(m.group(1)), int(m.group(2))) if m else (8, 32)


def sample_points(n, to, ho, wo, count, seed, tile_h=8, tile_w=32):
    """Output positions to check at full size: all corners and edge midpoints,
    positions on both sides of every few workgroup-tile boundaries, and
    uniform random positions, for every batch item and output frame."""
    rng = np.random.default_rng(seed)
    pts = set()
    for nn in range(n):
        for o in range(to):
            for i in (0, 1, ho // 2, ho - 2, ho - 1):
                for j in (0, 1, wo // 2, wo - 2, wo - 1):
                    pts.add((nn, o, max(i, 0), max(j, 0)))
            for t in range(1, min(ho // tile_h, 6) + 1):
                i = t * tile_h
                for di in (-1, 0):
                    if 0 <= i + di < ho:
                        pts.add((nn, o, i + di, int(rng.integers(wo))))
            for t in range(1, min(wo // tile_w, 6) + 1):
                j = t * tile_w
                for dj in (-1, 0):
                    if 0 <= j + dj < wo:
                        pts.add((nn, o, int(rng.integers(ho)), j + dj))
    while len(pts) < count:
        pts.add((int(rng.integers(n)), int(rng.integers(to)), int(rng.integers(ho)), int(rng.integers(wo))))
    return np.array(sorted(pts), dtype=np.int64)


def gather(out, pts):
    """out[n, o, i, j, :] for each point, as a float64 numpy array."""
    idx = torch.from_numpy(pts).to(out.device)
    vals = out[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]]
    return vals.float().cpu().numpy().astype(np.float64)
