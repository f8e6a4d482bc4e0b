"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle (oracle/cc3d_oracle.c) against something fixed by
"Cache-Aware Conv3D Lowering Across Embedded World-Model Decoders" (lowering
section, the paper's Sec. 4) or by mathematics:

* a pure-Python brute force over an explicitly zero-padded Z (padding
  materialised, rather than out-of-range terms skipped);
* torch.nn.functional.conv3d in float64 over the explicitly built
  [p_l zero frames; C; X] (the cached causal Conv3D is, by the page, the
  original Conv3D on that source);
* the per-tap identity: bias once plus the sum over active taps of bias-free
  torch conv2d responses (the page's reconstruction of Conv3D from Conv2D);
* closed forms: an impulse picks out one weight (cross-correlation, no flip,
  tap order), zero weights leave exactly the bias (bias added once), a
  1x1x1 kernel is a matrix product;
* streaming: chunked calls that carry the last p_base frames of Z equal one
  call over the whole sequence, bit for bit.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _rand(shape, rng, dtype=np.float32):
    return rng.uniform(-1, 1, size=shape).astype(dtype)


def _padded_source(x, cache, pbase):
    """[p_l zero frames; C; X] as float64 NTHWC (frames dropped when p_l < 0)."""
    z = x.astype(np.float64) if cache is None else np.concatenate([cache, x], axis=1).astype(np.float64)
    pl = pbase - (0 if cache is None else cache.shape[1])
    if pl >= 0:
        zeros = np.zeros((z.shape[0], pl) + z.shape[2:], dtype=np.float64)
        return np.concatenate([zeros, z], axis=1)
    return z[:, -pl:]


def _torch_ref(x, cache, w, b, stride, dilation, padding, pbase):
    zp = torch.from_numpy(_padded_source(x, cache, pbase)).permute(0, 4, 1, 2, 3)  # NCDHW
    wt = torch.from_numpy(w.astype(np.float64)).permute(0, 4, 1, 2, 3)             # OIDHW
    bt = None if b is None else torch.from_numpy(b.astype(np.float64))
    y = F.conv3d(zp, wt, bt, stride=stride, padding=(0,) + tuple(padding), dilation=dilation)
    return y.permute(0, 2, 3, 4, 1).numpy()


def _brute(x, cache, w, b, stride, dilation, padding, pbase):
    """7-deep Python loops over an explicitly zero-padded source."""
    zp = _padded_source(x, cache, pbase)
    ph, pw = padding
    n, tz, h, wd, cin = zp.shape
    padded = np.zeros((n, tz, h + 2 * ph, wd + 2 * pw, cin))
    padded[:, :, ph:ph + h, pw:pw + wd] = zp
    cout, kt, kh, kw, _ = w.shape
    st, sh, sw = stride
    dt, dh, dw = dilation
    to = (tz - dt * (kt - 1) - 1) // st + 1
    ho = (h + 2 * ph - dh * (kh - 1) - 1) // sh + 1
    wo = (wd + 2 * pw - dw * (kw - 1) - 1) // sw + 1
    y = np.zeros((n, to, ho, wo, cout))
    for nn, o, i, j, co in itertools.product(range(n), range(to), range(ho), range(wo), range(cout)):
        s = 0.0 if b is None else float(b[co])
        for k, a, c, ci in itertools.product(range(kt), range(kh), range(kw), range(cin)):
            s += padded[nn, o * st + k * dt, i * sh + a * dh, j * sw + c * dw, ci] * float(w[co, k, a, c, ci])
        y[nn, o, i, j, co] = s
    return y


def _call(x, cache, w, b, stride=(1, 1, 1), dilation=(1, 1, 1), padding=(1, 1), pbase=2, **kw):
    return oracle.conv3d(x, cache, w, b, stride=stride, dilation=dilation, padding=padding,
                         pbase=pbase, **kw)


CASES = [
    # (N, Tx, Tc, H, W, Cin, Cout, k, stride, dilation, padding, pbase)
    (1, 4, 0, 16, 16, 8, 8, (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1), 2),   # tiny call A
    (1, 4, 2, 16, 16, 8, 8, (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1), 2),   # tiny call B
    (2, 1, 0, 6, 7, 4, 5, (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1), 2),     # 1-frame, only last tap
    (1, 1, 1, 6, 5, 4, 3, (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1), 2),     # p_l = 1
    (1, 3, 4, 5, 6, 3, 4, (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1), 2),     # |C| > p_base
    (1, 4, 4, 5, 5, 3, 2, (3, 3, 3), (1, 1, 1), (2, 1, 1), (1, 1), 4),     # temporal dilation 2
    (1, 4, 2, 5, 5, 3, 2, (3, 3, 3), (1, 1, 1), (2, 1, 1), (1, 1), 4),     # d_t=2, short cache
    (1, 3, 2, 6, 6, 4, 6, (3, 1, 1), (1, 1, 1), (1, 1, 1), (0, 0), 2),     # temporal-only conv
    (1, 5, 2, 9, 8, 3, 2, (3, 3, 3), (2, 2, 2), (1, 2, 1), (2, 1), 2),     # strides, dilation
    (1, 3, 1, 7, 6, 2, 3, (2, 3, 1), (1, 1, 1), (1, 1, 1), (1, 0), 1),     # other kernel sizes
]


@pytest.mark.parametrize("case", CASES)
def test_oracle_matches_torch_conv3d_float64(case):
    n, tx, tc, h, w, cin, cout, k, stride, dil, pad, pbase = case
    rng = np.random.default_rng(1000 + CASES.index(case))
    x = _rand((n, tx, h, w, cin), rng)
    c = _rand((n, tc, h, w, cin), rng) if tc else None
    wt = _rand((cout,) + k + (cin,), rng)
    b = _rand((cout,), rng)
    got = _call(x, c, wt, b, stride, dil, pad, pbase)
    ref = _torch_ref(x, c, wt, b, stride, dil, pad, pbase)
    assert got.shape == ref.shape
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("case", [CASES[1], CASES[4], CASES[6], CASES[8]])
def test_oracle_matches_python_brute_force(case):
    n, tx, tc, h, w, cin, cout, k, stride, dil, pad, pbase = case
    rng = np.random.default_rng(2000 + CASES.index(case))
    h, w, cin, cout = min(h, 6), min(w, 6), min(cin, 3), min(cout, 3)
    x = _rand((n, tx, h, w, cin), rng)
    c = _rand((n, tc, h, w, cin), rng) if tc else None
    wt = _rand((cout,) + k + (cin,), rng)
    b = _rand((cout,), rng)
    got = _call(x, c, wt, b, stride, dil, pad, pbase)
    ref = _brute(x, c, wt, b, stride, dil, pad, pbase)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_impulse_selects_one_weight_no_flip():
    """A single unit source value at (t0, u0, v0, c0) puts W[co, c0, k, a, c] + b
    exactly at o = t0 + p_l - k, i = u0 + p_h - a, j = v0 + p_w - c."""
    rng = np.random.default_rng(7)
    n, tx, tc, h, wd, cin, cout, pbase = 1, 4, 2, 6, 7, 3, 4, 2
    wt = _rand((cout, 3, 3, 3, cin), rng)
    b = _rand((cout,), rng)
    for (t0, u0, v0, c0) in [(0, 0, 0, 0), (1, 3, 4, 2), (3, 5, 6, 1), (5, 2, 0, 0)]:
        x = np.zeros((n, tx, h, wd, cin), np.float32)
        c = np.zeros((n, tc, h, wd, cin), np.float32)
        if t0 < tc:
            c[0, t0, u0, v0, c0] = 1.0
        else:
            x[0, t0 - tc, u0, v0, c0] = 1.0
        y = _call(x, c, wt, b, pbase=pbase)
        pl = pbase - tc
        expect = np.broadcast_to(b.astype(np.float64), y.shape).copy()
        for k, a, cc in itertools.product(range(3), range(3), range(3)):
            o, i, j = t0 + pl - k, u0 + 1 - a, v0 + 1 - cc
            if 0 <= o < y.shape[1] and 0 <= i < h and 0 <= j < wd:
                expect[0, o, i, j] = b.astype(np.float64) + wt[:, k, a, cc, c0].astype(np.float64)
        assert np.array_equal(y, expect)


def test_zero_weights_give_bias_exactly_once():
    rng = np.random.default_rng(8)
    x = _rand((1, 4, 5, 5, 3), rng)
    c = _rand((1, 2, 5, 5, 3), rng)
    b = _rand((4,), rng)
    y = _call(x, c, np.zeros((4, 3, 3, 3, 3), np.float32), b)
    assert np.array_equal(y, np.broadcast_to(b.astype(np.float64), y.shape))
    y0 = _call(x, c, np.zeros((4, 3, 3, 3, 3), np.float32), None)
    assert np.array_equal(y0, np.zeros_like(y0))


def test_pointwise_kernel_is_matrix_product():
    rng = np.random.default_rng(9)
    x = _rand((2, 3, 4, 5, 6), rng)
    wt = _rand((7, 1, 1, 1, 6), rng)
    b = _rand((7,), rng)
    y = _call(x, None, wt, b, padding=(0, 0), pbase=0)
    ref = x.astype(np.float64).reshape(-1, 6) @ wt.reshape(7, 6).T.astype(np.float64) + b
    np.testing.assert_allclose(y.reshape(-1, 7), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("tc,dt,pbase", [(0, 1, 2), (1, 1, 2), (2, 1, 2), (3, 1, 2), (2, 2, 4), (4, 2, 4)])
def test_tap_sum_identity_with_conv2d(tc, dt, pbase):
    """bias + sum over active taps of bias-free spatial Conv2D responses."""
    rng = np.random.default_rng(10 + tc + 10 * dt)
    n, tx, h, wd, cin, cout = 1, 3, 6, 5, 4, 3
    x = _rand((n, tx, h, wd, cin), rng)
    c = _rand((n, tc, h, wd, cin), rng) if tc else None
    wt = _rand((cout, 3, 3, 3, cin), rng)
    b = _rand((cout,), rng)
    y = _call(x, c, wt, b, dilation=(dt, 1, 1), pbase=pbase)
    z = x if c is None else np.concatenate([c, x], axis=1)
    pl = pbase - tc
    for o in range(y.shape[1]):
        acc = torch.from_numpy(np.broadcast_to(b.astype(np.float64), (n, h, wd, cout)).copy())
        for k in range(3):
            t = o + k * dt - pl
            if 0 <= t < z.shape[1]:
                zi = torch.from_numpy(z[:, t].astype(np.float64)).permute(0, 3, 1, 2)
                wk = torch.from_numpy(wt[:, k].astype(np.float64)).permute(0, 3, 1, 2)
                acc = acc + F.conv2d(zi, wk, None, padding=1).permute(0, 2, 3, 1)
        np.testing.assert_allclose(y[:, o], acc.numpy(), rtol=0, atol=1e-12)


def test_linearity_in_source():
    # values on a 1/64 grid so that x1 + x2 is exact in float32
    rng = np.random.default_rng(11)
    q = lambda shape: (rng.integers(-64, 65, size=shape) / 64.0).astype(np.float32)
    x1, x2 = q((1, 3, 5, 5, 3)), q((1, 3, 5, 5, 3))
    c1, c2 = q((1, 2, 5, 5, 3)), q((1, 2, 5, 5, 3))
    wt = _rand((2, 3, 3, 3, 3), rng)
    y1 = _call(x1, c1, wt, None)
    y2 = _call(x2, c2, wt, None)
    y12 = _call(x1 + x2, c1 + c2, wt, None)
    np.testing.assert_allclose(y12, y1 + y2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("frames,dt,pbase,k", [
    ([4, 4, 4, 4, 4], 1, 2, (3, 3, 3)),
    ([1, 1, 1, 1, 1], 1, 2, (3, 3, 3)),     # one latent frame per chunk: cache grows 1, 2, 2, ...
    ([1, 4, 4, 4, 4], 1, 2, (3, 3, 3)),
    ([4, 4, 4, 4, 4], 2, 4, (3, 3, 3)),     # temporal dilation 2 with a p_base-deep carry
    ([1, 2, 1, 3], 2, 4, (3, 3, 3)),
    ([1, 1, 1], 1, 2, (3, 1, 1)),
])
def test_streaming_with_cache_carry_equals_one_shot_bitwise(frames, dt, pbase, k):
    rng = np.random.default_rng(12 + sum(frames) + dt)
    h, wd, cin, cout = 5, 4, 3, 2
    pad = (1, 1) if k[1] == 3 else (0, 0)
    xs = [_rand((1, f, h, wd, cin), rng) for f in frames]
    wt = _rand((cout,) + k + (cin,), rng)
    b = _rand((cout,), rng)
    whole = _call(np.concatenate(xs, axis=1), None, wt, b, dilation=(dt, 1, 1), padding=pad, pbase=pbase)
    cache, outs = None, []
    for xc in xs:
        outs.append(_call(xc, cache, wt, b, dilation=(dt, 1, 1), padding=pad, pbase=pbase))
        cache = oracle.cache_out(xc, cache, pbase)
    chunked = np.concatenate(outs, axis=1)
    assert chunked.shape == whole.shape
    assert np.array_equal(chunked, whole)


@pytest.mark.parametrize("frames,st,k", [
    ([4, 4, 4], 2, (3, 3, 3)),
    ([2, 4, 2, 6], 2, (3, 3, 3)),
    ([4, 2, 4], 2, (3, 1, 1)),   # the encoder's temporal downsampling conv
    ([3, 6, 3], 3, (3, 3, 3)),
])
def test_strided_streaming_with_cache_carry_equals_one_shot_bitwise(frames, st, k):
    """Temporal stride s_t with p_base = d_t*(k_t-1): when every chunk's
    length is a multiple of s_t, chunked calls carrying the last p_base
    frames of Z equal one call over the whole sequence (chunk c's first
    output is whole-sequence output sum(frames[:c]) / s_t)."""
    rng = np.random.default_rng(40 + sum(frames) + st)
    h, wd, cin, cout = 5, 4, 3, 2
    pad = (1, 1) if k[1] == 3 else (0, 0)
    xs = [_rand((1, f, h, wd, cin), rng) for f in frames]
    wt = _rand((cout,) + k + (cin,), rng)
    b = _rand((cout,), rng)
    whole = _call(np.concatenate(xs, axis=1), None, wt, b, stride=(st, 1, 1), padding=pad, pbase=2)
    assert whole.shape[1] == sum(frames) // st
    cache, outs = None, []
    for xc in xs:
        outs.append(_call(xc, cache, wt, b, stride=(st, 1, 1), padding=pad, pbase=2))
        cache = oracle.cache_out(xc, cache, 2)
    assert np.array_equal(np.concatenate(outs, axis=1), whole)


def test_points_mode_equals_full_and_thread_count_does_not_matter():
    rng = np.random.default_rng(13)
    x = _rand((2, 4, 7, 9, 5), rng)
    c = _rand((2, 2, 7, 9, 5), rng)
    wt = _rand((6, 3, 3, 3, 5), rng)
    b = _rand((6,), rng)
    full = _call(x, c, wt, b, nthreads=4)
    one = _call(x, c, wt, b, nthreads=1)
    assert np.array_equal(full, one)
    pts = np.array([[0, 0, 0, 0], [1, 3, 6, 8], [0, 2, 3, 4], [1, 1, 0, 8]])
    got = _call(x, c, wt, b, points=pts)
    for p, row in zip(pts, got):
        assert np.array_equal(row, full[tuple(p)])


def test_bfloat16_inputs_convert_exactly():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(1, 3, 4, 4, 8, generator=g).to(torch.bfloat16)
    c = torch.randn(1, 2, 4, 4, 8, generator=g).to(torch.bfloat16)
    wt = torch.randn(4, 3, 3, 3, 8, generator=g).to(torch.bfloat16)
    b = torch.randn(4, generator=g).to(torch.bfloat16)
    got = oracle.conv3d(x, c, wt, b)
    ref = oracle.conv3d(x.float(), c.float(), wt.float(), b.float())
    assert np.array_equal(got, ref)


def test_cache_out_is_last_frames_of_source():
    rng = np.random.default_rng(14)
    xa = _rand((1, 4, 3, 3, 2), rng)
    # no cache: the carry is the last two frames of X
    assert np.array_equal(oracle.cache_out(xa, None, 2), xa[:, 2:4])
    # one-frame X behind a one-frame cache: carry is [C; X]
    c1, x1 = _rand((1, 1, 3, 3, 2), rng), _rand((1, 1, 3, 3, 2), rng)
    assert np.array_equal(oracle.cache_out(x1, c1, 2), np.concatenate([c1, x1], axis=1))
    # one-frame X, no cache: carry is that one frame (no zero fill)
    assert np.array_equal(oracle.cache_out(x1, None, 2), x1)
    # p_base = 4 keeps four frames
    assert np.array_equal(oracle.cache_out(xa, c1, 4), np.concatenate([c1, xa], axis=1)[:, 1:])


def test_output_length_rule():
    # p_base = d_t*(k_t-1) keeps T_o = |X| for any cache depth
    for tx in range(1, 6):
        for tc in range(0, 5):
            assert oracle.out_shape(tx, tc, 4, 4, pbase=2)[0] == tx
            assert oracle.out_shape(tx, tc, 4, 4, dt=2, pbase=4)[0] == tx
    assert oracle.out_shape(4, 0, 16, 16, pbase=2) == (4, 16, 16)
    assert oracle.out_shape(4, 2, 16, 16, pbase=2) == (4, 16, 16)
    assert oracle.out_shape(1, 0, 90, 160, pbase=2) == (1, 90, 160)
    assert oracle.out_shape(4, 4, 8, 8, dt=2, pbase=4) == (4, 8, 8)
    assert oracle.out_shape(4, 2, 8, 8, dt=2, pbase=4) == (4, 8, 8)
    assert oracle.out_shape(1, 0, 8, 8, pbase=0) is None


# --- pixel quantisation of the head output (FastVideo pull request "[perf]
# Quantize frames to uint8 on-device before the post-decode D->H copy",
# Summary and Correctness: scale by 255, clamp to [0, 255], truncating uint8
# cast; y mapped to [0, 1] by y*0.5 + 0.5 first) ---

def test_pixel_codes_at_exact_points():
    """Points where every fp32 step is exact: truncation, not rounding
    (0 -> 127.5 -> 127), both clamps, and the affine map's offset and scale."""
    y = np.array([-3.0, -1.0, -0.5, 0.0, 0.5, 1.0, 3.0])
    assert oracle.pixels_u8(y).tolist() == [0, 0, 63, 127, 191, 255, 255]
    # another affine map: y already in [0, 1]
    assert oracle.pixels_u8(np.array([0.0, 0.25, 1.0, 1.5]), scale=1.0, offset=0.0).tolist() == [0, 63, 255, 255]
    assert oracle.pixels_u8(np.array([np.nan])).tolist() == [0]


def test_pixel_codes_match_torch_float32_pipeline():
    """With scale 0.5 the product y*0.5 is exact, so the fused map equals the
    plain torch float32 pipeline (y*0.5 + 0.5) * 255, clamp, uint8 cast."""
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.normal(0, 1.2, 200000), np.linspace(-1.1, 1.1, 50001)])
    t = torch.from_numpy(y).to(torch.float32)
    ref = ((t * 0.5 + 0.5) * 255).clamp(0, 255).to(torch.uint8).numpy()
    got = oracle.pixels_u8(y)
    assert np.array_equal(got, ref)
    # monotone in y, and every code is reached
    order = np.argsort(y, kind="stable")
    assert np.all(np.diff(got[order].astype(int)) >= 0)
    assert set(np.unique(got).tolist()) == set(range(256))
