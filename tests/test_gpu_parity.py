"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Tolerances: fp32 outputs within 1e-4 max-abs; bf16 outputs within
2e-2 x RMS(oracle) max-abs, the oracle computed in fp64 from the very same
bf16-rounded inputs; outputs that only the bias reaches equal it bit for bit.
The cache carry is compared byte for byte.  Every output is compared, also
at full size (frame by frame through the streaming comparator), and every
output buffer is NaN-filled before the launch that writes it.
"""
import numpy as np
import pytest
import torch

import causal_conv3d_video_amd as cc3d
import oracle
import synth
from comparator import compare_full, frame_points
from gpu_util import (assert_bf16_close, assert_bias_only_exact, assert_f32_close, gather, mask_for, nan_like,
                      plan_for, run, workspace_for)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np(t):
    return None if t is None else t.detach().cpu()


def _oracle(x, cache, w, b, *, k=(3, 3, 3), pad=(1, 1), dt=1, p_base=2, points=None, st=1, sst=(1, 1),
            sdil=(1, 1)):
    return oracle.conv3d(_np(x), _np(cache), _np(w), _np(b), stride=(st,) + tuple(sst), dilation=(dt,) + tuple(sdil),
                         padding=pad, pbase=p_base, points=points)


def test_tiny_fp32_calls_a_then_b(cuda_device):
    s = synth.TINY
    g = torch.Generator(device=DEV).manual_seed(synth.SEED_BASE)
    w = synth.draw((8, 3, 3, 3, 8), "uniform", g, DEV, torch.float32, 1.0)
    b = synth.draw((8,), "uniform", g, DEV, torch.float32, 0.1)
    xa = synth.draw((1, 4, 16, 16, 8), "uniform", g, DEV, torch.float32, 1.0)
    xb = synth.draw((1, 4, 16, 16, 8), "uniform", g, DEV, torch.float32, 1.0)
    # call A: no cache, p_l = 2
    ya, ca, plan_a = run(xa, None, w, b, p_base=s["p_base"])
    assert plan_a.info["p_l"] == 2 and plan_a.info["t_out"] == 4
    torch.cuda.synchronize()
    assert torch.equal(ca, xa[:, 2:4])
    assert_f32_close(ya, _oracle(xa, None, w, b), "call A")
    # call B: A's last two frames as cache, p_l = 0
    yb, cb, plan_b = run(xb, ca, w, b, p_base=s["p_base"])
    assert plan_b.info["p_l"] == 0 and plan_b.info["t_out"] == 4
    torch.cuda.synchronize()
    assert torch.equal(cb, xb[:, 2:4])
    assert_f32_close(yb, _oracle(xb, ca, w, b), "call B")
    # the two calls together equal one call over all eight frames
    whole = _oracle(torch.cat([xa, xb], 1), None, w, b)
    assert_f32_close(torch.cat([ya, yb], 1), whole, "A+B vs one shot")


# (C_in, C_out, H, W, T_x, T_cache, k, d_t, p_base, N, bias): shapes that hit
# every kernel variant with ragged tiles in both spatial directions.
SMALL = [
    (32, 192, 19, 45, 3, 2, (3, 3, 3), 1, 2, 1, True),    # 192-channel tile, ragged rows/cols
    (48, 96, 21, 37, 2, 1, (3, 3, 3), 1, 2, 1, True),     # 96-channel tile
    (16, 40, 9, 33, 1, 0, (3, 3, 3), 1, 2, 1, True),      # 32-channel tile, partial second block
    (32, 3, 10, 70, 4, 2, (3, 3, 3), 1, 2, 1, True),      # 3 output channels
    (64, 384, 11, 40, 1, 2, (3, 3, 3), 1, 2, 1, True),    # two 192-channel blocks
    (64, 192, 9, 50, 1, 2, (3, 1, 1), 1, 2, 1, True),     # temporal-only conv, 64-channel stages
    (48, 20, 5, 40, 2, 1, (3, 1, 1), 1, 2, 1, True),      # temporal-only, 16-channel stages
    (32, 768, 7, 33, 1, 1, (3, 1, 1), 1, 2, 1, True),     # temporal-only, 4 channel blocks
    (32, 96, 12, 34, 2, 2, (3, 3, 3), 1, 2, 2, True),     # batch of 2
    (32, 192, 10, 40, 4, 4, (3, 3, 3), 2, 4, 1, True),    # temporal dilation 2, 4-frame carry
    (32, 192, 10, 40, 4, 2, (3, 3, 3), 2, 4, 1, True),    # d_t = 2 behind a 2-frame cache
    (32, 96, 8, 32, 3, 3, (3, 3, 3), 1, 2, 1, True),      # |C| > p_base: leading frame unused
    (32, 96, 8, 32, 3, 1, (2, 3, 3), 1, 1, 1, True),      # k_t = 2
    (32, 96, 8, 32, 3, 0, (1, 3, 3), 1, 0, 1, True),      # k_t = 1
    (32, 192, 16, 64, 2, 2, (3, 3, 3), 1, 2, 1, False),   # no bias
    (16, 32, 1, 1, 1, 0, (3, 3, 3), 1, 2, 1, True),       # 1x1 frame: halo all padding
]


@pytest.mark.parametrize("case", SMALL, ids=[str(i) for i in range(len(SMALL))])
def test_bf16_small_shapes_full_compare(cuda_device, case):
    cin, cout, h, w_, tx, tc, k, dt, p_base, n, bias = case
    pad = (1, 1) if k[1] == 3 else (0, 0)
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV,
                                   seed=synth.SEED_BASE + 100 + SMALL.index(case), has_bias=bias)
    y, co, plan = run(x, c, w, b, k=k, pad=pad, dt=dt, p_base=p_base)
    torch.cuda.synchronize()
    ref = _oracle(x, c, w, b, k=k, pad=pad, dt=dt, p_base=p_base)
    assert tuple(y.shape) == ref.shape
    assert_bf16_close(y, ref, plan.info["kernel_name"])
    z = x if c is None else torch.cat([c, x], 1)
    keep = min(p_base, z.shape[1])
    assert torch.equal(co, z[:, z.shape[1] - keep:])


# (C_in, C_out, H, W, T_x, T_cache, k, d_t, p_base, N, bias) run on the
# group-staged 16x32 kernel (the default for large maps only), full compare.
GROUP_STAGED = [
    (32, 96, 20, 70, 2, 2, (3, 3, 3), 1, 2, 1, True),    # ragged rows (2nd patch row: 4 of 16) and columns
    (64, 192, 17, 45, 3, 2, (3, 3, 3), 1, 2, 1, True),   # 2 channel groups, 2 channel blocks, 1-row tail
    (96, 96, 33, 64, 4, 2, (3, 3, 3), 1, 2, 1, True),    # 3 channel groups, exact columns
    (32, 96, 16, 32, 1, 0, (3, 3, 3), 1, 2, 2, True),    # batch 2, one active tap (p_l = 2)
    (32, 96, 18, 40, 4, 2, (3, 3, 3), 2, 4, 1, True),    # temporal dilation 2
    (32, 96, 16, 40, 3, 1, (2, 3, 3), 1, 1, 1, True),    # k_t = 2
    (64, 96, 16, 33, 2, 0, (3, 3, 3), 1, 4, 1, True),    # p_base > (k_t-1)*d_t: bias-only frames
    (32, 192, 24, 50, 2, 3, (3, 3, 3), 1, 2, 1, False),  # no bias, |C| > p_base
    (32, 96, 16, 40, 1, 4, (3, 3, 3), 2, 4, 1, True),    # d_t = 2, one new frame: some carried frames
                                                          # are read by no tap (copied, not fused)
]


# The same checks on the group-staged 24x32-pixel x 64-channel tile (three
# rows per wave; C_out a multiple of 64).
GROUP_STAGED_N64 = [
    (32, 64, 30, 70, 2, 2, (3, 3, 3), 1, 2, 1, True),    # ragged rows (2nd patch row: 6 of 24) and columns
    (64, 128, 25, 45, 3, 2, (3, 3, 3), 1, 2, 1, True),   # 2 channel groups, 2 channel blocks, 1-row tail
    (96, 192, 48, 64, 4, 2, (3, 3, 3), 1, 2, 1, True),   # 3 channel groups, 3 blocks, exact rows and columns
    (32, 64, 24, 32, 1, 0, (3, 3, 3), 1, 2, 2, True),    # batch 2, one active tap (p_l = 2)
    (32, 64, 26, 40, 4, 2, (3, 3, 3), 2, 4, 1, True),    # temporal dilation 2
    (32, 64, 24, 40, 3, 1, (2, 3, 3), 1, 1, 1, True),    # k_t = 2
    (64, 64, 24, 33, 2, 0, (3, 3, 3), 1, 4, 1, True),    # p_base > (k_t-1)*d_t: bias-only frames
    (32, 384, 20, 50, 2, 3, (3, 3, 3), 1, 2, 1, False),  # no bias, |C| > p_base, 6 blocks, one patch row
    (64, 64, 64, 96, 1, 2, (3, 3, 3), 1, 2, 2, True),    # batch 2, one new frame: each item's cache-out is a
                                                          # cached and a new frame, 7 copy chunks each (one ragged)
]


def _pinned_case(case, seed, variant):
    cin, cout, h, w_, tx, tc, k, dt, p_base, n, bias = case
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV, seed=seed, has_bias=bias)
    y, co, plan = run(x, c, w, b, k=k, dt=dt, p_base=p_base, variant=variant)
    torch.cuda.synchronize()
    assert plan.info["kernel_name"] == variant
    ref = _oracle(x, c, w, b, k=k, dt=dt, p_base=p_base)
    assert tuple(y.shape) == ref.shape
    assert_bf16_close(y, ref, variant)
    z = x if c is None else torch.cat([c, x], 1)
    keep = min(p_base, z.shape[1])
    assert torch.equal(co, z[:, z.shape[1] - keep:])


@pytest.mark.parametrize("case", GROUP_STAGED_N64, ids=[str(i) for i in range(len(GROUP_STAGED_N64))])
def test_bf16_group_staged_n64_full_compare(cuda_device, case):
    _pinned_case(case, synth.SEED_BASE + 360 + GROUP_STAGED_N64.index(case), "bf16_s3_n64_p24x32_g32")


@pytest.mark.parametrize("variant", ["bf16_s3_n96_p16x32_g32", "bf16_s3_n96_p8x32_x2"])
@pytest.mark.parametrize("case", GROUP_STAGED, ids=[str(i) for i in range(len(GROUP_STAGED))])
def test_bf16_pinned_variants_full_compare(cuda_device, case, variant):
    cin, cout, h, w_, tx, tc, k, dt, p_base, n, bias = case
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV,
                                   seed=synth.SEED_BASE + 300 + GROUP_STAGED.index(case), has_bias=bias)
    y, co, plan = run(x, c, w, b, k=k, dt=dt, p_base=p_base, variant=variant)
    torch.cuda.synchronize()
    assert plan.info["kernel_name"] == variant
    ref = _oracle(x, c, w, b, k=k, dt=dt, p_base=p_base)
    assert tuple(y.shape) == ref.shape
    assert_bf16_close(y, ref, variant)
    z = x if c is None else torch.cat([c, x], 1)
    assert torch.equal(co, z[:, z.shape[1] - min(p_base, z.shape[1]):])


# (C_in, C_out, H, W, T_x, T_cache, p_base, N, bias) on the few-output-channel
# kernel (frames walked in time order, halo rows streamed, tap slots rotated
# across lanes).
FEW_CHANNELS = [
    (96, 3, 20, 70, 4, 2, 2, 1, True),     # the RGB head's channels, ragged patches
    (32, 1, 17, 33, 3, 0, 2, 1, True),     # one output channel, no cache (p_l = 2)
    (64, 5, 16, 32, 2, 3, 2, 1, True),     # five channels, |C| > p_base (leading frame unused)
    (96, 3, 18, 40, 2, 0, 4, 1, True),     # p_base = 4: two bias-only output frames
    (32, 2, 9, 50, 5, 1, 2, 2, False),     # batch 2, no bias, p_l = 1
    (64, 4, 33, 65, 1, 2, 2, 1, True),     # a single new frame behind a 2-frame cache
    (96, 3, 37, 300, 2, 2, 2, 1, True),    # three 128-column strips, the last ragged
    (64, 3, 21, 129, 3, 2, 2, 1, True),    # a second strip of one column
]
# patch heights: the tallest, and an odd short one (several patches per
# column, rows past the patch height computed and dropped)
FEW_HEIGHTS = ["bf16_s3_few_p16x128", "bf16_s3_few_p5x128"]


@pytest.mark.parametrize("variant", FEW_HEIGHTS)
@pytest.mark.parametrize("case", FEW_CHANNELS, ids=[str(i) for i in range(len(FEW_CHANNELS))])
def test_bf16_few_channel_kernel_full_compare(cuda_device, case, variant):
    cin, cout, h, w_, tx, tc, p_base, n, bias = case
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, device=DEV,
                                   seed=synth.SEED_BASE + 400 + FEW_CHANNELS.index(case), has_bias=bias)
    y, co, plan = run(x, c, w, b, p_base=p_base, variant=variant)
    torch.cuda.synchronize()
    assert plan.info["kernel_name"] == variant
    ref = _oracle(x, c, w, b, p_base=p_base)
    assert tuple(y.shape) == ref.shape
    assert_bf16_close(y, ref, "few")
    z = x if c is None else torch.cat([c, x], 1)
    assert torch.equal(co, z[:, z.shape[1] - min(p_base, z.shape[1]):])


def test_latent_config_full_compare(cuda_device):
    s = synth.LATENT
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], s["h"], s["w"], s["tx"], s["tc"], s["k"],
                                   device=DEV, seed=synth.SEED_BASE + 1)
    y, co, plan = run(x, c, w, b)
    torch.cuda.synchronize()
    ref = _oracle(x, c, w, b)
    m = assert_bf16_close(y, ref, "latent", strict=True)
    assert m["cos"] > 0.9999
    assert torch.equal(co, torch.cat([c, x], 1)[:, 1:])


@pytest.mark.parametrize("packed", [False, True], ids=["w_in_place", "packed"])
@pytest.mark.parametrize("sig", synth.SINGLE_CALLS[1:], ids=[s["name"] for s in synth.SINGLE_CALLS[1:]])
def test_full_size_signatures_every_output(cuda_device, sig, packed):
    """The mid- and full-resolution configurations at full size, every output
    against the oracle (frame by frame), through causal_conv3d_forward (W
    read in place) and through the packed weight image; the two are equal
    bit for bit (same arithmetic, same order)."""
    s = sig
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], s["h"], s["w"], s["tx"], s["tc"], s["k"],
                                   device=DEV, seed=synth.SEED_BASE + 2 + synth.SINGLE_CALLS.index(s))
    y, co, plan = run(x, c, w, b, k=s["k"], pad=s["pad"], p_base=s["p_base"], packed=packed)
    torch.cuda.synchronize()
    assert torch.equal(co, x[:, 2:4])
    if packed:
        y2, _, _ = run(x, c, w, b, k=s["k"], pad=s["pad"], p_base=s["p_base"], want_cache=False)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
        del y2
        return  # the outputs are those compared below, bit for bit
    m = compare_full(y, x, c, w, b, s["name"], strict=True, padding=s["pad"], pbase=s["p_base"])
    assert m["count"] == y.numel() and m["cos"] > 0.9999


def _replay(sig, frames, seed, device, h=None, w=None, packed=False):
    """Five (or len(frames)) chunks with cache carry through two ping-pong
    cache buffers, NaN-filled before each chunk writes them.  packed: every
    chunk plan runs from one packed image, packed once from the first plan
    (the chunk plans of a signature share the weight layout)."""
    h = sig["h"] if h is None else h
    w = sig["w"] if w is None else w
    wt, bt, xs = synth.replay_chunks(1, sig["cin"], sig["cout"], h, w, frames, sig["k"], device=device, seed=seed)
    outs, cache, image, layout = [], None, None, None
    for xc in xs:
        tc = 0 if cache is None else cache.shape[1]
        plan = plan_for(xc, tc, wt, k=sig["k"], pad=sig["pad"], dt=sig["dt"], p_base=sig["p_base"])
        if packed and image is None:
            image = cc3d.causal_conv3d_pack_weights(plan, wt)
            layout = (plan.info["weight_layout"], plan.info["packed_weight_bytes"])
        if packed:
            assert (plan.info["weight_layout"], plan.info["packed_weight_bytes"]) == layout
        y, cache_next, _ = run(xc, cache, wt, bt, k=sig["k"], pad=sig["pad"], dt=sig["dt"], p_base=sig["p_base"],
                               packed=packed, image=image)
        outs.append(y)
        cache = cache_next
    return wt, bt, xs, outs


@pytest.mark.parametrize("sig", synth.REPLAY_STACK + [synth.REPLAY_DILATED],
                         ids=[s["name"] for s in synth.REPLAY_STACK + [synth.REPLAY_DILATED]])
def test_streaming_replay_reduced_spatial_full_compare(cuda_device, sig):
    """Five chunks with cache carry at a reduced spatial size, every output
    against one oracle call over the whole concatenated sequence."""
    frames = [sig["tx"]] * synth.REPLAY_CHUNKS
    wt, bt, xs, outs = _replay(sig, frames, synth.SEED_BASE + 40, DEV, h=13, w=41)
    torch.cuda.synchronize()
    whole = oracle.conv3d(torch.cat(xs, 1).cpu(), None, wt.cpu(), bt.cpu(), dilation=(sig["dt"], 1, 1),
                          padding=sig["pad"], pbase=sig["p_base"])
    assert_bf16_close(torch.cat(outs, 1), whole, sig["name"])


@pytest.mark.parametrize("sig", synth.REPLAY_STACK + [synth.REPLAY_DILATED],
                         ids=[s["name"] for s in synth.REPLAY_STACK + [synth.REPLAY_DILATED]])
def test_streaming_replay_full_size_every_output(cuda_device, sig):
    """The full-size five-chunk replay, every chunk plan from one packed
    weight image, against one oracle call over the whole concatenated
    sequence: every output of every chunk, frame by frame."""
    frames = [sig["tx"]] * synth.REPLAY_CHUNKS
    wt, bt, xs, outs = _replay(sig, frames, synth.SEED_BASE + 4, DEV, packed=True)
    torch.cuda.synchronize()
    y = torch.cat(outs, 1)
    del outs
    whole_x = torch.cat(xs, 1)
    m = compare_full(y, whole_x, None, wt, bt, sig["name"], strict=True, dilation=(sig["dt"], 1, 1),
                     padding=sig["pad"], pbase=sig["p_base"])
    assert m["count"] == y.numel()


@pytest.mark.parametrize("sig", synth.DECODER_SIGNATURES, ids=[s["name"] for s in synth.DECODER_SIGNATURES])
def test_decoder_signatures_reduced_spatial_full_compare(cuda_device, sig):
    """Every decoder signature at a reduced spatial size (several patches and
    ragged edges) with its steady-state frames and 2-frame cache, through the
    default kernel choice, against the oracle everywhere."""
    s = sig
    i = synth.DECODER_SIGNATURES.index(s)
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], 40, 72, s["tx"], s["tc"], s["k"], device=DEV,
                                   seed=synth.SEED_BASE + 300 + i)
    y, co, plan = run(x, c, w, b, k=s["k"], pad=s["pad"], p_base=s["p_base"])
    torch.cuda.synchronize()
    assert plan.info["kernel_name"].startswith("bf16_")
    ref = _oracle(x, c, w, b, k=s["k"], pad=s["pad"], p_base=s["p_base"])
    assert_bf16_close(y, ref, s["name"] + "/" + plan.info["kernel_name"])
    assert torch.equal(co, torch.cat([c, x], 1)[:, -2:])


@pytest.mark.parametrize("name", ["mid_192", "head_96_3", "temporal_384_768", "conv_in_48_384"])
def test_autotune_returns_the_fastest_runnable_variant(cuda_device, name):
    """causal_conv3d_plan_autotune times every variant that can run the call
    and returns one of them: any variant that plans the call may win (the
    timing decides), and its output from a packed image matches the oracle
    and the default plan's within tolerance."""
    s = next(v for v in synth.DECODER_SIGNATURES if v["name"] == name)
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], 40, 72, s["tx"], s["tc"], s["k"], device=DEV,
                                   seed=synth.SEED_BASE + 320)
    desc = cc3d.make_desc(1, s["cin"], s["cout"], 40, 72, s["tx"], s["tc"], k=s["k"], padding=s["pad"],
                          p_base=s["p_base"])
    runnable = [cc3d.causal_conv3d_plan(desc).info["kernel_name"]]
    for v in cc3d.VARIANTS:
        try:
            cc3d.causal_conv3d_plan_variant(desc, v).close()
            runnable.append(v)
        except cc3d.CC3DError as e:
            assert e.status == cc3d.CC3D_ERR_UNSUPPORTED
    scratch = torch.empty(cc3d.causal_conv3d_plan(desc).shapes()["out"], dtype=torch.bfloat16, device=DEV)
    plan, ms = cc3d.causal_conv3d_plan_autotune(desc, x, c, w, b, scratch, launches=3)
    assert plan.info["kernel_name"] in runnable and ms > 0
    y = nan_like(scratch.shape, torch.bfloat16, DEV)
    cc3d.causal_conv3d_forward_packed(plan, x, c, cc3d.causal_conv3d_pack_weights(plan, w), b, y, None,
                                      workspace_for(plan, DEV))
    y_def, _, _ = run(x, c, w, b, k=s["k"], pad=s["pad"], p_base=s["p_base"])
    torch.cuda.synchronize()
    ref = _oracle(x, c, w, b, k=s["k"], pad=s["pad"], p_base=s["p_base"])
    assert_bf16_close(y, ref, name + "/" + plan.info["kernel_name"])
    assert_bf16_close(y_def, ref, name + "/default")


@pytest.mark.parametrize("name", ["mid_192", "full_96", "head_96_3"])
def test_streaming_17_frame_schedule_full_compare(cuda_device, name):
    """The 1 + 4*4 frame schedule of a 17-frame decode at the 360x640 and
    720x1280 stages (reduced spatial size): the first chunk decodes one frame
    with no cache, each later one four frames with the carried cache; all 17
    output frames against one oracle call over the whole sequence."""
    s = next(v for v in synth.DECODER_SIGNATURES if v["name"] == name)
    wt, bt, xs, outs = _replay(s, synth.SCHEDULE_17, synth.SEED_BASE + 330, DEV, h=21, w=40)
    torch.cuda.synchronize()
    assert sum(o.shape[1] for o in outs) == 17
    whole = oracle.conv3d(torch.cat(xs, 1).cpu(), None, wt.cpu(), bt.cpu(), dilation=(s["dt"], 1, 1),
                          padding=s["pad"], pbase=s["p_base"])
    assert_bf16_close(torch.cat(outs, 1), whole, name)


def test_unread_frames_and_guard_bands_are_never_touched(cuda_device):
    """Frames of Z outside every tap's source interval, and bytes just outside
    each buffer, hold NaN; the output must be finite and bit-identical to the
    run where they hold zeros, and guard bytes around the output must stay."""
    cin, cout, h, w_ = 32, 96, 12, 40
    # d_t = 2 behind a 4-frame cache with one new frame: taps read Z[0], Z[2], Z[4];
    # Z[1] and Z[3] (cache frames 1 and 3) are never read.
    x, c, w, b = synth.conv_inputs(1, cin, cout, h, w_, 1, 4, device=DEV, seed=synth.SEED_BASE + 60)
    guard = 4096
    def embed(t, fill):
        buf = torch.full((t.numel() + 2 * guard,), fill, dtype=t.dtype, device=DEV)
        v = buf[guard:guard + t.numel()].view(t.shape)
        v.copy_(t)
        return buf, v
    results = []
    for fill in (0.0, float("nan")):
        cc = c.clone()
        cc[:, 1] = fill
        cc[:, 3] = fill
        _, xv = embed(x, fill)
        _, cv = embed(cc, fill)
        _, wv = embed(w, fill)
        plan = plan_for(xv, 4, wv, k=(3, 3, 3), pad=(1, 1), dt=2, p_base=4)
        obuf = torch.full((int(np.prod(plan.shapes()["out"])) + 2 * guard,), 7.0, dtype=x.dtype, device=DEV)
        ov = obuf[guard:guard + int(np.prod(plan.shapes()["out"]))].view(plan.shapes()["out"])
        cc3d.causal_conv3d_forward(plan, xv, cv, wv, b, ov, None)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(ov).all())
        assert bool((obuf[:guard] == 7.0).all()) and bool((obuf[-guard:] == 7.0).all())
        results.append(ov.clone())
    assert torch.equal(results[0], results[1])
    ref = _oracle(x, c, w, b, dt=2, p_base=4)
    assert_bf16_close(results[0], ref, "poisoned")


@pytest.mark.parametrize("cout,variant,tiles,sst", [(96, "bf16_s3_n96_p16x32_g32", 640, (1, 1)),
                                                    (128, "bf16_s3_n64_p24x32_g32", 880, (1, 1)),
                                                    (96, "bf16_s3s2_n96_p4x32_g32", 640, (2, 2))])
def test_group_staged_schedule_writes_every_tile_across_launches(cuda_device, cout, variant, tiles, sst):
    """640 (880) tiles on at most 256 workgroups: two fixed tiles each, the
    rest claimed from per-XCD counters (and stolen across XCDs).  Every
    launch takes the next slot of the counter table, and the kernel leaves
    its slot zeroed.  The output is poisoned with NaN before each of 130
    launches: every tile must be written every time, bitwise equal to the
    first launch, which is compared with the oracle everywhere.  (The
    strided kernel's 4x32 tiles of the half-size map come to 640 as well.)"""
    x, c, w, b = synth.conv_inputs(1, 32, cout, 256, 320, 4, 2, device=DEV, seed=synth.SEED_BASE + 90)
    plan = plan_for(x, 2, w, k=(3, 3, 3), pad=(1, 1), variant=variant, sst=sst)
    assert plan.info["tiles"] == tiles
    img = cc3d.causal_conv3d_pack_weights(plan, w)
    first = nan_like(plan.shapes()["out"], torch.bfloat16, DEV)
    cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, first, None)
    y = torch.empty_like(first)
    bad = []
    for i in range(130):
        y.fill_(float("nan"))
        cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, y, None)
        if not torch.equal(y, first):
            bad.append(i)
    torch.cuda.synchronize()
    assert not bad, "launches with unwritten or different tiles: %s" % bad[:10]
    assert_bf16_close(first, _oracle(x, c, w, b, sst=sst), "dynamic schedule")


def test_repeated_runs_are_bitwise_identical(cuda_device):
    s = synth.MID_192
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], 64, 128, 4, 2, device=DEV, seed=synth.SEED_BASE + 70)
    y1, _, _ = run(x, c, w, b)
    y2, _, _ = run(x, c, w, b)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("cin,cout,variant", [
    (16, 192, None),
    (32, 96, "bf16_s3_n96_p16x32_g32"),
    (32, 64, "bf16_s3_n64_p24x32_g32"),
    (16, 32, "bf16_s3_n32_p8x32"),
    (32, 3, "bf16_s3_few_p16x128"),
])
def test_epilogue_rounds_to_nearest_even(cuda_device, cin, cout, variant):
    """With a single unit source value the fp32 sum is exactly w + b, so the
    bf16 output must equal that exact value rounded to nearest even (every
    bf16 kernel's epilogue)."""
    h, w_ = 8, 32
    g = torch.Generator(device=DEV).manual_seed(5)
    w = torch.randn((cout, 3, 3, 3, cin), generator=g, device=DEV).to(torch.bfloat16)
    b = (torch.randn((cout,), generator=g, device=DEV) * 3).to(torch.bfloat16)
    x = torch.zeros((1, 1, h, w_, cin), dtype=torch.bfloat16, device=DEV)
    c = torch.zeros((1, 2, h, w_, cin), dtype=torch.bfloat16, device=DEV)
    c[0, 1, 3, 5, 7] = 1.0
    y, _, plan = run(x, c, w, b, variant=variant)
    torch.cuda.synchronize()
    if variant is not None:
        assert plan.info["kernel_name"] == variant
    ref = _oracle(x, c, w, b)
    ref_bf16 = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)  # exact in fp32
    assert torch.equal(y.cpu().view(torch.int16), ref_bf16.view(torch.int16))


def test_counters_count_fast_path(cuda_device):
    x, c, w, b = synth.conv_inputs(1, 16, 32, 8, 32, 2, 2, device=DEV, seed=1)
    cc3d.causal_conv3d_counters(reset=True)
    for _ in range(3):
        run(x, c, w, b)
    torch.cuda.synchronize()
    cnt = cc3d.causal_conv3d_counters()
    assert cnt["fast_path"] == 3 and cnt["device_error"] == 0 and cnt["invalid"] == 0


def test_packed_weights_path_matches_forward_bitwise(cuda_device):
    """causal_conv3d_forward (W gathered in place) and
    causal_conv3d_forward_packed give the same bits: the same LDS weight
    layout feeds the same MFMA sequence.  The image packed from one plan
    serves another plan of the same weight layout (a different frame count
    and cache depth), and an image of the wrong size is refused."""
    # (enough tiles that the packed call does not split its K stages)
    x, c, w, b = synth.conv_inputs(1, 48, 96, 136, 512, 2, 2, device=DEV, seed=synth.SEED_BASE + 80)
    plan = plan_for(x, 2, w, k=(3, 3, 3), pad=(1, 1))
    assert plan.info["splits"] == 1
    y1, _, _ = run(x, c, w, b)
    x0 = synth.conv_inputs(1, 48, 96, 136, 512, 4, 0, device=DEV, seed=synth.SEED_BASE + 81)[0]
    other = plan_for(x0, 0, w, k=(3, 3, 3), pad=(1, 1))
    assert other.info["weight_layout"] == plan.info["weight_layout"]
    img = cc3d.causal_conv3d_pack_weights(other, w)
    y2 = nan_like(plan.shapes()["out"], x.dtype, DEV)
    cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, y2, None)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert_bf16_close(y2, _oracle(x, c, w, b), "packed")
    with pytest.raises(ValueError):
        cc3d.causal_conv3d_forward_packed(plan, x, c, img[:16], b, y2, None)


def _u8_compare(got_u8, y_ref, what, margin=0.01):
    """8-bit pixel codes against the oracle's: equal wherever the oracle's
    pre-truncation value (y*0.5 + 0.5)*255 is farther than ``margin`` from
    an integer (the fp32 sum and the fp64 one differ by far less); within
    that band the code may be either neighbour."""
    got = np.asarray(got_u8).astype(np.int64)
    ref = oracle.pixels_u8(y_ref).astype(np.int64)
    p = np.clip((np.asarray(y_ref, dtype=np.float64) * 0.5 + 0.5) * 255, 0, 255)
    near = np.abs(p - np.round(p)) < margin
    far_bad = (got != ref) & ~near
    assert not far_bad.any(), (what, int(far_bad.sum()), got[far_bad][:8], ref[far_bad][:8])
    assert np.all(np.abs(got - ref)[near] <= 1), what
    return int((got != ref).sum())


def _u8_twice(plan, x, c, w, b, co=None):
    """Two u8 launches into buffers pre-filled with 0x00 and 0xFF: a byte the
    kernel never writes keeps its fill, so the two must be equal."""
    o0 = torch.zeros(plan.shapes()["out"], dtype=torch.uint8, device=DEV)
    o1 = torch.full(plan.shapes()["out"], 255, dtype=torch.uint8, device=DEV)
    cc3d.causal_conv3d_forward_u8(plan, x, c, w, b, o0, co)
    cc3d.causal_conv3d_forward_u8(plan, x, c, w, b, o1, None)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1), "bytes left unwritten"
    return o0


def test_head_u8_codes_match_oracle(cuda_device):
    """The RGB head with the pixel quantisation fused: every code against the
    oracle's quantisation of its fp64 output; codes span the clamps; the
    cache carry is that of the plain forward."""
    s = synth.HEAD_96_3
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], 40, 72, s["tx"], s["tc"], device=DEV,
                                   seed=synth.SEED_BASE + 340)
    plan = plan_for(x, s["tc"], w, k=(3, 3, 3), pad=(1, 1))
    assert plan.info["kernel_name"].startswith("bf16_s3_few_")
    co = nan_like(plan.shapes()["cache_out"], x.dtype, DEV)
    out = _u8_twice(plan, x, c, w, b, co)
    ref = _oracle(x, c, w, b)
    _u8_compare(out.cpu().numpy(), ref, "head u8")
    got = out.cpu().numpy()
    assert got.min() == 0 and got.max() == 255
    assert torch.equal(co, torch.cat([c, x], 1)[:, -2:])


def test_head_u8_full_size_every_code(cuda_device):
    """At 720x1280: every code against the oracle, frame by frame; bias-only
    frames (p_base = 4) go through the same quantisation."""
    s = synth.HEAD_96_3
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], s["h"], s["w"], s["tx"], s["tc"], device=DEV,
                                   seed=synth.SEED_BASE + 341)
    plan = plan_for(x, s["tc"], w, k=(3, 3, 3), pad=(1, 1))
    out = _u8_twice(plan, x, c, w, b)
    xc, cc, wc, bc = x.cpu(), c.cpu(), w.cpu(), b.cpu()
    i = plan.info
    for o in range(i["t_out"]):
        ref = oracle.conv3d(xc, cc, wc, bc, points=frame_points(0, o, i["h_out"], i["w_out"]))
        _u8_compare(out[0, o].reshape(-1, 3).cpu().numpy(), ref, "head u8 full size frame %d" % o)
    # bias-only leading frames
    x2, _, w2, b2 = synth.conv_inputs(1, 64, 3, 18, 40, 2, 0, device=DEV, seed=synth.SEED_BASE + 342)
    p2 = plan_for(x2, 0, w2, k=(3, 3, 3), pad=(1, 1), p_base=4)
    assert p2.info["kernel_name"].startswith("bf16_s3_few_") and p2.info["t_out"] == 4
    o2 = _u8_twice(p2, x2, None, w2, b2)
    _u8_compare(o2.cpu().numpy(), _oracle(x2, None, w2, b2, p_base=4), "head u8 bias-only frames")


def test_u8_output_refused_off_the_head_kernel(cuda_device):
    x, c, w, b = synth.conv_inputs(1, 32, 96, 16, 32, 2, 2, device=DEV, seed=synth.SEED_BASE + 343)
    plan = plan_for(x, 2, w, k=(3, 3, 3), pad=(1, 1))
    out = torch.zeros(plan.shapes()["out"], dtype=torch.uint8, device=DEV)
    with pytest.raises(cc3d.CC3DError) as e:
        cc3d.causal_conv3d_forward_u8(plan, x, c, w, b, out, None)
    assert e.value.status == cc3d.CC3D_ERR_UNSUPPORTED


# Temporal stride (the encoder's downsampling convs): (C_in, C_out, H, W,
# T_x, T_cache, k, s_t, variant) on every kernel that runs it.
STRIDED = [
    (32, 96, 20, 70, 4, 2, (3, 3, 3), 2, "bf16_s3_n96_p16x32_g32"),
    (32, 128, 30, 70, 4, 2, (3, 3, 3), 2, "bf16_s3_n64_p24x32_g32"),
    (64, 192, 17, 45, 6, 2, (3, 3, 3), 2, "bf16_s3_n96_p8x32_x2"),
    (32, 40, 13, 41, 5, 0, (3, 3, 3), 2, "bf16_s3_n32_p8x32"),       # chunk 0: odd length, no cache
    (64, 192, 16, 40, 4, 2, (3, 1, 1), 2, "bf16_s1_n192_p8x32"),
    (128, 192, 16, 40, 4, 2, (3, 1, 1), 2, "bf16_s1_n192_p256_rd"),
    (48, 40, 9, 33, 6, 2, (3, 1, 1), 3, "bf16_s1_n32_p8x32"),
    (96, 3, 16, 32, 4, 2, (3, 3, 3), 2, "bf16_s3_n32_p8x32"),         # head shape: not the few kernel
]


@pytest.mark.parametrize("case", STRIDED)
def test_temporal_stride_full_compare(cuda_device, case):
    cin, cout, h, w_, tx, tc, k, st, variant = case
    pad = (1, 1) if k[1] == 3 else (0, 0)
    x, c, w, b = synth.conv_inputs(1, cin, cout, h, w_, tx, tc, k, device=DEV, seed=synth.SEED_BASE + 350 + h)
    y, co, plan = run(x, c, w, b, k=k, pad=pad, st=st, variant=variant)
    torch.cuda.synchronize()
    assert plan.info["kernel_name"] == variant
    ref = _oracle(x, c, w, b, k=k, pad=pad, st=st)
    assert_bf16_close(y, ref, variant)
    z = x if c is None else torch.cat([c, x], 1)
    assert torch.equal(co, z[:, -min(2, z.shape[1]):])


def test_temporal_stride_fp32_direct(cuda_device):
    x, c, w, b = synth.conv_inputs(1, 8, 8, 16, 16, 4, 2, kind="uniform", dtype=torch.float32, device=DEV,
                                   seed=synth.SEED_BASE + 360)
    y, _, plan = run(x, c, w, b, st=2)
    torch.cuda.synchronize()
    assert plan.info["kernel_name"] == "f32_direct" and plan.info["t_out"] == 2  # floor((6 - 3) / 2) + 1
    assert_f32_close(y, _oracle(x, c, w, b, st=2), "f32 s_t=2")


@pytest.mark.parametrize("k", [(3, 3, 3), (3, 1, 1)])
def test_temporal_stride_streaming_equals_one_shot(cuda_device, k):
    """Stride-2 streaming with chunks of even length and the 2-frame carry:
    every output against one oracle call over the whole sequence."""
    cin, cout = (64, 96) if k[1] == 3 else (64, 192)
    pad = (1, 1) if k[1] == 3 else (0, 0)
    wt, bt, xs = synth.replay_chunks(1, cin, cout, 21, 40, [2, 4, 4, 6], k, device=DEV, seed=synth.SEED_BASE + 361)
    outs, cache = [], None
    for xc in xs:
        y, cache, _ = run(xc, cache, wt, bt, k=k, pad=pad, st=2)
        outs.append(y)
    torch.cuda.synchronize()
    whole = oracle.conv3d(torch.cat(xs, 1).cpu(), None, wt.cpu(), bt.cpu(), stride=(2, 1, 1), padding=pad, pbase=2)
    got = torch.cat(outs, 1)
    assert got.shape[1] == 8
    assert_bf16_close(got, whole, "stride-2 streaming %s" % (k,))


@pytest.mark.parametrize("sig", synth.ENCODER_DOWNSAMPLE, ids=[s["name"] for s in synth.ENCODER_DOWNSAMPLE])
def test_encoder_downsample_full_size_every_output(cuda_device, sig):
    """The encoder's stride-2 temporal downsampling convs at full size, every
    output against the oracle."""
    s = sig
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], s["h"], s["w"], s["tx"], s["tc"], s["k"], device=DEV,
                                   seed=synth.SEED_BASE + 370)
    y, co, plan = run(x, c, w, b, k=s["k"], pad=s["pad"], p_base=s["p_base"], st=s["st"])
    torch.cuda.synchronize()
    assert plan.info["kernel_name"].startswith("bf16_") and plan.info["t_out"] == s["tx"] // s["st"]
    assert torch.equal(co, x[:, -2:])
    compare_full(y, x, c, w, b, s["name"], stride=(s["st"], 1, 1), padding=s["pad"], pbase=s["p_base"])


# General spatial parameters on the gather kernel: (C_in, C_out, H, W, T_x,
# T_cache, k, pad, spatial stride, spatial dilation, s_t, d_t, p_base, N, bias)
GENERAL = [
    (32, 40, 20, 36, 4, 2, (3, 5, 5), (2, 2), (1, 1), (1, 1), 1, 1, 2, 1, True),   # 5x5 "same"
    (32, 96, 21, 37, 4, 2, (3, 3, 3), (1, 1), (2, 2), (1, 1), 1, 1, 2, 1, True),   # spatial stride 2
    (48, 40, 16, 40, 3, 2, (3, 3, 3), (2, 2), (1, 1), (2, 2), 1, 1, 2, 1, True),   # spatial dilation 2
    (64, 64, 15, 33, 2, 2, (3, 1, 3), (0, 1), (1, 1), (1, 1), 1, 1, 2, 1, True),   # 1x3
    (32, 70, 24, 50, 4, 2, (3, 3, 3), (0, 0), (1, 1), (1, 1), 1, 1, 2, 1, True),   # "valid", ragged C_out
    (32, 96, 18, 34, 4, 2, (3, 3, 3), (1, 1), (2, 2), (1, 1), 2, 1, 2, 1, True),   # stride 2 in t, h, w
    (32, 40, 12, 20, 2, 2, (3, 3, 3), (1, 1), (2, 1), (1, 1), 1, 1, 2, 2, True),   # batch 2, stride (2, 1)
    (16, 32, 14, 30, 4, 4, (3, 3, 3), (2, 1), (1, 1), (2, 1), 1, 2, 4, 1, False),  # d_t 2, d_h 2, no bias
    (48, 33, 9, 70, 1, 0, (3, 3, 3), (1, 1), (1, 2), (1, 1), 1, 1, 2, 1, True),    # one frame, no cache
    (32, 192, 17, 35, 2, 2, (3, 3, 3), (1, 1), (2, 2), (1, 1), 1, 1, 2, 1, True),  # stride 2, two 96-wide blocks
    (64, 192, 13, 40, 3, 1, (3, 3, 3), (2, 2), (1, 1), (2, 2), 1, 1, 2, 1, False), # dilation 2, no bias
]


def _gen_name(cout, cin=32, k=(3, 3, 3), pad=(1, 1), sst=(1, 1), sdil=(1, 1)):
    """The default kernel of a call outside the 3x3 / 1x1 "same" envelope."""
    if (k[1:] == (3, 3) and sst == (1, 1) and sdil == (2, 2) and tuple(pad) == (2, 2) and cout % 64 == 0
            and cin % 32 == 0):
        return "bf16_s3d2_n64_p16x32_g32"
    if (k[1:] == (3, 3) and sst == (2, 2) and sdil == (1, 1) and tuple(pad) == (1, 1) and cout % 96 == 0
            and cin % 32 == 0):
        return "bf16_s3s2_n96_p4x32_g32"
    if (k[1:] == (3, 3) and sst == (2, 2) and sdil == (1, 1) and tuple(pad) == (1, 1) and cout % 64 == 0
            and cin % 32 == 0):
        return "bf16_s3s2_n64_p4x32_g32"
    return "bf16_gen_n96_p8x32" if cout % 96 == 0 else "bf16_gen_n64_p8x32"


@pytest.mark.parametrize("case", GENERAL)
def test_general_spatial_parameters_full_compare(cuda_device, case):
    cin, cout, h, w_, tx, tc, k, pad, sst, sdil, st, dt, p_base, n, bias = case
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV, seed=synth.SEED_BASE + 380 + h,
                                   has_bias=bias)
    y, co, plan = run(x, c, w, b, k=k, pad=pad, dt=dt, p_base=p_base, st=st, sst=sst, sdil=sdil)
    torch.cuda.synchronize()
    assert plan.info["kernel_name"] == _gen_name(cout, cin, k, pad, sst, sdil)
    ref = _oracle(x, c, w, b, k=k, pad=pad, dt=dt, p_base=p_base, st=st, sst=sst, sdil=sdil)
    assert_bf16_close(y, ref, "general %s" % (case,))
    z = x if c is None else torch.cat([c, x], 1)
    assert torch.equal(co, z[:, z.shape[1] - min(p_base, z.shape[1]):])


# The group-staged kernel at spatial dilation 2 ("same": padding 2): (C_in,
# C_out, H, W, T_x, T_cache, k, d_t, p_base, N, bias), full compare.
DILATED = [
    (32, 64, 20, 70, 2, 2, (3, 3, 3), 1, 2, 1, True),    # ragged rows and columns, halo reaching 2 past
    (64, 128, 17, 45, 3, 2, (3, 3, 3), 1, 2, 1, True),   # 2 channel groups, 2 channel blocks, 1-row tail
    (96, 192, 33, 64, 4, 2, (3, 3, 3), 1, 2, 1, False),  # 3 groups, 3 blocks, no bias
    (32, 64, 16, 32, 1, 0, (3, 3, 3), 1, 2, 2, True),    # batch 2, one active tap
    (32, 64, 18, 40, 4, 2, (3, 3, 3), 2, 4, 1, True),    # temporal dilation 2 as well
    (32, 64, 16, 40, 3, 1, (2, 3, 3), 1, 1, 1, True),    # k_t = 2
    (64, 64, 16, 33, 2, 0, (3, 3, 3), 1, 4, 1, True),    # bias-only output frames
    (32, 64, 3, 5, 2, 2, (3, 3, 3), 1, 2, 1, True),      # map smaller than the dilated window
]


@pytest.mark.parametrize("case", DILATED, ids=[str(i) for i in range(len(DILATED))])
def test_dilated_group_staged_full_compare(cuda_device, case):
    cin, cout, h, w_, tx, tc, k, dt, p_base, n, bias = case
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV,
                                   seed=synth.SEED_BASE + 420 + DILATED.index(case), has_bias=bias)
    y, co, plan = run(x, c, w, b, k=k, pad=(2, 2), dt=dt, p_base=p_base, sdil=(2, 2))
    torch.cuda.synchronize()
    assert plan.info["kernel_name"] == "bf16_s3d2_n64_p16x32_g32"
    ref = _oracle(x, c, w, b, k=k, pad=(2, 2), dt=dt, p_base=p_base, sdil=(2, 2))
    assert tuple(y.shape) == ref.shape
    assert_bf16_close(y, ref, "dilated %s" % (case,))
    z = x if c is None else torch.cat([c, x], 1)
    assert torch.equal(co, z[:, z.shape[1] - min(p_base, z.shape[1]):])


# The group-staged kernel at spatial stride 2 (3x3, padding 1): (C_in, C_out,
# H, W, T_x, T_cache, k, d_t, s_t, p_base, N, bias), full compare.  Output
# tiles are 4 rows x 32 columns of the half-size map.
STRIDED_3X3 = [
    (32, 96, 21, 37, 2, 2, (3, 3, 3), 1, 1, 2, 1, True),    # odd sizes: ragged rows and columns
    (64, 192, 17, 70, 3, 2, (3, 3, 3), 1, 1, 2, 1, True),   # 2 channel groups, 2 channel blocks
    (96, 96, 33, 130, 2, 2, (3, 3, 3), 1, 1, 2, 1, False),  # 3 groups, 1-row and 1-column tails, no bias
    (32, 96, 16, 64, 1, 0, (3, 3, 3), 1, 1, 2, 2, True),    # exact tiles, batch 2, one active tap
    (32, 192, 18, 40, 4, 2, (3, 3, 3), 2, 1, 4, 1, True),   # temporal dilation 2
    (32, 96, 14, 44, 4, 2, (3, 3, 3), 1, 2, 2, 1, True),    # temporal stride 2
    (32, 96, 16, 40, 3, 1, (2, 3, 3), 1, 1, 1, 1, True),    # k_t = 2
    (64, 96, 16, 33, 2, 0, (3, 3, 3), 1, 1, 4, 1, True),    # bias-only output frames
    (32, 96, 3, 5, 2, 2, (3, 3, 3), 1, 1, 2, 1, True),      # map smaller than one tile
    (32, 96, 1, 1, 2, 2, (3, 3, 3), 1, 1, 2, 1, True),      # a single pixel
    (64, 128, 19, 70, 2, 2, (3, 3, 3), 1, 1, 2, 1, True),   # 64-wide tile: 2 blocks, ragged
    (32, 64, 16, 64, 3, 1, (3, 3, 3), 2, 1, 3, 2, False),   # 64-wide tile: batch 2, d_t 2, no bias
]


@pytest.mark.parametrize("case", STRIDED_3X3, ids=[str(i) for i in range(len(STRIDED_3X3))])
def test_strided_group_staged_full_compare(cuda_device, case):
    cin, cout, h, w_, tx, tc, k, dt, st, p_base, n, bias = case
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV,
                                   seed=synth.SEED_BASE + 440 + STRIDED_3X3.index(case), has_bias=bias)
    y, co, plan = run(x, c, w, b, k=k, dt=dt, st=st, p_base=p_base, sst=(2, 2))
    torch.cuda.synchronize()
    assert plan.info["kernel_name"] == ("bf16_s3s2_n96_p4x32_g32" if cout % 96 == 0 else "bf16_s3s2_n64_p4x32_g32")
    ref = _oracle(x, c, w, b, k=k, dt=dt, st=st, p_base=p_base, sst=(2, 2))
    assert tuple(y.shape) == ref.shape
    assert_bf16_close(y, ref, "strided %s" % (case,))
    z = x if c is None else torch.cat([c, x], 1)
    assert torch.equal(co, z[:, z.shape[1] - min(p_base, z.shape[1]):])


@pytest.mark.parametrize("case,variant", [(STRIDED_3X3[i], v) for i in range(3)
                                          for v in ["bf16_gen_n64_p8x32", "bf16_gen_n96_p8x32"]] +
                         [(STRIDED_3X3[1], "bf16_s3s2_n64_p4x32_g32")],
                         ids=["%d-%s" % (i, v) for i in range(3) for v in ["gen64", "gen96"]] + ["1-s3s2_n64"])
def test_gather_kernel_on_strided_convs_full_compare(cuda_device, case, variant):
    """The gather kernel, and the 64-wide strided tile, pinned on stride-2
    shapes whose default is the 96-wide strided tile, against the oracle."""
    cin, cout, h, w_, tx, tc, k, dt, st, p_base, n, bias = case
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV,
                                   seed=synth.SEED_BASE + 440 + STRIDED_3X3.index(case), has_bias=bias)
    y, _, plan = run(x, c, w, b, k=k, dt=dt, st=st, p_base=p_base, sst=(2, 2), variant=variant)
    torch.cuda.synchronize()
    assert plan.info["kernel_name"] == variant
    assert_bf16_close(y, _oracle(x, c, w, b, k=k, dt=dt, st=st, p_base=p_base, sst=(2, 2)), "gather strided")


@pytest.mark.parametrize("variant", ["bf16_gen_n64_p8x32", "bf16_gen_n96_p8x32"])
@pytest.mark.parametrize("case", GROUP_STAGED[:4])
def test_gather_kernel_on_same_convs_full_compare(cuda_device, case, variant):
    """The gather kernel (both tile widths) pinned on the 3x3 "same" shapes
    the halo-staged kernels run, against the oracle."""
    cin, cout, h, w_, tx, tc, k, dt, p_base, n, bias = case
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV, seed=synth.SEED_BASE + 390 + h,
                                   has_bias=bias)
    y, _, plan = run(x, c, w, b, k=k, dt=dt, p_base=p_base, variant=variant)
    torch.cuda.synchronize()
    assert_bf16_close(y, _oracle(x, c, w, b, k=k, dt=dt, p_base=p_base), "gather kernel")


@pytest.mark.parametrize("sig", synth.GENERAL_SPATIAL, ids=[s["name"] for s in synth.GENERAL_SPATIAL])
def test_general_spatial_full_size_every_output(cuda_device, sig):
    s = sig
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], s["h"], s["w"], s["tx"], s["tc"], s["k"], device=DEV,
                                   seed=synth.SEED_BASE + 395)
    y, _, plan = run(x, c, w, b, k=s["k"], pad=s["pad"], p_base=s["p_base"], sst=s["sst"], sdil=s["sdil"])
    torch.cuda.synchronize()
    assert plan.info["kernel_name"] == _gen_name(s["cout"], s["cin"], s["k"], s["pad"], s["sst"], s["sdil"])
    compare_full(y, x, c, w, b, s["name"], stride=(1,) + tuple(s["sst"]), dilation=(1,) + tuple(s["sdil"]),
                 padding=s["pad"], pbase=s["p_base"])


@pytest.mark.parametrize("cout,h,variant", [(96, 512, "bf16_s3_n96_p16x32_g32"), (64, 768, "bf16_s3_n64_p24x32_g32")])
def test_group_staged_schedule_with_single_group_tiles(cuda_device, cout, h, variant):
    """Tiles of a single group (C_in = 32, one active tap: the first chunk of
    a stream with no cache) with about three tiles per workgroup: the load
    cursor steps past a whole tile within one group, to a tile claimed in
    that same group."""
    x, _, w, b = synth.conv_inputs(1, 32, cout, h, 800, 1, 0, device=DEV, seed=synth.SEED_BASE + 96)
    y, _, plan = run(x, None, w, b, variant=variant)
    torch.cuda.synchronize()
    assert plan.info["tiles"] == 800 and plan.info["taps"][2]["active"] and not plan.info["taps"][0]["active"]
    assert_bf16_close(y, _oracle(x, None, w, b), "single-group tiles")


@pytest.mark.parametrize("cin,cout,variant", [(32, 96, "bf16_s3_n96_p16x32_g32"), (32, 96, "bf16_s3_n96_p8x32_x2"),
                                               (32, 64, "bf16_s3_n64_p24x32_g32"), (96, 3, "bf16_s3_few_p16x128"),
                                               (32, 96, "bf16_s3s2_n96_p4x32_g32")])
def test_graph_replays_match_eager(cuda_device, cin, cout, variant):
    """The packed-image forward (with its cache-out) captured in a HIP graph:
    the group-staged kernel's tile counters are cleared by the kernel itself
    (no memset nodes), and every replay reuses the captured counter slot; the
    head kernel writes the cache-out itself.  Several replays, each into a
    NaN-poisoned output with eager work and synchronisations between them,
    all equal the eager call bitwise."""
    x, c, w, b = synth.conv_inputs(1, cin, cout, 256, 320, 4, 2, device=DEV, seed=synth.SEED_BASE + 97)
    sst = (2, 2) if "s3s2" in variant else (1, 1)
    plan = plan_for(x, 2, w, k=(3, 3, 3), pad=(1, 1), variant=variant, sst=sst)
    img = cc3d.causal_conv3d_pack_weights(plan, w)
    ref = nan_like(plan.shapes()["out"], torch.bfloat16, DEV)
    cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, ref, None)
    out = torch.empty_like(ref)
    co = torch.empty(plan.shapes()["cache_out"], dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, out, co)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, out, co)
    other = torch.empty_like(ref)
    for i in range(5):
        out.fill_(float("nan"))
        co.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d" % i
        assert torch.equal(co, x[:, -2:]), "replay %d cache" % i
        other.fill_(float("nan"))
        cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, other, None)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, ref)


@pytest.mark.parametrize("packed", [False, True], ids=["w_in_place", "packed"])
@pytest.mark.parametrize("cin,cout,variant", [(32, 96, "bf16_s3_n96_p16x32_g32"), (32, 64, "bf16_s3_n64_p24x32_g32"),
                                               (64, 96, "bf16_s3_n96_p8x32_x2"), (96, 3, "bf16_s3_few_p16x128"),
                                               (64, 192, "bf16_s1_n192_p8x32"),
                                               (128, 192, "bf16_s1_n192_p256_rd")])
def test_first_forward_of_a_fresh_plan_captured_in_a_graph(cuda_device, cin, cout, variant, packed):
    """A plan is host metadata only and the forward calls allocate, set and
    synchronise nothing, so the very first call of a fresh plan can be
    recorded in a graph: its replays (NaN-poisoned outputs before each)
    equal the eager call of another fresh plan bit for bit, cache-out
    included."""
    k = (3, 1, 1) if "s1_" in variant else (3, 3, 3)
    pad = (0, 0) if "s1_" in variant else (1, 1)
    x, c, w, b = synth.conv_inputs(1, cin, cout, 96, 160, 4, 2, k, device=DEV, seed=synth.SEED_BASE + 99)
    eager_plan = plan_for(x, 2, w, k=k, pad=pad, variant=variant)
    img = cc3d.causal_conv3d_pack_weights(eager_plan, w) if packed else None
    ws = workspace_for(eager_plan, DEV) if packed else None  # (a split call, where the plan splits)
    ref, ref_co, _ = run(x, c, w, b, k=k, pad=pad, variant=variant, packed=packed, image=img)
    torch.cuda.synchronize()
    plan = plan_for(x, 2, w, k=k, pad=pad, variant=variant)  # fresh: never run
    out = torch.empty_like(ref)
    co = torch.empty_like(ref_co)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        if packed:
            cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, out, co, ws)
        else:
            cc3d.causal_conv3d_forward(plan, x, c, w, b, out, co)
    for i in range(4):
        out.fill_(float("nan"))
        co.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d" % i
        assert torch.equal(co, ref_co), "replay %d cache" % i


@pytest.mark.parametrize("cout,variant", [(96, "bf16_s3_n96_p16x32_g32"), (128, "bf16_s3_n64_p24x32_g32")])
def test_packed_forwards_of_one_plan_overlap_on_two_streams(cuda_device, cout, variant):
    """Launches of one plan on two streams may run at the same time: each
    takes its own slot of the group-staged kernel's tile counters.  Twelve
    interleaved launches, no synchronisation between them; every output is
    the eager one bitwise."""
    x, c, w, b = synth.conv_inputs(1, 32, cout, 256, 320, 4, 2, device=DEV, seed=synth.SEED_BASE + 98)
    plan = plan_for(x, 2, w, k=(3, 3, 3), pad=(1, 1), variant=variant)
    img = cc3d.causal_conv3d_pack_weights(plan, w)
    ref = nan_like(plan.shapes()["out"], torch.bfloat16, DEV)
    cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, ref, None)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full_like(ref, float("nan")) for _ in range(12)]
    torch.cuda.synchronize()  # the NaN fills (current stream) before the side-stream launches
    for i, o in enumerate(outs):
        cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, o, None, stream=streams[i % 2])
    torch.cuda.synchronize()
    assert all(torch.equal(o, ref) for o in outs)


# The two-workgroup / LDS-staged kernels when a workgroup's tiles alternate
# between output frames no tap reaches (bias only, no K stage) and frames
# with stages: the load cursor runs ahead across tile boundaries, so a
# bias-only tile must stage its outputs through the one LDS buffer the next
# tile's prefetched stages leave free.  (variant, n, C_in, C_out, k, H, W,
# T_x, T_cache, d_t, p_base, bias); T_out is 6 or 7, so the per-XCD tile
# stride (32 or 64 workgroups) moves a workgroup from a bias-only frame to
# a frame with stages.
EMPTY_THEN_STAGED = [
    ("bf16_s1_n32_p8x32", 3, 64, 192, (3, 1, 1), 11, 69, 5, 0, 2, 5, False),   # d_t = 2: frame 0 bias only
    ("bf16_s1_n32_p8x32", 1, 64, 64, (3, 1, 1), 40, 320, 4, 0, 1, 5, True),
    ("bf16_s1_n192_p8x32", 1, 64, 192, (3, 1, 1), 64, 320, 4, 0, 1, 5, True),
    ("bf16_s3_n32_p8x32", 1, 32, 64, (3, 3, 3), 64, 288, 4, 0, 1, 5, True),
    ("bf16_s3_n96_p8x32_x2", 1, 32, 96, (3, 3, 3), 96, 416, 4, 0, 1, 5, True),
]


def _empty_then_staged(tiles, to, staged, grid):
    """Whether, under the persistent schedule (workgroup b on XCD b % 8; each
    XCD walks its contiguous tile range with a stride of its workgroup
    count; output frame = tile % T_out), some workgroup runs a tile without
    stages and then one with stages."""
    per, rem = divmod(tiles, 8)
    for xcd in range(8):
        nblk = grid // 8 + (1 if xcd < grid % 8 else 0)
        beg = xcd * per + min(xcd, rem)
        end = beg + per + (1 if xcd < rem else 0)
        for t in range(beg, min(beg + nblk, end)):
            if not staged[t % to] and t + nblk < end and any(staged[u % to] for u in range(t + nblk, end, nblk)):
                return True
    return False


@pytest.mark.parametrize("case", EMPTY_THEN_STAGED, ids=["%s_%d" % (c[0], i) for i, c in enumerate(EMPTY_THEN_STAGED)])
def test_bias_only_tiles_before_staged_tiles(cuda_device, case):
    v, n, cin, cout, k, h, w_, tx, tc, dt, p_base, bias = case
    pad = (0, 0) if k[1] == 1 else (1, 1)
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV, has_bias=bias,
                                   seed=synth.SEED_BASE + 680 + EMPTY_THEN_STAGED.index(case))
    y, co, plan = run(x, c, w, b, k=k, pad=pad, dt=dt, p_base=p_base, variant=v)
    yp, _, _ = run(x, c, w, b, k=k, pad=pad, dt=dt, p_base=p_base, variant=v, packed=True, want_cache=False)
    torch.cuda.synchronize()
    i = plan.info
    assert i["kernel_name"] == v and i["splits"] == 1
    to = i["t_out"]
    staged = [any(0 <= o + tp * dt - i["p_l"] < i["t_z"] for tp in range(k[0])) for o in range(to)]
    assert not all(staged) and any(staged)
    # the case walks a bias-only tile into a staged one at one and at two
    # workgroups per compute unit
    assert all(_empty_then_staged(i["tiles"], to, staged, min(i["tiles"], 256 * occ)) for occ in (1, 2))
    assert torch.equal(y, yp)
    ref = _oracle(x, c, w, b, k=k, pad=pad, dt=dt, p_base=p_base)
    mask = mask_for(plan, x.shape, k=k, pad=pad, dt=dt)
    assert_bias_only_exact(y, b, mask, v)
    assert_bf16_close(y, ref, v, exclude=mask)


# The register-direct 1x1 kernel: (n, C_in, C_out, H, W, T_x, T_cache, k_t,
# d_t, p_base, bias).  Its stage depth follows C_in / 64 (3 for 3, 6 and 12
# chunks, 4 for 4 and 8, 2 for 2); frames of any pixel count (the last tile
# ragged, or a single partial tile); more tiles than workgroups (each runs
# several, prefetching across tile boundaries); leading output frames with
# no active tap (bias only); k_t = 1, 2 and temporal dilation 2.
RD_CASES = [
    (1, 384, 768, 20, 36, 1, 2, 3, 1, 2, True),     # the decoder's temporal conv, small map
    (1, 128, 192, 100, 192, 4, 2, 3, 1, 2, True),   # 75 pixel tiles x 4 frames = 300 tiles
    (2, 128, 192, 17, 23, 3, 0, 3, 1, 2, True),     # two items, first chunk, 391 pixels
    (1, 256, 384, 9, 13, 2, 2, 3, 2, 4, True),      # depth 4, d_t = 2, one partial tile
    (1, 192, 192, 31, 33, 5, 1, 2, 1, 1, False),    # k_t = 2, 1-frame cache, no bias
    (1, 768, 192, 8, 64, 1, 2, 1, 1, 0, True),      # k_t = 1: pointwise, 12 chunks
    (1, 128, 192, 10, 30, 2, 0, 3, 1, 5, True),     # p_base 5: output frames 0-2 bias only
]


@pytest.mark.parametrize("case", RD_CASES, ids=["%d_%d_%d_%dx%d_%d_%d" % c[:7] for c in RD_CASES])
def test_register_direct_1x1_every_output(cuda_device, case):
    """Every output against the oracle (bias-only outputs bit for bit), the
    cache-out byte for byte, and the packed image giving the same bits as W
    read in place."""
    n, cin, cout, h, w_, tx, tc, kt, dt, p_base, bias = case
    k = (kt, 1, 1)
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV, has_bias=bias,
                                   seed=synth.SEED_BASE + 640 + RD_CASES.index(case))
    v = "bf16_s1_n192_p256_rd"
    y, co, plan = run(x, c, w, b, k=k, pad=(0, 0), dt=dt, p_base=p_base, variant=v)
    yp, _, _ = run(x, c, w, b, k=k, pad=(0, 0), dt=dt, p_base=p_base, variant=v, packed=True, want_cache=False)
    torch.cuda.synchronize()
    assert plan.info["kernel_name"] == v and plan.info["splits"] == 1
    assert torch.equal(y, yp)
    ref = _oracle(x, c, w, b, k=k, pad=(0, 0), dt=dt, p_base=p_base)
    mask = mask_for(plan, x.shape, k=k, pad=(0, 0), dt=dt)
    assert_bias_only_exact(y, b, mask, str(case))
    if not mask.all():
        assert_bf16_close(y, ref, str(case), exclude=mask)
    z = x if c is None else torch.cat([c, x], 1)
    assert torch.equal(co, z[:, z.shape[1] - min(p_base, z.shape[1]):])


# Calls whose tiles leave most workgroup slots idle:
# causal_conv3d_forward_packed divides each tile's K stages among several
# units and sums their fp32 partials in split order (plan_info splits > 1, a
# workspace).  (name, n, c_in, c_out, k, h, w, t_x, t_cache, kernel, splits):
# every kernel that splits, split counts from 4 to 16, stage counts that do
# not divide evenly, a first chunk (one active temporal tap), two batch items.
SPLIT_CASES = [
    ("latent_384_30x52", 1, 384, 384, (3, 3, 3), 30, 52, 1, 2, "bf16_s3_n96_p8x32_x2", 16),
    ("latent_384_60x104", 1, 384, 384, (3, 3, 3), 60, 104, 1, 2, "bf16_s3_n96_p8x32_x2", 4),
    ("latent_384_45x80", 1, 384, 384, (3, 3, 3), 45, 80, 1, 2, "bf16_s3_n96_p8x32_x2", 7),
    ("latent_384_24x40_2f", 1, 384, 384, (3, 3, 3), 24, 40, 2, 2, "bf16_s3_n96_p8x32_x2", 10),
    ("latent_384_30x52_first", 1, 384, 384, (3, 3, 3), 30, 52, 1, 0, "bf16_s3_n96_p8x32_x2", 6),
    ("latent_384_12x20_n2", 2, 384, 384, (3, 3, 3), 12, 20, 1, 2, "bf16_s3_n96_p8x32_x2", 16),
    ("conv_256_96_30x52", 1, 256, 96, (3, 3, 3), 30, 52, 1, 2, "bf16_s3_n96_p8x32_x2", 12),
    ("conv_96_32_60x104_2f", 1, 96, 32, (3, 3, 3), 60, 104, 2, 2, "bf16_s3_n32_p8x32", 4),
    ("conv_512_512_24x40", 1, 512, 512, (3, 3, 3), 24, 40, 1, 2, "bf16_s3_n32_p8x32", 5),
    ("temporal_384_768_30x52", 1, 384, 768, (3, 1, 1), 30, 52, 1, 2, "bf16_s1_n192_p8x32", 4),
    ("temporal_384_768_16x64_2f", 1, 384, 768, (3, 1, 1), 16, 64, 2, 2, "bf16_s1_n192_p8x32", 4),
    # the group-staged kernel's splits of a tile's 32-channel group sequence
    ("g32_n64_latent_90x160", 1, 384, 384, (3, 3, 3), 90, 160, 1, 2, "bf16_s3_n64_p24x32_g32", 2),
    ("g32_n96_192_45x80", 1, 384, 192, (3, 3, 3), 45, 80, 1, 2, "bf16_s3_n96_p16x32_g32", 4),
    ("g32_n64_first_chunk_3f", 1, 64, 64, (3, 3, 3), 48, 64, 3, 0, "bf16_s3_n64_p24x32_g32", 2),
    ("g32_n64_n2_2f", 2, 128, 128, (3, 3, 3), 40, 70, 2, 2, "bf16_s3_n64_p24x32_g32", 4),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_reduction_every_output_and_repeatable(cuda_device, case):
    """Every output against the oracle; five launches into NaN-filled
    outputs give the same bits (the partials are summed in split order,
    whichever unit arrives last); the arrival counters are left zero."""
    name, n, cin, cout, k, h, w_, tx, tc, kernel, splits = case
    pad = (k[1] // 2, k[2] // 2)
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV,
                                   seed=synth.SEED_BASE + 600 + SPLIT_CASES.index(case))
    plan = plan_for(x, tc, w, k=k, pad=pad, p_base=2, variant=kernel)
    i = plan.info
    assert (i["kernel_name"], i["splits"]) == (kernel, splits) and i["workspace_bytes"] > 0
    img = cc3d.causal_conv3d_pack_weights(plan, w)
    ws = workspace_for(plan, DEV)
    outs = []
    for _ in range(5):
        y = nan_like(plan.shapes()["out"], torch.bfloat16, DEV)
        co = nan_like(plan.shapes()["cache_out"], torch.bfloat16, DEV)
        cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, y, co, ws)
        outs.append(y)
    torch.cuda.synchronize()
    assert all(torch.equal(o, outs[0]) for o in outs[1:])
    z = x if c is None else torch.cat([c, x], 1)
    assert torch.equal(co, z[:, -min(2, z.shape[1]):])
    counters = ws[: i["tiles"] * 4].view(torch.int32)
    assert int(counters.abs().sum()) == 0
    ref = _oracle(x, c, w, b, k=k, pad=pad, p_base=2)
    mask = mask_for(plan, x.shape, k=k, pad=pad)
    assert_bias_only_exact(outs[0], b, mask, name)
    assert_bf16_close(outs[0], ref, name, exclude=mask)
    # without a workspace the call is refused; forward (W in place) runs unsplit
    with pytest.raises(ValueError):
        cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, outs[1], None)
    y1, _, _ = run(x, c, w, b, k=k, pad=pad, p_base=2, want_cache=False, variant=kernel)
    torch.cuda.synchronize()
    assert_bf16_close(y1, ref, name + " unsplit", exclude=mask)


@pytest.mark.parametrize("variant", [None, "bf16_s3_n64_p24x32_g32"], ids=["default", "group_staged"])
def test_split_reduction_replays_in_a_graph(cuda_device, variant):
    """A split call captured in a graph: the arrival counters are reset by
    the last unit of each tile, so every replay starts from zero (the
    group-staged kernel also keeps its captured scheduler slot)."""
    s = next(v for v in synth.DECODER_SIGNATURES_480 if v["name"] == "latent_384_30x52")
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], s["h"], s["w"], s["tx"], s["tc"], s["k"], device=DEV,
                                   seed=synth.SEED_BASE + 610)
    plan = plan_for(x, s["tc"], w, k=s["k"], pad=s["pad"], p_base=s["p_base"], variant=variant)
    assert plan.info["splits"] > 1
    img = cc3d.causal_conv3d_pack_weights(plan, w)
    ws = workspace_for(plan, DEV)
    ref = nan_like(plan.shapes()["out"], torch.bfloat16, DEV)
    cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, ref, None, ws)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, out, None, ws)
    for i in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d" % i
