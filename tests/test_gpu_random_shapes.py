"""Seeded random shapes -- small ones, and maps large enough that every
kernel runs several tiles per workgroup -- each on the default kernel choice
and on every bf16 variant that accepts it, against the fp64 oracle (every output) and the
cache-out against its source frames (byte-exact); each variant also from its
packed weight image, which must give the same bits as reading W in place
(unless the packed call splits its K stages, whose sums round differently).

Outputs that no term of the sum reaches (frames with no active temporal tap,
rows or columns whose spatial taps all fall in the padding) must equal the
bias bit for bit; the bf16 bar (2e-2 x RMS of the oracle) is applied to the
other outputs, whose RMS it is taken over.  So shapes whose output is mostly
bias are drawn like any other: relative to the RMS of the whole output, the
rounding of the largest reached outputs to bf16 alone (half a unit in the
last place, 1/64 at |y| in [4, 8)) could exceed the bar there."""
import numpy as np
import pytest
import torch

import causal_conv3d_video_amd as cc3d
import oracle
import synth
from gpu_util import assert_bf16_close, assert_bias_only_exact, mask_for, nan_like, plan_for, run, workspace_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

VARIANTS = ["bf16_s3_n96_p16x32_g32", "bf16_s3_n64_p24x32_g32", "bf16_s3_n96_p8x32_x2", "bf16_s3_n32_p8x32",
            "bf16_s3_few_p16x128", "bf16_s3_few_p7x128", "bf16_s1_n192_p8x32", "bf16_s1_n192_p256_rd", "bf16_s1_n32_p8x32",
            "bf16_gen_n64_p8x32", "bf16_gen_n96_p8x32", "bf16_s3d2_n64_p16x32_g32", "bf16_s3s2_n96_p4x32_g32",
            "bf16_s3s2_n64_p4x32_g32"]


def _cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        kind = rng.choice(["s3", "s1", "gen", "few"])
        n = int(rng.choice([1, 1, 1, 2]))
        h, w = int(rng.integers(1, 25)), int(rng.integers(1, 73))
        tx, tc = int(rng.integers(1, 6)), int(rng.integers(0, 5))
        sst, sdil = (1, 1), (1, 1)
        if kind == "few":
            cin, cout = int(rng.choice([32, 64, 96])), int(rng.integers(1, 6))
            k, pad, dt, st = (3, 3, 3), (1, 1), 1, 1
        else:
            cin = int(rng.choice([16, 32, 32, 48, 64, 64, 96]))
            cout = int(rng.choice([8, 32, 40, 64, 96, 96, 128, 192, 192]))
            kt = int(rng.choice([1, 2, 3, 3, 3]))
            dt, st = int(rng.choice([1, 1, 2])), int(rng.choice([1, 1, 1, 2]))
            if kind == "s3":
                k, pad = (kt, 3, 3), (1, 1)
            elif kind == "s1":
                k, pad = (kt, 1, 1), (0, 0)
            else:
                ks = int(rng.choice([1, 3, 5]))
                k = (kt, ks, int(rng.choice([1, 3])))
                sst = (int(rng.choice([1, 2])), int(rng.choice([1, 2])))
                sdil = (int(rng.choice([1, 2])), 1) if ks != 3 or rng.integers(0, 2) else (2, 2)
                # up to one past the kernel's reach: an output row or column
                # that sees only padding holds exactly the bias
                pad = (int(rng.integers(0, sdil[0] * (k[1] - 1) + 2)), int(rng.integers(0, sdil[1] * (k[2] - 1) + 2)))
        p_base = dt * (k[0] - 1) + int(rng.choice([0, 0, 0, 1]))
        z = tx + tc
        t_out = (z + p_base - tc - dt * (k[0] - 1) - 1) // st + 1
        h_out = (h + 2 * pad[0] - sdil[0] * (k[1] - 1) - 1) // sst[0] + 1
        w_out = (w + 2 * pad[1] - sdil[1] * (k[2] - 1) - 1) // sst[1] + 1
        if t_out < 1 or h_out < 1 or w_out < 1:
            continue
        bias = bool(rng.integers(0, 4) > 0)
        out.append((cin, cout, h, w, tx, tc, k, pad, sst, sdil, st, dt, p_base, n, bias))
    return out


def _halo_staged_spatial_cases(count, seed):
    """3x3 convs at spatial stride 2 (padding 1) or spatial dilation 2
    (padding 2): the envelopes of the strided and dilated group-staged
    kernels (which the draws above rarely reach), with channel counts they
    accept and ones they refuse."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        strided = bool(rng.integers(0, 2))
        cin = int(rng.choice([32, 64, 96, 48]))
        cout = int(rng.choice([64, 96, 128, 192, 40]))
        n = int(rng.choice([1, 1, 2]))
        h, w = int(rng.integers(1, 41)), int(rng.integers(1, 101))
        tx, tc = int(rng.integers(1, 5)), int(rng.integers(0, 4))
        kt = int(rng.choice([2, 3, 3]))
        dt, st = int(rng.choice([1, 1, 2])), int(rng.choice([1, 1, 2]))
        k = (kt, 3, 3)
        sst, sdil, pad = ((2, 2), (1, 1), (1, 1)) if strided else ((1, 1), (2, 2), (2, 2))
        p_base = dt * (kt - 1)
        z = tx + tc
        t_out = (z + p_base - tc - dt * (kt - 1) - 1) // st + 1
        if t_out < 1:
            continue
        bias = bool(rng.integers(0, 4) > 0)
        out.append((cin, cout, h, w, tx, tc, k, pad, sst, sdil, st, dt, p_base, n, bias))
    return out


def _multi_tile_cases(count, seed):
    """Maps large enough that every kernel runs several tiles per workgroup
    (its load cursor crossing tile boundaries), with leading output frames
    that no temporal tap reaches (p_base up to 3 past d_t (k_t - 1)) and
    frame counts that do not divide the per-XCD tile stride."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        kind = rng.choice(["s3", "s1", "s1", "few"])
        n = int(rng.choice([1, 1, 2]))
        h, w = int(rng.integers(40, 73)), int(rng.integers(160, 289))
        tx, tc = int(rng.integers(2, 6)), int(rng.integers(0, 5))
        kt = int(rng.choice([2, 3, 3]))
        dt = int(rng.choice([1, 1, 2]))
        if kind == "few":
            cin, cout, kt, dt = int(rng.choice([32, 64, 96])), int(rng.integers(1, 6)), 3, 1
        else:
            cin = int(rng.choice([32, 64, 64, 96, 128]))
            cout = int(rng.choice([32, 64, 96, 192]))
        k, pad = ((kt, 3, 3), (1, 1)) if kind in ("s3", "few") else ((kt, 1, 1), (0, 0))
        p_base = dt * (kt - 1) + int(rng.choice([0, 1, 2, 3]))
        t_out = tx + tc + p_base - tc - dt * (kt - 1)
        if t_out < 3:
            continue
        bias = bool(rng.integers(0, 4) > 0)
        out.append((cin, cout, h, w, tx, tc, k, pad, (1, 1), (1, 1), 1, dt, p_base, n, bias))
    return out


CASES = _cases(56, 20261203 + 777) + _halo_staged_spatial_cases(12, 20261203 + 778)
MULTI_TILE_CASES = _multi_tile_cases(24, 20261203 + 780)


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_random_shape_on_every_accepting_variant(cuda_device, case):
    _every_accepting_variant(case, synth.SEED_BASE + 500 + CASES.index(case))


@pytest.mark.parametrize("case", MULTI_TILE_CASES, ids=[str(i) for i in range(len(MULTI_TILE_CASES))])
def test_random_multi_tile_shape_on_every_accepting_variant(cuda_device, case):
    _every_accepting_variant(case, synth.SEED_BASE + 900 + MULTI_TILE_CASES.index(case))


def _every_accepting_variant(case, seed):
    cin, cout, h, w_, tx, tc, k, pad, sst, sdil, st, dt, p_base, n, bias = case
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV, seed=seed, has_bias=bias)
    def cpu(t):
        return None if t is None else t.detach().cpu()

    # the oracle takes the bf16 tensors themselves (their bits, widened exactly)
    ref = oracle.conv3d(cpu(x), cpu(c), cpu(w), cpu(b), stride=(st,) + sst, dilation=(dt,) + sdil, padding=pad,
                        pbase=p_base)
    z = x if c is None else torch.cat([c, x], 1)
    desc = cc3d.make_desc(n, cin, cout, h, w_, tx, tc, k=k, stride=(st,) + sst, dilation=(dt,) + sdil, padding=pad,
                          p_base=p_base, has_bias=bias)
    names = [None]
    for v in VARIANTS:
        try:
            cc3d.causal_conv3d_plan_variant(desc, v).close()
            names.append(v)
        except cc3d.CC3DError as e:
            assert e.status == cc3d.CC3D_ERR_UNSUPPORTED, (v, e.status)
    mask = None
    for v in names:
        y, co, plan = run(x, c, w, b, k=k, pad=pad, dt=dt, p_base=p_base, st=st, sst=sst, sdil=sdil, variant=v)
        yp, _, _ = run(x, c, w, b, k=k, pad=pad, dt=dt, p_base=p_base, st=st, sst=sst, sdil=sdil, variant=v,
                       packed=True, want_cache=False)
        torch.cuda.synchronize()
        name = "%s %s" % (plan.info["kernel_name"], case)
        assert tuple(y.shape) == ref.shape
        if mask is None:
            mask = mask_for(plan, x.shape, k=k, pad=pad, st=st, sst=sst, dt=dt, sdil=sdil)
        assert_bias_only_exact(y, b, mask, name)
        if not mask.all():
            assert_bf16_close(y, ref, name, exclude=mask)
        if plan.info["splits"] == 1:
            assert torch.equal(y, yp), "packed image and W in place differ: " + name
        else:  # the packed call splits K: other rounding, the same bar
            assert_bias_only_exact(yp, b, mask, name + " split")
            if not mask.all():
                assert_bf16_close(yp, ref, name + " split", exclude=mask)
        keep = min(p_base, z.shape[1])
        assert torch.equal(co, z[:, z.shape[1] - keep:]), plan.info["kernel_name"]


def _group_staged_split_cases(count, seed):
    """Maps small enough that the group-staged kernel splits its tiles'
    channel groups (or, with one 32-channel group, does not), with temporal
    taps, dilation, cache depth and batch drawn as above."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        v = str(rng.choice(["bf16_s3_n64_p24x32_g32", "bf16_s3_n96_p16x32_g32"]))
        cin = int(rng.choice([32, 64, 96, 128, 192]))
        cout = int(rng.choice([64, 128, 192])) if "n64" in v else int(rng.choice([96, 192, 288]))
        n = int(rng.choice([1, 1, 2]))
        h, w = int(rng.integers(1, 60)), int(rng.integers(1, 100))
        tx, tc = int(rng.integers(1, 5)), int(rng.integers(0, 5))
        kt, dt = int(rng.choice([1, 2, 3, 3])), int(rng.choice([1, 1, 2]))
        p_base = dt * (kt - 1) + int(rng.choice([0, 0, 1]))
        if tx + p_base - dt * (kt - 1) < 1:
            continue
        out.append((v, cin, cout, h, w, tx, tc, kt, dt, p_base, n))
    return out


SPLIT_CASES = _group_staged_split_cases(24, 20261203 + 779)


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[str(i) for i in range(len(SPLIT_CASES))])
def test_group_staged_split_units_packed_with_cache_out(cuda_device, case):
    """The packed-image forward with a workspace (split units where the
    planner splits): every output against the oracle, the cache-out copied in
    the kernel's tail byte for byte, and the arrival counters left zero."""
    v, cin, cout, h, w_, tx, tc, kt, dt, p_base, n = case
    k = (kt, 3, 3)
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV,
                                   seed=synth.SEED_BASE + 700 + SPLIT_CASES.index(case))
    plan = plan_for(x, tc, w, k=k, pad=(1, 1), dt=dt, p_base=p_base, variant=v)
    img = cc3d.causal_conv3d_pack_weights(plan, w)
    ws = workspace_for(plan, DEV)
    y = nan_like(plan.shapes()["out"], torch.bfloat16, DEV)
    co = nan_like(plan.shapes()["cache_out"], torch.bfloat16, DEV)
    cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, y, co, ws)
    torch.cuda.synchronize()

    def cpu(t):
        return None if t is None else t.detach().cpu()

    ref = oracle.conv3d(cpu(x), cpu(c), cpu(w), cpu(b), dilation=(dt, 1, 1), padding=(1, 1), pbase=p_base)
    name = "%s splits=%d %s" % (v, plan.info["splits"], case)
    mask = mask_for(plan, x.shape, k=k, pad=(1, 1), dt=dt)
    assert_bias_only_exact(y, b, mask, name)
    if not mask.all():
        assert_bf16_close(y, ref, name, exclude=mask)
    z = x if c is None else torch.cat([c, x], 1)
    keep = min(p_base, z.shape[1])
    assert torch.equal(co, z[:, z.shape[1] - keep:]), name
    if ws is not None:
        assert int(ws[: plan.info["tiles"] * 4].view(torch.int32).abs().sum()) == 0, name


def test_group_staged_split_cases_do_split():
    """(host) most of the draws above are split, some are not"""
    splits = []
    for v, cin, cout, h, w_, tx, tc, kt, dt, p_base, n in SPLIT_CASES:
        d = cc3d.make_desc(n, cin, cout, h, w_, tx, tc, k=(kt, 3, 3), dilation=(dt, 1, 1), p_base=p_base)
        splits.append(cc3d.causal_conv3d_plan_variant(d, v).info["splits"])
    assert sum(s > 1 for s in splits) >= len(splits) // 2 and min(splits) == 1
