"""Seeded random small shapes, each on the default kernel choice and on every
bf16 variant that accepts it, against the fp64 oracle (every output) and the
cache-out against its source frames (byte-exact).

The bf16 bar is relative to the RMS of the whole output, so shapes whose
output is mostly exact zeros or bias (rows that see only padding, or mostly
bias-only frames) are not drawn: there the RMS falls so low that rounding
the largest outputs to bf16 alone (half a unit in the last place, 1/64 at
|y| in [4, 8)) would exceed the bar."""
import numpy as np
import pytest
import torch

import causal_conv3d_video_amd as cc3d
import oracle
import synth
from gpu_util import assert_bf16_close, run

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

VARIANTS = ["bf16_s3_n96_p16x32_g32", "bf16_s3_n64_p24x32_g32", "bf16_s3_n96_p8x32_x2", "bf16_s3_n32_p8x32",
            "bf16_s3_few_p16x128", "bf16_s3_few_p7x128", "bf16_s1_n192_p8x32", "bf16_s1_n32_p8x32",
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
                # at most the kernel's reach: an output row or column that
                # sees only padding holds exactly the bias
                pad = (int(rng.integers(0, sdil[0] * (k[1] - 1) + 1)), int(rng.integers(0, sdil[1] * (k[2] - 1) + 1)))
        p_base = dt * (k[0] - 1) + int(rng.choice([0, 0, 0, 1]))
        z = tx + tc
        t_out = (z + p_base - tc - dt * (k[0] - 1) - 1) // st + 1
        h_out = (h + 2 * pad[0] - sdil[0] * (k[1] - 1) - 1) // sst[0] + 1
        w_out = (w + 2 * pad[1] - sdil[1] * (k[2] - 1) - 1) // sst[1] + 1
        if t_out < 1 or h_out < 1 or w_out < 1:
            continue
        # a frame no tap reaches is the bias alone: keep such frames a minority
        if tc == 0 and p_base > dt * (k[0] - 1) and t_out < 3:
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


CASES = _cases(48, 20261203 + 777) + _halo_staged_spatial_cases(12, 20261203 + 778)


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_random_shape_on_every_accepting_variant(cuda_device, case):
    cin, cout, h, w_, tx, tc, k, pad, sst, sdil, st, dt, p_base, n, bias = case
    x, c, w, b = synth.conv_inputs(n, cin, cout, h, w_, tx, tc, k, device=DEV,
                                   seed=synth.SEED_BASE + 500 + CASES.index(case), has_bias=bias)
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
    for v in names:
        y, co, plan = run(x, c, w, b, k=k, pad=pad, dt=dt, p_base=p_base, st=st, sst=sst, sdil=sdil, variant=v)
        torch.cuda.synchronize()
        assert tuple(y.shape) == ref.shape
        assert_bf16_close(y, ref, "%s %s" % (plan.info["kernel_name"], case))
        keep = min(p_base, z.shape[1])
        assert torch.equal(co, z[:, z.shape[1] - keep:]), plan.info["kernel_name"]
