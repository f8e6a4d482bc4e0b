"""causal_conv3d_forward_packed_noalloc: the packed-image forward with its
split workspace in the library's static per-device array, for callers that
cannot allocate device memory.  Two calls in a row, the second on a smaller
input, each against causal_conv3d_forward_packed with a caller workspace:
identical bits (the same kernels and the same split order), and the carried
cache byte for byte."""
import pytest
import torch

import causal_conv3d_video_amd as cc3d
import synth
from gpu_util import nan_like, plan_for, workspace_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


# a small latent-width map (384->384 at 12x20): 8 tiles, 16 splits
SMALL_LATENT = dict(name="latent_384_12x20", cin=384, cout=384, h=12, w=20, tx=1, tc=2, k=(3, 3, 3), pad=(1, 1),
                    p_base=2)


def _sig(name):
    return next(v for v in synth.DECODER_SIGNATURES + synth.DECODER_SIGNATURES_480 + [SMALL_LATENT]
                if v["name"] == name)


def _both(s, seed, variant=None):
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], s["h"], s["w"], s["tx"], s["tc"], s["k"], device=DEV,
                                   seed=seed)
    plan = plan_for(x, s["tc"], w, k=s["k"], pad=s["pad"], p_base=s["p_base"], variant=variant)
    img = cc3d.causal_conv3d_pack_weights(plan, w)
    ref = nan_like(plan.shapes()["out"], torch.bfloat16, DEV)
    ref_co = nan_like(plan.shapes()["cache_out"], torch.bfloat16, DEV)
    cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, ref, ref_co, workspace_for(plan, DEV))
    got = nan_like(plan.shapes()["out"], torch.bfloat16, DEV)
    got_co = nan_like(plan.shapes()["cache_out"], torch.bfloat16, DEV)
    cc3d.causal_conv3d_forward_packed_noalloc(plan, x, c, img, b, got, got_co)
    torch.cuda.synchronize()
    return plan, ref, ref_co, got, got_co


@pytest.mark.parametrize("first,second,variant", [("latent_384_60x104", "latent_384_30x52", None),
                                                  ("latent_384_30x52", "latent_384_12x20", None),
                                                  ("latent_384", "latent_384_30x52", "bf16_s3_n64_p24x32_g32")])
def test_noalloc_matches_the_caller_workspace_call_twice_in_a_row(cuda_device, first, second, variant):
    big, small = _sig(first), _sig(second)
    p1, ref1, rco1, got1, gco1 = _both(big, synth.SEED_BASE + 800, variant)
    p2, ref2, rco2, got2, gco2 = _both(small, synth.SEED_BASE + 801, variant)
    assert p1.info["splits"] > 1 and p2.info["splits"] > 1
    assert small["h"] * small["w"] * small["cin"] < big["h"] * big["w"] * big["cin"]  # a smaller input second
    assert max(p1.info["workspace_bytes"], p2.info["workspace_bytes"]) <= cc3d.NOALLOC_SCRATCH_BYTES
    assert int(torch.isnan(got1).sum()) == 0 and int(torch.isnan(got2).sum()) == 0
    assert torch.equal(got1, ref1) and torch.equal(gco1, rco1)
    assert torch.equal(got2, ref2) and torch.equal(gco2, rco2)


def test_noalloc_runs_plans_without_a_split(cuda_device):
    s = _sig("mid_192_240x416")
    plan, ref, ref_co, got, got_co = _both(s, synth.SEED_BASE + 802)
    assert plan.info["splits"] == 1 and plan.info["workspace_bytes"] == 0
    assert torch.equal(got, ref) and torch.equal(got_co, ref_co)
