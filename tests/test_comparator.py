"""CPU checks of the test-side comparison tools: the streaming comparator
gives the metrics of the all-at-once comparison, and the bias-only mask
marks exactly the outputs the oracle's sum never reaches."""
import numpy as np
import pytest
import torch

import oracle
import synth
from comparator import Comparator, frame_points
from gpu_util import bias_only_mask, metrics


def test_streaming_comparator_equals_the_whole_comparison():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((2, 3, 5, 7, 4))
    got = ref + rng.standard_normal(ref.shape) * 1e-3
    got[1, 2, 4, 6, 3] += 0.5  # one outlier
    exclude = rng.random((2, 3, 5, 7, 1)) < 0.2
    exclude[1, 2, 4, 6] = False
    whole = metrics(got, ref, exclude)
    cmp = Comparator("t")
    for n in range(2):
        for o in range(3):
            cmp.add(got[n, o], ref[n, o], exclude[n, o])
    part = cmp.metrics()
    for key in ("max_abs", "mean_abs", "rmse", "rms_ref", "cos"):
        assert part[key] == pytest.approx(whole[key], rel=1e-12, abs=1e-15), key
    assert part["count"] == whole["count"]
    assert part["max_abs"] >= 0.5 - 1e-3
    with pytest.raises(AssertionError):
        cmp.assert_bf16()  # the outlier exceeds 2e-2 * RMS


def test_streaming_comparator_counts_nonfinite_values():
    cmp = Comparator("t")
    ref = np.ones((4, 4))
    got = ref.copy()
    got[1, 1] = np.nan
    cmp.add(got, ref)
    assert cmp.metrics()["nonfinite_gpu"] == 1
    with pytest.raises(AssertionError):
        cmp.assert_bf16()


def test_frame_points_cover_one_frame_in_row_major_order():
    p = frame_points(1, 2, 3, 4)
    assert p.shape == (12, 4)
    assert (p[:, 0] == 1).all() and (p[:, 1] == 2).all()
    assert p[:, 2].tolist() == [0] * 4 + [1] * 4 + [2] * 4 and p[:, 3].tolist() == [0, 1, 2, 3] * 3


@pytest.mark.parametrize("case", [
    # (h, w, tx, tc, k, stride, dilation, pad, p_base)
    (6, 9, 2, 0, (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1), 4),     # bias-only leading frames
    (5, 7, 3, 1, (3, 3, 3), (1, 1, 1), (1, 1, 1), (3, 2), 2),     # rows and columns all padding
    (7, 6, 2, 2, (2, 5, 3), (2, 2, 1), (2, 2, 1), (9, 2), 2),     # stride and dilation, padded rows
    (4, 4, 1, 0, (3, 1, 1), (1, 1, 1), (1, 1, 1), (0, 0), 3),     # (3,1,1) with a deep base pad
    (3, 8, 4, 3, (3, 3, 1), (2, 1, 2), (1, 2, 1), (5, 0), 5),     # temporal stride, padded rows
])
def test_bias_only_mask_marks_exactly_the_unreached_outputs(case):
    """With no bias and random inputs, the oracle's output is exactly zero in
    every channel where no term is summed, and (almost surely) nonzero
    elsewhere: the mask must match that pattern."""
    h, w, tx, tc, k, stride, dil, pad, p_base = case
    x, c, wt, _ = synth.conv_inputs(1, 16, 5, h, w, tx, tc, k, seed=11, has_bias=False)
    y = oracle.conv3d(x, c, wt, None, stride=stride, dilation=dil, padding=pad, pbase=p_base)
    zero = (y == 0).all(-1)
    m = bias_only_mask(1, y.shape[1], y.shape[2], y.shape[3], tz=tx + tc, p_l=p_base - tc, kt=k[0], kh=k[1], kw=k[2],
                       st=stride[0], sh=stride[1], sw=stride[2], dt=dil[0], dh=dil[1], dw=dil[2], ph=pad[0], pw=pad[1],
                       h=h, w=w)
    assert m.shape == y.shape[:4] + (1,)
    assert np.array_equal(m[..., 0], zero)
    assert zero.any() and not zero.all()


def test_bf16_bar_falls_back_to_faithful_rounding_below_the_bf16_step():
    """An output of 5 rounded to bf16 is 1/64 off at worst; beside an RMS of
    0.5 the stated bar (2e-2 x RMS = 0.01) is below that step, so the bar
    becomes faithful rounding: either bf16 neighbour passes, one step and a
    half off fails, and the strict bar alone fails both."""
    from gpu_util import assert_bf16_close, bf16_step
    ref = np.full(128, 0.25)
    ref[0] = 5.0 + 1.0 / 64  # exactly between two bf16 numbers (5.0 and 5.03125); RMS ~0.51
    assert bf16_step(5.0) == 1.0 / 32 and bf16_step(0.25) == 1.0 / 512
    near = ref.copy()
    near[0] = 5.0  # a bf16 neighbour, 1/64 off
    m = assert_bf16_close(near, ref)
    assert m["max_abs"] == pytest.approx(1.0 / 64) and m["unfaithful"] == 0
    with pytest.raises(AssertionError):
        assert_bf16_close(near, ref, strict=True)
    far = ref.copy()
    far[0] = 5.0 - 1.0 / 32  # the next bf16 number down: 3/64 off, beyond one step
    with pytest.raises(AssertionError):
        assert_bf16_close(far, ref)
    cmp = Comparator("t")
    cmp.add(near[:64], ref[:64])
    cmp.add(near[64:], ref[64:])
    assert cmp.assert_bf16()["beyond_step"] <= 0
    with pytest.raises(AssertionError):
        cmp.assert_bf16(strict=True)
