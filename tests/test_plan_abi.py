"""Host-side tests of the C ABI: the library loads and exports what
include/cc3d.h declares, the planner's tap intervals match a brute-force
enumeration of the lowering's source-time rule ("Cache-Aware Conv3D Lowering
Across Embedded World-Model Decoders", lowering section), and the contract
checks return the documented status codes.  No GPU is used: planning is
host-only."""
import ctypes
import itertools
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_if_missing():
    lib = os.path.join(ROOT, "causal_conv3d_video_amd", "libcc3d.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location("cc3d_build", os.path.join(ROOT, "causal_conv3d_video_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return lib


LIB = _build_if_missing()

import causal_conv3d_video_amd as cc3d  # noqa: E402
import oracle  # noqa: E402


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "cc3d.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(causal_conv3d_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert declared, "no declarations found"
    assert set(declared) == set(cc3d.EXPORTED_SYMBOLS)
    lib = ctypes.CDLL(LIB)
    for name in declared:
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)", nm))
    for name in declared:
        assert name in exported, name


def test_library_has_no_undefined_internal_symbols():
    # every kernel launch stub and helper must be defined inside the library
    nm = subprocess.run(["nm", "-D", "--undefined-only", LIB], capture_output=True, text=True, check=True).stdout
    bad = [l for l in nm.splitlines() if "_GLOBAL__N_" in l or "cc3d" in l or "conv_" in l]
    assert not bad, bad


def test_library_has_gfx950_code_object():
    # the embedded HIP fat binary names its one offload target
    data = open(LIB, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def _desc(**kw):
    base = dict(n=1, c_in=16, c_out=16, h=8, w=8, t_x=4, t_cache=0, k=(3, 3, 3), stride=(1, 1, 1),
                dilation=(1, 1, 1), padding=(1, 1), p_base=2, dtype=torch.bfloat16)
    base.update(kw)
    return cc3d.make_desc(**base)


def _brute_intervals(t_x, t_c, k_t, d_t, p_base, t_out):
    """Active (o, k) pairs straight from the rule: tap k of output o reads
    source frame o + k*d_t - (p_base - |C|), valid iff inside [0, |Z|)."""
    tz = t_x + t_c
    pl = p_base - t_c
    res = []
    for k in range(k_t):
        outs = [o for o in range(t_out) if 0 <= o + k * d_t - pl < tz]
        res.append(outs)
    return res


def test_tap_intervals_match_brute_force_enumeration():
    n_checked = 0
    for k_t, d_t in itertools.product((1, 2, 3), (1, 2, 3)):
        for p_base in range(0, d_t * (k_t - 1) + 2):
            for t_x in range(1, 9):
                for t_c in range(0, p_base + 2):
                    shp = oracle.out_shape(t_x, t_c, 8, 8, kt=k_t, kh=3, kw=3, dt=d_t, pbase=p_base)
                    desc = _desc(t_x=t_x, t_cache=t_c, k=(k_t, 3, 3), dilation=(d_t, 1, 1), p_base=p_base)
                    if shp is None:
                        with pytest.raises(cc3d.CC3DError) as e:
                            cc3d.causal_conv3d_plan(desc)
                        assert e.value.status == cc3d.CC3D_ERR_INVALID_ARG
                        continue
                    plan = cc3d.causal_conv3d_plan(desc)
                    info = plan.info
                    assert (info["t_out"], info["h_out"], info["w_out"]) == shp
                    assert info["t_z"] == t_x + t_c
                    assert info["p_l"] == p_base - t_c
                    assert info["t_cache_out"] == min(p_base, t_x + t_c)
                    brute = _brute_intervals(t_x, t_c, k_t, d_t, p_base, info["t_out"])
                    active = 0
                    for k, tap in enumerate(info["taps"]):
                        outs = brute[k]
                        assert tap["delta"] == k * d_t - (p_base - t_c)
                        # I3: the active outputs form exactly [o_lo, o_hi)
                        assert list(range(tap["o_lo"], tap["o_hi"])) == outs
                        assert bool(tap["active"]) == bool(outs)
                        # I1: source interval has the output interval's length
                        assert tap["src_hi"] - tap["src_lo"] == tap["o_hi"] - tap["o_lo"]
                        if outs:
                            active += 1
                            # I2: source interval inside Z
                            assert 0 <= tap["src_lo"] < tap["src_hi"] <= t_x + t_c
                            assert tap["src_lo"] == outs[0] + tap["delta"]
                    assert info["n_active_taps"] == active
                    if p_base == d_t * (k_t - 1):
                        # I4: output length equals input length
                        assert info["t_out"] == t_x
                        # I5: the last tap reads exactly X
                        last = info["taps"][k_t - 1]
                        assert (last["o_lo"], last["o_hi"]) == (0, t_x)
                        assert (last["src_lo"], last["src_hi"]) == (t_c, t_c + t_x)
                    n_checked += 1
    assert n_checked > 500


def test_tiny_workload_intervals():
    # No cache, 4 frames, base pad 2: p_l = 2, four output frames; taps
    # (delta, o_lo, o_hi) = (-2, 2, 4), (-1, 1, 4), (0, 0, 4).
    a = cc3d.causal_conv3d_plan(_desc(c_in=8, c_out=8, t_x=4, t_cache=0, dtype=torch.float32)).info
    assert a["p_l"] == 2 and a["t_out"] == 4
    assert [(t["delta"], t["o_lo"], t["o_hi"]) for t in a["taps"]] == [(-2, 2, 4), (-1, 1, 4), (0, 0, 4)]
    # Two cached frames ahead of four new ones: p_l = 0, every tap on every frame.
    b = cc3d.causal_conv3d_plan(_desc(c_in=8, c_out=8, t_x=4, t_cache=2, dtype=torch.float32)).info
    assert b["p_l"] == 0 and b["t_out"] == 4
    assert [(t["delta"], t["o_lo"], t["o_hi"]) for t in b["taps"]] == [(0, 0, 4), (1, 0, 4), (2, 0, 4)]
    # One latent frame, no cache: only the last tap is active.
    c = cc3d.causal_conv3d_plan(_desc(c_in=384, c_out=384, h=90, w=160, t_x=1, t_cache=0)).info
    assert [t["active"] for t in c["taps"]] == [0, 0, 1]
    # One latent frame behind a one-frame cache: taps 1 and 2.
    d = cc3d.causal_conv3d_plan(_desc(c_in=384, c_out=384, h=90, w=160, t_x=1, t_cache=1)).info
    assert [t["active"] for t in d["taps"]] == [0, 1, 1] and d["p_l"] == 1


def test_strided_tap_intervals_match_brute_force_enumeration():
    """Temporal stride s_t > 1: tap k of output o reads source frame
    o*s_t + k*d_t - p_l; the outputs reading a tap are still one interval
    [o_lo, o_hi), their source frames every s_t-th one of [src_lo, src_hi)."""
    checked = 0
    for s_t, k_t, d_t in itertools.product((2, 3), (1, 2, 3), (1, 2)):
        for p_base in range(0, d_t * (k_t - 1) + 2):
            for t_x in range(1, 10):
                for t_c in range(0, p_base + 2):
                    shp = oracle.out_shape(t_x, t_c, 8, 8, kt=k_t, st=s_t, dt=d_t, pbase=p_base)
                    desc = _desc(t_x=t_x, t_cache=t_c, k=(k_t, 3, 3), stride=(s_t, 1, 1), dilation=(d_t, 1, 1),
                                 p_base=p_base)
                    if shp is None:
                        with pytest.raises(cc3d.CC3DError) as e:
                            cc3d.causal_conv3d_plan(desc)
                        assert e.value.status == cc3d.CC3D_ERR_INVALID_ARG
                        continue
                    info = cc3d.causal_conv3d_plan(desc).info
                    assert (info["t_out"], info["h_out"], info["w_out"]) == shp
                    pl, tz = p_base - t_c, t_x + t_c
                    pairs = 0
                    for k, tap in enumerate(info["taps"]):
                        outs = [o for o in range(info["t_out"]) if 0 <= o * s_t + k * d_t - pl < tz]
                        assert list(range(tap["o_lo"], tap["o_hi"])) == outs
                        if outs:
                            assert tap["src_lo"] == outs[0] * s_t + tap["delta"]
                            assert tap["src_hi"] == outs[-1] * s_t + tap["delta"] + 1
                            assert 0 <= tap["src_lo"] < tap["src_hi"] <= tz
                        pairs += len(outs)
                    per = 2 * 8 * 8 * 16 * 16 * 9
                    assert info["flops_active"] == pairs * per
                    checked += 1
    assert checked > 300


@pytest.mark.parametrize("kw", [
    dict(k=(3, 5, 5), padding=(2, 2)),
    dict(stride=(1, 2, 2)),
    dict(padding=(0, 0)),
    dict(dilation=(1, 2, 2), padding=(2, 2)),
    dict(k=(3, 1, 3), padding=(0, 1)),
    dict(k=(3, 3, 3), stride=(2, 2, 2), padding=(1, 1)),
])
def test_general_spatial_parameters_take_the_gather_kernel(kw):
    """bf16 calls outside the halo-staged kernels' envelope (3x3 "same" or
    1x1, stride and dilation 1) run on the general-spatial kernel, which
    reads W as it is (its packed image is a copy of W)."""
    p = cc3d.causal_conv3d_plan(_desc(c_in=32, c_out=40, h=20, w=36, **kw))
    assert p.info["kernel_name"] == "bf16_gen_n64_p8x32" and p.info["block_m"] == 256 and p.info["block_n"] == 64
    k = kw.get("k", (3, 3, 3))
    assert p.info["packed_weight_bytes"] == 40 * k[0] * k[1] * k[2] * 32 * 2
    assert p.info["workspace_bytes"] == 0
    for name in ["bf16_s3_n96_p16x32_g32", "bf16_s3_n64_p24x32_g32", "bf16_s3_n96_p8x32_x2", "bf16_s3_n32_p8x32",
                 "bf16_s1_n32_p8x32"]:
        with pytest.raises(cc3d.CC3DError):
            cc3d.causal_conv3d_plan_variant(_desc(c_in=32, c_out=192, h=20, w=36, **kw), name)
    # C_out a multiple of 96: the 96-wide gather tile; it refuses other C_out
    # (3x3 "same" at dilation 2, and 3x3 at stride 2 with padding 1, have
    # halo-staged kernels of their own)
    cin = 32
    if kw.get("dilation") == (1, 2, 2) and kw.get("padding") == (2, 2):
        d2 = cc3d.causal_conv3d_plan(_desc(c_in=32, c_out=192, h=20, w=36, **kw))
        assert d2.info["kernel_name"] == "bf16_s3d2_n64_p16x32_g32" and d2.info["block_n"] == 64
        cin = 48  # C_in % 32 != 0: not the dilated kernel
    if kw.get("stride", (1, 1, 1))[1:] == (2, 2) and kw.get("padding", (1, 1)) == (1, 1):
        s2 = cc3d.causal_conv3d_plan(_desc(c_in=32, c_out=192, h=20, w=36, **kw))
        assert s2.info["kernel_name"] == "bf16_s3s2_n96_p4x32_g32" and s2.info["block_n"] == 96
        assert s2.info["block_m"] == 128 and s2.info["h_out"] == 10 and s2.info["w_out"] == 18
        cin = 48  # C_in % 32 != 0: not the strided kernel
    q = cc3d.causal_conv3d_plan(_desc(c_in=cin, c_out=192, h=20, w=36, **kw))
    assert q.info["kernel_name"] == "bf16_gen_n96_p8x32" and q.info["block_n"] == 96 and q.info["tiles"] % 2 == 0
    with pytest.raises(cc3d.CC3DError):
        cc3d.causal_conv3d_plan_variant(_desc(c_in=cin, c_out=40, h=20, w=36, **kw), "bf16_gen_n96_p8x32")


def test_head_patch_height_rule():
    """The default few-channel patch height: the one (4 .. 16) with the fewest
    halo rows per compute unit, ceil(patches / 256) * (rows + 2), tallest on
    ties; checked against brute force over map sizes and batches."""
    import math
    for (n, h, w) in [(1, 720, 1280), (1, 480, 848), (1, 360, 640), (2, 180, 320), (1, 40, 72), (1, 1, 1),
                      (1, 17, 129), (3, 1080, 1920), (1, 256, 4096)]:
        strips = n * math.ceil(w / 128)
        cost = {r: math.ceil(strips * math.ceil(h / r) / 256) * (r + 2) for r in range(4, 17)}
        want = max(r for r in cost if cost[r] == min(cost.values()))
        p = cc3d.causal_conv3d_plan(_desc(n=n, c_in=96, c_out=3, h=h, w=w, t_x=2, t_cache=2))
        assert p.info["kernel_name"] == "bf16_s3_few_p%dx128" % want, (n, h, w)
        assert p.info["tiles"] == strips * math.ceil(h / want) and p.info["block_m"] == want * 128


def test_strided_calls_never_take_the_head_kernel():
    d = _desc(c_in=96, c_out=3, h=64, w=64, t_x=4, t_cache=2, stride=(2, 1, 1))
    assert cc3d.causal_conv3d_plan(d).info["kernel_name"] == "bf16_s3_n32_p8x32"
    with pytest.raises(cc3d.CC3DError) as e:
        cc3d.causal_conv3d_plan_variant(d, "bf16_s3_few_p16x128")
    assert e.value.status == cc3d.CC3D_ERR_UNSUPPORTED


def test_flops_and_bytes():
    p = cc3d.causal_conv3d_plan(_desc(c_in=192, c_out=192, h=360, w=640, t_x=4, t_cache=2)).info
    nominal = 2 * 1 * 4 * 360 * 640 * 192 * 192 * 27
    assert p["flops_nominal"] == nominal
    assert p["flops_active"] == nominal
    frame = 360 * 640 * 192 * 2
    assert p["bytes_conv"] == 6 * frame + 192 * 27 * 192 * 2 + 192 * 2 + 4 * frame
    assert p["bytes_cache_out"] == 2 * 2 * frame
    # the head kernel writes the cache-out from its staged rows: written only
    h = cc3d.causal_conv3d_plan(_desc(c_in=96, c_out=3, h=72, w=128, t_x=4, t_cache=2)).info
    assert h["kernel_name"].startswith("bf16_s3_few_") and h["bytes_cache_out"] == 2 * 72 * 128 * 96 * 2
    q = cc3d.causal_conv3d_plan(_desc(c_in=16, c_out=16, t_x=1, t_cache=0)).info
    assert q["flops_active"] == q["flops_nominal"] / 3


@pytest.mark.parametrize("kw,status", [
    (dict(groups=2), cc3d.CC3D_ERR_UNSUPPORTED),
    (dict(k=(9, 3, 3), p_base=8), cc3d.CC3D_ERR_UNSUPPORTED),      # k_t above the maximum
    (dict(k=(5, 3, 3), p_base=4), cc3d.CC3D_ERR_UNSUPPORTED),      # bf16: k_t > 4
    (dict(c_in=24), cc3d.CC3D_ERR_UNSUPPORTED),                    # bf16 needs C_in % 16 == 0
    (dict(n=0), cc3d.CC3D_ERR_INVALID_ARG),
    (dict(t_x=0), cc3d.CC3D_ERR_INVALID_ARG),
    (dict(t_cache=-1), cc3d.CC3D_ERR_INVALID_ARG),
    (dict(t_x=1, p_base=0), cc3d.CC3D_ERR_INVALID_ARG),            # empty output
    (dict(h=1, padding=(0, 0), k=(3, 3, 3), dtype=torch.float32), cc3d.CC3D_ERR_INVALID_ARG),
])
def test_refusals_and_counters(kw, status):
    cc3d.causal_conv3d_counters(reset=True)
    with pytest.raises(cc3d.CC3DError) as e:
        cc3d.causal_conv3d_plan(_desc(**kw))
    assert e.value.status == status
    c = cc3d.causal_conv3d_counters()
    key = "unsupported" if status == cc3d.CC3D_ERR_UNSUPPORTED else "invalid"
    assert c[key] == 1 and c["fast_path"] == 0


def test_fp32_accepts_general_spatial_parameters():
    p = cc3d.causal_conv3d_plan(_desc(c_in=3, c_out=5, k=(3, 5, 5), stride=(1, 2, 2), dilation=(2, 2, 1),
                                      padding=(2, 1), p_base=4, dtype=torch.float32))
    assert p.info["kernel_name"] == "f32_direct"


def test_forward_refuses_bad_pointers_without_launching():
    lib = ctypes.CDLL(LIB)
    lib.causal_conv3d_forward.argtypes = [ctypes.c_void_p] * 8
    lib.causal_conv3d_forward.restype = ctypes.c_int
    plan = cc3d.causal_conv3d_plan(_desc(t_cache=2))
    cc3d.causal_conv3d_counters(reset=True)
    base = 1 << 40  # never dereferenced: every call below is refused before any launch
    mb = 1 << 20
    x, c, w, b, out, co = base, base + mb, base + 2 * mb, base + 3 * mb, base + 4 * mb, base + 5 * mb
    f = lib.causal_conv3d_forward
    assert f(None, x, c, w, b, out, co, None) == cc3d.CC3D_ERR_INVALID_ARG      # no plan
    assert f(plan.handle, None, c, w, b, out, co, None) == cc3d.CC3D_ERR_INVALID_ARG  # no x
    assert f(plan.handle, x, None, w, b, out, co, None) == cc3d.CC3D_ERR_INVALID_ARG  # cache needed
    assert f(plan.handle, x, c, w, None, out, co, None) == cc3d.CC3D_ERR_INVALID_ARG  # bias needed
    assert f(plan.handle, x + 2, c, w, b, out, co, None) == cc3d.CC3D_ERR_INVALID_ARG  # misaligned
    assert f(plan.handle, x, c, w, b, x + 16, co, None) == cc3d.CC3D_ERR_INVALID_ARG  # out overlaps x
    assert f(plan.handle, x, c, w, b, out, c, None) == cc3d.CC3D_ERR_INVALID_ARG  # cache_out aliases cache_in
    assert f(plan.handle, x, c, w, b, out, out, None) == cc3d.CC3D_ERR_INVALID_ARG  # cache_out aliases out
    cnt = cc3d.causal_conv3d_counters()
    assert cnt["invalid"] == 8 and cnt["fast_path"] == 0


def test_status_strings():
    for s in range(5):
        assert cc3d.causal_conv3d_status_string(s)
    assert "unknown" in cc3d.causal_conv3d_status_string(99)


def test_workload_signatures_get_mfma_kernels():
    sigs = [
        (384, 384, 90, 160, 1, 2, (3, 3, 3)),
        (384, 768, 90, 160, 1, 2, (3, 1, 1)),
        (192, 192, 360, 640, 4, 2, (3, 3, 3)),
        (384, 192, 360, 640, 4, 2, (3, 3, 3)),
        (96, 96, 720, 1280, 4, 2, (3, 3, 3)),
        (96, 3, 720, 1280, 4, 2, (3, 3, 3)),
    ]
    for cin, cout, h, w, tx, tc, k in sigs:
        pad = (1, 1) if k[1] == 3 else (0, 0)
        p = cc3d.causal_conv3d_plan(_desc(c_in=cin, c_out=cout, h=h, w=w, t_x=tx, t_cache=tc, k=k, padding=pad))
        assert p.info["kernel_name"].startswith("bf16_"), p.info["kernel_name"]
        assert p.info["tiles"] > 0 and p.info["packed_weight_bytes"] >= cout * k[0] * k[1] * k[2] * cin * 2


def test_packed_entry_points_refuse_fp32_plans_and_null_pointers():
    lib = ctypes.CDLL(LIB)
    vp = ctypes.c_void_p
    lib.causal_conv3d_pack_weights.argtypes = [vp] * 4
    lib.causal_conv3d_pack_weights.restype = ctypes.c_int
    lib.causal_conv3d_forward_packed.argtypes = [vp] * 8 + [ctypes.c_int64, vp]
    lib.causal_conv3d_forward_packed.restype = ctypes.c_int
    f32 = cc3d.causal_conv3d_plan(_desc(dtype=torch.float32))
    bf = cc3d.causal_conv3d_plan(_desc(t_cache=2))
    base = 1 << 40  # never dereferenced: every call below is refused before any device call
    mb = 1 << 20
    x, c, wp, b, out = base, base + mb, base + 2 * mb, base + 3 * mb, base + 4 * mb
    assert lib.causal_conv3d_pack_weights(f32.handle, x, wp, None) == cc3d.CC3D_ERR_INVALID_ARG
    assert lib.causal_conv3d_forward_packed(f32.handle, x, c, wp, b, out, None, None, 0,
                                            None) == cc3d.CC3D_ERR_INVALID_ARG
    assert lib.causal_conv3d_pack_weights(bf.handle, None, wp, None) == cc3d.CC3D_ERR_INVALID_ARG
    assert lib.causal_conv3d_pack_weights(bf.handle, x, None, None) == cc3d.CC3D_ERR_INVALID_ARG
    # the image overlapping the weights it is packed from
    assert lib.causal_conv3d_pack_weights(bf.handle, x, x + 16, None) == cc3d.CC3D_ERR_INVALID_ARG
    assert lib.causal_conv3d_pack_weights(bf.handle, x, wp + 8, None) == cc3d.CC3D_ERR_INVALID_ARG  # misaligned
    assert lib.causal_conv3d_forward_packed(bf.handle, None, c, wp, b, out, None, None, 0,
                                            None) == cc3d.CC3D_ERR_INVALID_ARG
    assert lib.causal_conv3d_forward_packed(bf.handle, x, c, None, b, out, None, None, 0,
                                            None) == cc3d.CC3D_ERR_INVALID_ARG
    # the output overlapping the packed image
    assert lib.causal_conv3d_forward_packed(bf.handle, x, c, wp, b, wp, None, None, 0,
                                            None) == cc3d.CC3D_ERR_INVALID_ARG
    # a negative workspace size, or a size without a buffer
    assert lib.causal_conv3d_forward_packed(bf.handle, x, c, wp, b, out, None, None, -1,
                                            None) == cc3d.CC3D_ERR_INVALID_ARG
    assert lib.causal_conv3d_forward_packed(bf.handle, x, c, wp, b, out, None, None, 64,
                                            None) == cc3d.CC3D_ERR_INVALID_ARG
    assert lib.causal_conv3d_forward_packed(None, x, c, wp, b, out, None, None, 0,
                                            None) == cc3d.CC3D_ERR_INVALID_ARG


def test_plans_hold_no_device_memory_and_chunk_plans_share_one_weight_image():
    """A plan is host metadata: no device workspace.  The five chunk plans of
    a streaming signature (chunk 0 without a cache, the others with the
    2-frame carry) read one packed weight image: equal weight_layout and
    packed_weight_bytes; the layout changes with the kernel's tile or the
    weight shape, not with the frame counts."""
    for cin, cout, h, w, tx, k in [(192, 192, 360, 640, 4, (3, 3, 3)), (96, 96, 720, 1280, 4, (3, 3, 3)),
                                   (384, 384, 90, 160, 1, (3, 3, 3)), (384, 768, 90, 160, 1, (3, 1, 1)),
                                   (96, 3, 720, 1280, 4, (3, 3, 3))]:
        pad = (1, 1) if k[1] == 3 else (0, 0)
        plans = [cc3d.causal_conv3d_plan(_desc(c_in=cin, c_out=cout, h=h, w=w, t_x=tx, t_cache=tc, k=k, padding=pad))
                 for tc in (0, 2, 2, 2, 2)]
        assert len({(p.info["weight_layout"], p.info["packed_weight_bytes"]) for p in plans}) == 1
        assert all((p.info["workspace_bytes"] > 0) == (p.info["splits"] > 1) for p in plans)
    a = cc3d.causal_conv3d_plan(_desc(c_in=192, c_out=192, h=360, w=640, t_x=4, t_cache=2))
    b = cc3d.causal_conv3d_plan_variant(_desc(c_in=192, c_out=192, h=360, w=640, t_x=4, t_cache=2),
                                        "bf16_s3_n96_p16x32_g32")
    c = cc3d.causal_conv3d_plan(_desc(c_in=192, c_out=96, h=360, w=640, t_x=4, t_cache=2))
    assert a.info["weight_layout"] != b.info["weight_layout"]
    assert a.info["weight_layout"] != c.info["weight_layout"]


def test_default_kernel_choice():
    # large 3x3 maps with C_in % 32 == 0: the group-staged kernel, 24x32 x 64
    # channels where C_out % 64 == 0, else 16x32 x 96 where C_out % 96 == 0;
    # small maps: the two-workgroup 8x32 kernel
    big = cc3d.causal_conv3d_plan(_desc(c_in=192, c_out=192, h=360, w=640, t_x=4, t_cache=2))
    assert big.info["kernel_name"] == "bf16_s3_n64_p24x32_g32"
    assert big.info["block_m"] == 768 and big.info["block_n"] == 64
    assert big.info["tiles"] == 15 * 20 * 3 * 4
    big96 = cc3d.causal_conv3d_plan(_desc(c_in=96, c_out=96, h=720, w=1280, t_x=4, t_cache=2))
    assert big96.info["kernel_name"] == "bf16_s3_n96_p16x32_g32"
    assert big96.info["block_m"] == 512 and big96.info["block_n"] == 96
    assert big96.info["tiles"] == 45 * 40 * 1 * 4
    mid = cc3d.causal_conv3d_plan(_desc(c_in=64, c_out=128, h=360, w=640, t_x=4, t_cache=2))
    assert mid.info["kernel_name"] == "bf16_s3_n64_p24x32_g32"   # C_out % 96 != 0
    lat = cc3d.causal_conv3d_plan(_desc(c_in=384, c_out=384, h=90, w=160, t_x=1, t_cache=2))
    # (120 tiles of 24x32 x 64, no more row padding than 8-row tiles: the
    # group-staged tile in split units)
    assert lat.info["kernel_name"] == "bf16_s3_n64_p24x32_g32" and lat.info["splits"] == 2
    # 60 rows: 24-row tiles pad to 72, 8-row ones to 64
    lat60 = cc3d.causal_conv3d_plan(_desc(c_in=384, c_out=384, h=60, w=104, t_x=1, t_cache=2))
    assert lat60.info["kernel_name"] == "bf16_s3_n96_p8x32_x2"
    odd = cc3d.causal_conv3d_plan(_desc(c_in=48, c_out=96, h=360, w=640, t_x=4, t_cache=2))
    assert odd.info["kernel_name"] == "bf16_s3_n96_p8x32_x2"   # C_in % 32 != 0
    head = cc3d.causal_conv3d_plan(_desc(c_in=96, c_out=3, h=720, w=1280, t_x=4, t_cache=2))
    assert head.info["kernel_name"] == "bf16_s3_few_p15x128"
    # one patch walks all output frames: tiles count patches only
    assert head.info["tiles"] == 48 * 10 and head.info["block_n"] == 3
    wide = cc3d.causal_conv3d_plan(_desc(c_in=128, c_out=3, h=64, w=64, t_x=4, t_cache=2))
    assert wide.info["kernel_name"] == "bf16_s3_n32_p8x32"     # C_in > 96
    dil = cc3d.causal_conv3d_plan(_desc(c_in=96, c_out=3, h=64, w=64, t_x=4, t_cache=4, dilation=(2, 1, 1), p_base=4))
    assert dil.info["kernel_name"] == "bf16_s3_n32_p8x32"      # d_t = 2


def test_every_decoder_signature_takes_a_bf16_fast_path():
    """Every call of the 17-frame streaming decode (first chunk: one frame,
    no cache; later chunks: the steady-state frames and a 2-frame cache)
    plans onto a bf16 kernel at full size: none is refused."""
    import synth
    calls = 0
    for s in synth.DECODER_SIGNATURES:
        for t_x, t_cache in [(1, 0)] + [(s["tx"], s["tc"])] * 4:
            p = cc3d.causal_conv3d_plan(_desc(c_in=s["cin"], c_out=s["cout"], h=s["h"], w=s["w"], t_x=t_x,
                                              t_cache=t_cache, k=s["k"], padding=s["pad"], p_base=s["p_base"]))
            assert p.info["kernel_name"].startswith("bf16_"), (s["name"], p.info["kernel_name"])
            assert p.info["t_out"] == t_x and p.info["t_cache_out"] == min(2, t_x + t_cache)
            calls += 1
    assert calls == 5 * len(synth.DECODER_SIGNATURES)


VARIANTS_3X3 = ["bf16_s3_n96_p16x32_g32", "bf16_s3_n64_p24x32_g32", "bf16_s3_n96_p8x32_x2", "bf16_s3_n32_p8x32"]
VARIANTS_FEW = ["bf16_s3_few_p4x128", "bf16_s3_few_p11x128", "bf16_s3_few_p16x128", "bf16_s3_n32_p8x32"]
VARIANTS_1X1 = ["bf16_s1_n192_p8x32", "bf16_s1_n192_p256_rd", "bf16_s1_n32_p8x32"]


def test_plan_variant_pins_the_kernel():
    d3 = _desc(c_in=64, c_out=192, h=20, w=70, t_x=2, t_cache=2)
    for name in VARIANTS_3X3:
        p = cc3d.causal_conv3d_plan_variant(d3, name)
        assert p.info["kernel_name"] == name
        ref = cc3d.causal_conv3d_plan(d3)
        for key in ("t_out", "h_out", "w_out", "t_cache_out", "flops_active", "bytes_conv"):
            assert p.info[key] == ref.info[key], key
    dfew = _desc(c_in=64, c_out=3, h=20, w=70, t_x=2, t_cache=2)
    for name in VARIANTS_FEW:
        assert cc3d.causal_conv3d_plan_variant(dfew, name).info["kernel_name"] == name
    d1 = _desc(c_in=128, c_out=192, h=20, w=70, t_x=2, t_cache=2, k=(3, 1, 1), padding=(0, 0))
    for name in VARIANTS_1X1:
        assert cc3d.causal_conv3d_plan_variant(d1, name).info["kernel_name"] == name
    f32 = _desc(dtype=torch.float32)
    assert cc3d.causal_conv3d_plan_variant(f32, "f32_direct").info["kernel_name"] == "f32_direct"


@pytest.mark.parametrize("name,kw", [
    ("bf16_s3_n96_p16x32_g32", dict(c_in=48, c_out=96)),      # C_in % 32 != 0
    ("bf16_s3_n96_p16x32_g32", dict(c_in=32, c_out=64)),      # C_out % 96 != 0
    ("bf16_s3_n64_p24x32_g32", dict(c_in=32, c_out=96)),      # C_out % 64 != 0
    ("bf16_s3_n64_p24x32_g32", dict(c_in=48, c_out=64)),      # C_in % 32 != 0
    ("bf16_s3_n64_p24x32_g32", dict(c_in=32, c_out=64, k=(3, 1, 1), padding=(0, 0))),  # not 3x3
    ("bf16_s3d2_n64_p16x32_g32", dict(c_in=32, c_out=64)),   # dilation 1
    ("bf16_s3d2_n64_p16x32_g32", dict(c_in=32, c_out=96, dilation=(1, 2, 2), padding=(2, 2))),  # C_out % 64
    ("bf16_s3d2_n64_p16x32_g32", dict(c_in=48, c_out=64, dilation=(1, 2, 2), padding=(2, 2))),  # C_in % 32
    ("bf16_s3d2_n64_p16x32_g32", dict(c_in=32, c_out=64, dilation=(1, 2, 2), padding=(1, 1))),  # not "same"
    ("bf16_s3d2_n64_p16x32_g32", dict(c_in=32, c_out=64, dilation=(1, 2, 2), padding=(2, 2), stride=(1, 2, 2))),
    ("bf16_s3s2_n96_p4x32_g32", dict(c_in=32, c_out=96)),     # stride 1
    ("bf16_s3s2_n96_p4x32_g32", dict(c_in=32, c_out=64, stride=(1, 2, 2))),   # C_out % 96
    ("bf16_s3s2_n96_p4x32_g32", dict(c_in=48, c_out=96, stride=(1, 2, 2))),   # C_in % 32
    ("bf16_s3s2_n96_p4x32_g32", dict(c_in=32, c_out=96, stride=(1, 2, 2), padding=(0, 0))),   # padding 0
    ("bf16_s3s2_n96_p4x32_g32", dict(c_in=32, c_out=96, stride=(1, 2, 1))),   # stride 2 in one axis
    ("bf16_s3s2_n96_p4x32_g32", dict(c_in=32, c_out=96, stride=(1, 2, 2), dilation=(1, 2, 2), padding=(2, 2))),
    ("bf16_s3s2_n96_p4x32_g32", dict(c_in=32, c_out=96, k=(3, 5, 5), stride=(1, 2, 2), padding=(2, 2))),
    ("bf16_s3s2_n64_p4x32_g32", dict(c_in=32, c_out=96, stride=(1, 2, 2))),   # C_out % 64
    ("bf16_s3s2_n64_p4x32_g32", dict(c_in=48, c_out=64, stride=(1, 2, 2))),   # C_in % 32
    ("bf16_s3s2_n64_p4x32_g32", dict(c_in=32, c_out=64)),     # stride 1
    ("bf16_s3_n96_p8x32_x2", dict(c_in=32, c_out=40)),
    ("bf16_s1_n32_p8x32", dict(c_in=32, c_out=32)),           # 1x1 variant on a 3x3 call
    ("bf16_s3_n32_p8x32", dict(c_in=32, c_out=32, k=(3, 1, 1), padding=(0, 0))),
    ("bf16_s1_n192_p8x32", dict(c_in=16, c_out=192, k=(3, 1, 1), padding=(0, 0))),  # C_in % 32 != 0
    ("bf16_s1_n192_p256_rd", dict(c_in=64, c_out=192, k=(3, 1, 1), padding=(0, 0))),   # one 64-channel chunk
    ("bf16_s1_n192_p256_rd", dict(c_in=320, c_out=192, k=(3, 1, 1), padding=(0, 0))),  # 5 chunks
    ("bf16_s1_n192_p256_rd", dict(c_in=96, c_out=192, k=(3, 1, 1), padding=(0, 0))),   # C_in % 64 != 0
    ("bf16_s1_n192_p256_rd", dict(c_in=128, c_out=96, k=(3, 1, 1), padding=(0, 0))),   # C_out % 192 != 0
    ("bf16_s1_n192_p256_rd", dict(c_in=128, c_out=192)),                               # 3x3 call
    ("f32_direct", dict(c_in=32, c_out=32)),                  # fp32 kernel on a bf16 call
    ("bf16_s3_n32_p8x32", dict(c_in=32, c_out=32, dtype=torch.float32)),
    ("no_such_kernel", dict(c_in=32, c_out=32)),
    ("bf16_s3_few_p16x128", dict(c_in=32, c_out=6)),          # C_out > 5
    ("bf16_s3_few_p16x128", dict(c_in=128, c_out=3)),         # C_in > 96
    ("bf16_s3_few_p16x128", dict(c_in=48, c_out=3)),          # C_in % 32 != 0
    ("bf16_s3_few_p16x128", dict(c_in=32, c_out=3, k=(2, 3, 3), p_base=1)),        # k_t != 3
    ("bf16_s3_few_p16x128", dict(c_in=32, c_out=3, dilation=(2, 1, 1), p_base=4)),  # d_t != 1
    ("bf16_s3_few_p3x128", dict(c_in=32, c_out=3)),           # patch heights are 4 .. 16
    ("bf16_s3_few_p17x128", dict(c_in=32, c_out=3)),
    ("bf16_s3_few_p16x32", dict(c_in=32, c_out=3)),           # strips are 128 columns
])
def test_plan_variant_refuses_what_it_cannot_run(name, kw):
    with pytest.raises(cc3d.CC3DError) as e:
        cc3d.causal_conv3d_plan_variant(_desc(**kw), name)
    assert e.value.status == cc3d.CC3D_ERR_UNSUPPORTED


def test_plan_variant_refuses_null_name():
    lib = ctypes.CDLL(LIB)
    lib.causal_conv3d_plan_variant.argtypes = [ctypes.c_void_p, ctypes.c_char_p, ctypes.POINTER(ctypes.c_void_p)]
    lib.causal_conv3d_plan_variant.restype = ctypes.c_int
    d = _desc()
    h = ctypes.c_void_p(1)
    assert lib.causal_conv3d_plan_variant(ctypes.addressof(d), None, ctypes.byref(h)) == cc3d.CC3D_ERR_INVALID_ARG
    assert h.value is None


def test_size_limits_of_the_32_bit_buffer_offsets():
    """The bf16 kernels address one frame and the weights with 32-bit byte
    offsets: a frame (input or output) or the weights reaching 2^31 bytes is
    refused as unsupported; just below, the call plans."""
    ok = cc3d.causal_conv3d_plan(_desc(c_in=112, c_out=112, h=2048, w=4096, t_x=1, t_cache=2))
    assert 2048 * 4096 * 112 * 2 < 2 ** 31 and ok.info["kernel_name"].startswith("bf16_")
    for kw in [dict(c_in=128, c_out=16, h=2048, w=4096),                  # input frame = 2^31 bytes
               dict(c_in=16, c_out=128, h=2048, w=4096),                  # output frame = 2^31 bytes
               dict(c_in=8192, c_out=4864, h=8, w=8, k=(3, 3, 3))]:      # weights >= 2^31 bytes
        with pytest.raises(cc3d.CC3DError) as e:
            cc3d.causal_conv3d_plan(_desc(t_x=1, t_cache=2, **kw))
        assert e.value.status == cc3d.CC3D_ERR_UNSUPPORTED, kw
    assert 8192 * 4864 * 27 * 2 >= 2 ** 31


def test_split_reduction_only_where_tiles_leave_slots_idle():
    """causal_conv3d_forward_packed splits each tile's K stages among units
    when the call's tiles fill at most a quarter of the workgroup slots (two
    per compute unit for the two-workgroup kernels, of 256 units): up to 16
    units, at least 4 stages each, and no split below 4 units.  Its
    workspace holds an int per tile (rounded to 256 bytes) and one fp32
    tile of partials per unit."""
    x2 = "bf16_s3_n96_p8x32_x2"
    small = cc3d.causal_conv3d_plan_variant(_desc(c_in=384, c_out=384, h=30, w=52, t_x=1, t_cache=2), x2)
    i = small.info
    assert i["kernel_name"] == x2 and i["tiles"] == 32 and i["splits"] == 16  # 72 stages
    assert i["workspace_bytes"] == 256 + 32 * 16 * 256 * 96 * 4
    # (by default that map takes the 32-wide tiles: 96 of them, split 5 ways)
    n32 = cc3d.causal_conv3d_plan(_desc(c_in=384, c_out=384, h=30, w=52, t_x=1, t_cache=2)).info
    assert n32["kernel_name"] == "bf16_s3_n32_p8x32" and n32["tiles"] == 96 and n32["splits"] == 5
    mid = cc3d.causal_conv3d_plan(_desc(c_in=384, c_out=384, h=60, w=104, t_x=1, t_cache=2))
    assert mid.info["tiles"] == 128 and mid.info["splits"] == 4               # 512 slots / 128 tiles
    lat = cc3d.causal_conv3d_plan_variant(_desc(c_in=384, c_out=384, h=90, w=160, t_x=1, t_cache=2), x2)
    assert lat.info["tiles"] == 240 and lat.info["splits"] == 1 and lat.info["workspace_bytes"] == 0  # 2 < 4
    first = cc3d.causal_conv3d_plan_variant(_desc(c_in=384, c_out=384, h=30, w=52, t_x=1, t_cache=0), x2)
    assert first.info["splits"] == 6                                         # one active tap: 24 stages
    two = cc3d.causal_conv3d_plan_variant(_desc(c_in=48, c_out=384, h=30, w=52, t_x=1, t_cache=2), x2)
    assert two.info["tiles"] == 32 and two.info["splits"] == 1               # 9 stages: 2 units at most
    few_stages = cc3d.causal_conv3d_plan(_desc(c_in=16, c_out=384, h=90, w=160, t_x=1, t_cache=2))
    assert few_stages.info["splits"] == 1 and few_stages.info["workspace_bytes"] == 0  # 3 stages
    big = cc3d.causal_conv3d_plan(_desc(c_in=192, c_out=192, h=360, w=640, t_x=4, t_cache=2))
    assert big.info["splits"] == 1 and big.info["workspace_bytes"] == 0    # the group-staged kernel
    full = cc3d.causal_conv3d_plan(_desc(c_in=384, c_out=768, h=90, w=160, t_x=1, t_cache=2, k=(3, 1, 1),
                                         padding=(0, 0)))
    assert full.info["kernel_name"] == "bf16_s1_n192_p256_rd"               # 57 pixel tiles x 4 channel blocks
    assert full.info["tiles"] == 228 and full.info["splits"] == 1          # (this kernel never splits)


def test_plan_dump_with_cc3d_log():
    """With CC3D_LOG=1 each plan built is printed to stderr: the descriptor,
    one line per temporal tap with its interval, and the kernel.  The two
    calls of the tiny fp32 workload (4 frames without a cache, then 4 frames
    behind a 2-frame cache; p_base = 2) print the intervals the lowering
    section's source-time rule gives: p_l = 2, then 0."""
    code = ("import torch, causal_conv3d_video_amd as cc3d\n"
            "for tc in (0, 2):\n"
            "    cc3d.causal_conv3d_plan(cc3d.make_desc(1, 8, 8, 16, 16, 4, tc, dtype=torch.float32)).close()\n"
            "try:\n"
            "    cc3d.causal_conv3d_plan(cc3d.make_desc(1, 8, 8, 16, 16, 4, 0, groups=2))\n"
            "except cc3d.CC3DError:\n"
            "    pass\n")
    env = dict(os.environ, CC3D_LOG="1", PYTHONPATH=ROOT)
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env, cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [ln.strip() for ln in r.stderr.splitlines() if ln.startswith(("cc3d", "  "))]
    plans = [i for i, ln in enumerate(lines) if ln.startswith("cc3d plan:")]
    assert len(plans) == 2, r.stderr
    a, b = lines[plans[0]:plans[1]], lines[plans[1]:]
    assert "T_x=4 T_cache=0" in a[0] and "p_l=2 T_o=4" in a[1] and "cache_out=2 active taps=3" in a[1], a[:2]
    assert a[2:5] == ["tap 0: delta=-2 out=[2,4) src=[0,2)", "tap 1: delta=-1 out=[1,4) src=[0,3)",
                      "tap 2: delta=0 out=[0,4) src=[0,4)"], a
    assert "T_x=4 T_cache=2" in b[0] and "|Z|=6 p_l=0 T_o=4" in b[1], b[:2]
    assert b[2:5] == ["tap 0: delta=0 out=[0,4) src=[0,4)", "tap 1: delta=1 out=[0,4) src=[1,5)",
                      "tap 2: delta=2 out=[0,4) src=[2,6)"], b
    assert a[5].startswith("kernel f32_direct") and b[5].startswith("kernel f32_direct")
    assert any(ln.startswith("cc3d plan refused") for ln in b[6:]), r.stderr
    # without the variable nothing is printed
    env.pop("CC3D_LOG")
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env, cwd=ROOT, timeout=120)
    assert r.returncode == 0 and "cc3d plan" not in r.stderr
