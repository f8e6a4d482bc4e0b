"""Seeded synthetic inputs for the cached causal Conv3D.

Shared by the tests, the benchmark and the smoke check, and by both sides of
every parity comparison (the GPU path and the CPU oracle read the very same
buffers).  This module holds none of the convolution's arithmetic: it only
draws random tensors and rounds them to the storage dtype.

Value recipe (the decoder workloads of "Cache-Aware Conv3D Lowering Across
Embedded World-Model Decoders" run on trained weights and real latents, which
are not available; these seeded draws stand in for them):
  * "uniform" (tiny fp32 case): x, cache, w ~ U(-1, 1); b ~ U(-0.1, 0.1).
  * "normal" (every bf16 case): x, cache ~ N(0, 1); w ~ N(0, 1/fan_in) with
    fan_in = C_in*Kt*Kh*Kw; b ~ N(0, 0.01) (variance 0.01, std 0.1).
Draw order is w, b, cache, x from one torch.Generator seeded with ``seed`` on
the device the tensors are made on; values are drawn in float32 and rounded
once (round to nearest even) to the storage dtype.

Layouts are the physical ones the library uses: activations
[N][T][H][W][C] contiguous, weights [Cout][Kt][Kh][Kw][Cin] contiguous,
bias [Cout].
"""
import torch

__all__ = ["SEED_BASE", "draw", "conv_inputs", "replay_chunks"]

SEED_BASE = 20261203


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def draw(shape, kind, g, device, dtype, scale=1.0):
    """One tensor of ``shape``: kind 'normal' (N(0, scale^2)) or 'uniform'
    (U(-scale, scale)), drawn in float32 then rounded to ``dtype``."""
    if kind == "normal":
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            t.mul_(scale)
    elif kind == "uniform":
        t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        t.mul_(2.0 * scale).sub_(scale)
    else:
        raise ValueError(kind)
    return t.to(dtype)


def conv_inputs(n, cin, cout, h, w, tx, tc, k=(3, 3, 3), *, kind="normal",
                dtype=torch.bfloat16, device="cpu", seed=SEED_BASE, has_bias=True):
    """Seeded (x, cache, w, b) for one call.  cache is None when tc == 0."""
    g = _gen(device, seed)
    kt, kh, kw = k
    if kind == "uniform":
        wt = draw((cout, kt, kh, kw, cin), "uniform", g, device, dtype, 1.0)
        bt = draw((cout,), "uniform", g, device, dtype, 0.1) if has_bias else None
        ct = draw((n, tc, h, w, cin), "uniform", g, device, dtype, 1.0) if tc else None
        xt = draw((n, tx, h, w, cin), "uniform", g, device, dtype, 1.0)
    else:
        fan_in = cin * kt * kh * kw
        wt = draw((cout, kt, kh, kw, cin), "normal", g, device, dtype, fan_in ** -0.5)
        bt = draw((cout,), "normal", g, device, dtype, 0.1) if has_bias else None
        ct = draw((n, tc, h, w, cin), "normal", g, device, dtype, 1.0) if tc else None
        xt = draw((n, tx, h, w, cin), "normal", g, device, dtype, 1.0)
    return xt, ct, wt, bt


def replay_chunks(n, cin, cout, h, w, frames, k=(3, 3, 3), *, dtype=torch.bfloat16,
                  device="cpu", seed=SEED_BASE, has_bias=True):
    """Seeded weights and a list of per-chunk inputs for a streaming replay:
    w, b, then x for each chunk (frames[c] frames in chunk c), all 'normal'."""
    g = _gen(device, seed)
    kt, kh, kw = k
    fan_in = cin * kt * kh * kw
    wt = draw((cout, kt, kh, kw, cin), "normal", g, device, dtype, fan_in ** -0.5)
    bt = draw((cout,), "normal", g, device, dtype, 0.1) if has_bias else None
    xs = [draw((n, f, h, w, cin), "normal", g, device, dtype, 1.0) for f in frames]
    return wt, bt, xs


# Workload shapes (N = 1, channels last).  Each entry: C_in, C_out, H, W,
# frames of X per call, cached frames, kernel, temporal dilation, base pad.
def _sig(name, cin, cout, h, w, tx, tc, k=(3, 3, 3), dt=1, p_base=None, kind="normal", dtype="bf16", st=1,
         pad=None, sst=(1, 1), sdil=(1, 1)):
    if pad is None:
        pad = (1, 1) if k[1] == 3 else (0, 0)
    return dict(name=name, n=1, cin=cin, cout=cout, h=h, w=w, tx=tx, tc=tc, k=k, pad=pad, dt=dt, st=st,
                sst=sst, sdil=sdil, p_base=dt * (k[0] - 1) if p_base is None else p_base, kind=kind, dtype=dtype)


# Tiny fp32 case: call A (no cache, 4 frames), then call B (the last 2 frames
# of A's input as cache, 4 new frames).
TINY = _sig("tiny_fp32", 8, 8, 16, 16, 4, 0, kind="uniform", dtype="f32")
# Latent-resolution decoder conv: 2 cached frames + 1 new latent frame.
LATENT = _sig("latent_384", 384, 384, 90, 160, 1, 2)
# Mid resolution: 4 new frames + 2 cached.
MID_192 = _sig("mid_192", 192, 192, 360, 640, 4, 2)
MID_384_192 = _sig("mid_384_192", 384, 192, 360, 640, 4, 2)
# Full resolution: 4 new frames + 2 cached.
FULL_96 = _sig("full_96", 96, 96, 720, 1280, 4, 2)
HEAD_96_3 = _sig("head_96_3", 96, 3, 720, 1280, 4, 2)

SINGLE_CALLS = [LATENT, MID_192, MID_384_192, FULL_96, HEAD_96_3]

# Streaming decoder replay: five chunks, chunk 0 causally zero-padded (no
# cache), later chunks carry the previous chunk's trailing p_base source
# frames.  tx is frames per chunk.
REPLAY_CHUNKS = 5
REPLAY_STACK = [
    _sig("latent_384", 384, 384, 90, 160, 1, 0),
    _sig("temporal_384_768", 384, 768, 90, 160, 1, 0, k=(3, 1, 1)),
    _sig("mid_192", 192, 192, 360, 640, 4, 0),
    _sig("full_96", 96, 96, 720, 1280, 4, 0),
    _sig("head_96_3", 96, 3, 720, 1280, 4, 0),
]
# Temporal dilation 2 variant of the mid-resolution conv (carry depth 4).
REPLAY_DILATED = _sig("mid_192_dt2", 192, 192, 360, 640, 4, 0, dt=2)

# Causal Conv3D signatures of a whole decoder at 720x1280 output, derived
# from the workloads above: their resolution stages (latent 90x160, 360x640,
# 720x1280) and channel widths (384, 192, 96), plus what a decoder built of
# such stages implies between them -- the latent input conv (16 latent
# channels for the Wan2.1-family decoder, 48 for the Wan2.2 one, as the
# pages' latents have), a 180x320 stage at 384 channels with its own
# temporal (3,1,1) upsampling conv, and the 192->96 channel change at full
# resolution.  Every call has k_t = 3, as every observed call has.  Frames
# per steady-state chunk follow the 1 + 4*4 schedule: one latent frame per
# chunk, two frames after the first temporal upsampling, four after the
# second.  The cache is the previous chunk's last two frames.
DECODER_SIGNATURES = [
    _sig("conv_in_16_384", 16, 384, 90, 160, 1, 2),
    _sig("conv_in_48_384", 48, 384, 90, 160, 1, 2),
    _sig("latent_384", 384, 384, 90, 160, 1, 2),
    _sig("temporal_384_768", 384, 768, 90, 160, 1, 2, k=(3, 1, 1)),
    _sig("stage_180x320_384", 384, 384, 180, 320, 2, 2),
    _sig("temporal_384_768_180x320", 384, 768, 180, 320, 2, 2, k=(3, 1, 1)),
    _sig("mid_384_192", 384, 192, 360, 640, 4, 2),
    _sig("mid_192", 192, 192, 360, 640, 4, 2),
    _sig("full_192_96", 192, 96, 720, 1280, 4, 2),
    _sig("full_96", 96, 96, 720, 1280, 4, 2),
    _sig("head_96_3", 96, 3, 720, 1280, 4, 2),
]
# Causal Conv3D signatures of the two 480x832 decodes the pages run (setup
# section): the image-to-video decoder whose latents are [1, 48, T, 30, 52]
# (48 latent channels, 16x spatial compression) and the world-model decoder
# fed [1, 16, T, 60, 104] latents (16 channels, 8x).  Their layer tables are
# not on the pages; each is derived as the 720x1280 table above is: the same
# channel widths per stage (384 at the latent-side stages, 192, then 96 at
# full resolution), one 2x spatial upsampling between stages, the latent
# input conv from the latent channels, a temporal (3,1,1) 384->768 conv at
# each of the two stages that double the frame rate, and 1, 2, then 4 frames
# per steady-state chunk (the 1 + 4*4 schedule).  The 16x decoder has one
# 384-channel stage more than the 8x one (30x52 -> 60x104 -> 120x208).  Calls
# the two decoders share (from 240x416 on) are listed once.
DECODER_SIGNATURES_480 = [
    # 48-channel latents at 30x52
    _sig("conv_in_48_384_30x52", 48, 384, 30, 52, 1, 2),
    _sig("latent_384_30x52", 384, 384, 30, 52, 1, 2),
    _sig("temporal_384_768_30x52", 384, 768, 30, 52, 1, 2, k=(3, 1, 1)),
    _sig("stage_384_60x104_2f", 384, 384, 60, 104, 2, 2),
    _sig("temporal_384_768_60x104_2f", 384, 768, 60, 104, 2, 2, k=(3, 1, 1)),
    _sig("stage_384_120x208_4f", 384, 384, 120, 208, 4, 2),
    # 16-channel latents at 60x104
    _sig("conv_in_16_384_60x104", 16, 384, 60, 104, 1, 2),
    _sig("latent_384_60x104", 384, 384, 60, 104, 1, 2),
    _sig("temporal_384_768_60x104", 384, 768, 60, 104, 1, 2, k=(3, 1, 1)),
    _sig("stage_384_120x208_2f", 384, 384, 120, 208, 2, 2),
    _sig("temporal_384_768_120x208_2f", 384, 768, 120, 208, 2, 2, k=(3, 1, 1)),
    # both decoders from 240x416 on
    _sig("mid_384_192_240x416", 384, 192, 240, 416, 4, 2),
    _sig("mid_192_240x416", 192, 192, 240, 416, 4, 2),
    _sig("full_192_96_480x832", 192, 96, 480, 832, 4, 2),
    _sig("full_96_480x832", 96, 96, 480, 832, 4, 2),
    _sig("head_96_3_480x832", 96, 3, 480, 832, 4, 2),
]
# The encoder's stride-2 temporal downsampling convs (the pages' only
# fallbacks: outside the unit-stride contract), as temporal-only (3,1,1)
# convs at the two coarsest stages of a 720x1280 encoder, four new frames
# and the 2-frame carry per call (two output frames).
ENCODER_DOWNSAMPLE = [
    _sig("enc_tdown_384_180x320", 384, 384, 180, 320, 4, 2, k=(3, 1, 1), st=2),
    _sig("enc_tdown_384_90x160", 384, 384, 90, 160, 4, 2, k=(3, 1, 1), st=2),
]
# Spatial parameters outside the halo-staged kernels' envelope (they run on
# the gather kernel): a stride-2 3x3 conv taking 720x1280 to 360x640 with a
# channel doubling, and a dilation-2 3x3 conv at 360x640.
GENERAL_SPATIAL = [
    _sig("gen_s2_96_192_720x1280", 96, 192, 720, 1280, 4, 2, sst=(2, 2)),
    _sig("gen_d2_192_360x640", 192, 192, 360, 640, 4, 2, pad=(2, 2), sdil=(2, 2)),
]
# Frames per chunk of the streaming 17-frame decode at the 360x640 and
# 720x1280 stages: the first chunk decodes one frame, the next four decode
# four each.
SCHEDULE_17 = [1, 4, 4, 4, 4]
