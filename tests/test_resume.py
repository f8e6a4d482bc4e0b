"""Checkpoint and resume of a streaming decode: the temporal cache is the
whole state carried from chunk to chunk ("Cache-Aware Conv3D Lowering Across
Embedded World-Model Decoders", lowering section and setup section: the
cache holds the previous chunk's trailing frames, and it is cleared before
each run).  Saving cache_out after a chunk, starting a fresh process and
continuing from the saved cache must give outputs bitwise equal to the
uninterrupted run -- with the CPU oracle, and with the GPU kernels, whose
results do not depend on scheduling."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD = os.path.join(ROOT, "tests", "resume_child.py")


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _save_state(d, xs, w, b, cache, k, pad, p_base, packed=False):
    arrays = {"x_%d" % i: _bits(x) for i, x in enumerate(xs)}
    np.savez(os.path.join(d, "state.npz"), w=_bits(w), b=_bits(b), cache=_bits(cache), k=np.array(k),
             pad=np.array(pad), p_base=np.array(p_base), nchunks=np.array(len(xs)), packed=np.array(int(packed)),
             **arrays)


def _run_child(d, mode):
    r = subprocess.run([sys.executable, CHILD, d, mode], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    return np.load(os.path.join(d, "outputs.npz"))


def test_oracle_stream_resumes_bitwise_from_a_saved_cache(tmp_path):
    k, pad, p_base = (3, 3, 3), (1, 1), 2
    wt, bt, xs = synth.replay_chunks(1, 16, 8, 9, 13, [1, 4, 4, 4, 4], k, seed=synth.SEED_BASE + 700)
    # uninterrupted
    cache, whole = None, []
    for x in xs:
        whole.append(oracle.conv3d(x, cache, wt, bt, padding=pad, pbase=p_base))
        cache = torch.from_numpy(oracle.cache_out(x, cache, p_base).view(np.int16)).view(torch.bfloat16)
    # interrupted after chunk 1: the carried cache goes to disk, a fresh
    # process continues from it
    cache = None
    for x in xs[:2]:
        cache = torch.from_numpy(oracle.cache_out(x, cache, p_base).view(np.int16)).view(torch.bfloat16)
    _save_state(str(tmp_path), xs[2:], wt, bt, cache, k, pad, p_base)
    got = _run_child(str(tmp_path), "oracle")
    for i in range(3):
        assert np.array_equal(got["y_%d" % i], whole[2 + i])  # bitwise: fp64 in a fixed order


@pytest.mark.gpu
@pytest.mark.parametrize("sig,packed", [("mid_192", False), ("mid_192", True), ("full_96", True),
                                        ("latent_384_30x52", True), ("head_96_3", False)])
def test_gpu_stream_resumes_bitwise_from_a_saved_cache(cuda_device, tmp_path, sig, packed):
    import causal_conv3d_video_amd as cc3d
    s = next(v for v in synth.DECODER_SIGNATURES + synth.DECODER_SIGNATURES_480 if v["name"] == sig)
    h, w_ = (s["h"], s["w"]) if s["h"] * s["w"] <= 128 * 160 else (64, 96)
    frames = [1] + [s["tx"]] * 3
    dev = "cuda:0"
    wt, bt, xs = synth.replay_chunks(1, s["cin"], s["cout"], h, w_, frames, s["k"], device=dev,
                                     seed=synth.SEED_BASE + 710)
    image, layout = None, None
    cache, outs, caches = None, [], []
    for x in xs:
        tc = 0 if cache is None else cache.shape[1]
        plan = cc3d.causal_conv3d_plan(cc3d.make_desc(1, s["cin"], s["cout"], h, w_, x.shape[1], tc, k=s["k"],
                                                      padding=s["pad"], p_base=s["p_base"]))
        y = torch.full(plan.shapes()["out"], float("nan"), dtype=torch.bfloat16, device=dev)
        co = torch.full(plan.shapes()["cache_out"], float("nan"), dtype=torch.bfloat16, device=dev)
        if packed:
            # one image per weight layout: the plans of chunks of other lengths may
            # pick another kernel, whose image differs (plan_info weight_layout)
            if image is None or layout != plan.info["weight_layout"]:
                image, layout = cc3d.causal_conv3d_pack_weights(plan, wt), plan.info["weight_layout"]
            nb = plan.info["workspace_bytes"]
            ws = torch.zeros(nb, dtype=torch.uint8, device=dev) if nb else None
            cc3d.causal_conv3d_forward_packed(plan, x, cache, image, bt, y, co, ws)
        else:
            cc3d.causal_conv3d_forward(plan, x, cache, wt, bt, y, co)
        outs.append(y)
        caches.append(co)
        cache = co
    torch.cuda.synchronize()
    # interrupted after chunk 1
    _save_state(str(tmp_path), xs[2:], wt, bt, caches[1], s["k"], s["pad"], s["p_base"], packed)
    got = _run_child(str(tmp_path), "gpu")
    for i in range(2):
        assert np.array_equal(got["y_%d" % i], outs[2 + i].cpu().view(torch.int16).numpy()), (sig, i)
    # and the run is the oracle's, within the bar
    whole = oracle.conv3d(torch.cat([x.cpu() for x in xs], 1), None, wt.cpu(), bt.cpu(), padding=s["pad"],
                          pbase=s["p_base"])
    got_all = torch.cat(outs, 1).float().cpu().numpy()
    rms = float(np.sqrt(np.mean(whole * whole)))
    assert float(np.max(np.abs(got_all - whole))) <= 2e-2 * rms
