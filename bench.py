"""Benchmark of the cached causal Conv3D on one MI355X.

One step is the streaming decoder conv replay: five chunks, each running the
signature stack 384->384 (3,3,3) at 90x160 on 1 frame, 384->768 (3,1,1) at
90x160 on 1 frame, 192->192 (3,3,3) at 360x640 on 4 frames, 96->96 (3,3,3)
at 720x1280 on 4 frames and 96->3 (3,3,3) at 720x1280 on 4 frames, plus a
temporal-dilation-2 192->192 conv at 360x640 on 4 frames.  Chunk 0 is
causally zero-padded; every later chunk carries the previous chunk's trailing
source frames through cache_out -> cache_in.  Every call launches the conv
kernel and the cache-out writer.  All inputs are seeded synthetic tensors
already resident in HBM when timing starts.

Prints one JSON line: whole-step bf16 TFLOP/s (active-tap FLOPs / time),
per-signature kernel timings, the roofline of the dominant kernel (its
average launch time measured with HIP events on its stream) and the CPU
oracle's throughput on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X's published dense bf16 MFMA peak (2.5 PFLOP/s); the unit count
# gives 256 CU x 4096 flop/clk x 2.4 GHz = 2516.6 TFLOP/s before rounding.
MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MALL_BYTES = 256 * 2 ** 20      # MI355X Infinity Cache
METRIC = "causal Conv3D BF16 TFLOP/s and % MFMA peak; 17-frame conv-replay ms"
CSRC = os.path.join(ROOT, "causal_conv3d_video_amd", "csrc")


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3,
                   help="untimed warm-up steps (at least; warm-up also lasts at least --warm-seconds)")
    p.add_argument("--warm-seconds", type=float, default=0.5,
                   help="minimum warm-up time: the GPU clocks ramp up over the first ~0.2 s of load")
    p.add_argument("--kernel-launches", type=int, default=20,
                   help="launches per signature for the per-kernel timing")
    p.add_argument("--cpu-seconds", type=float, default=25.0,
                   help="target CPU time of the oracle baseline sample (0 disables it)")
    p.add_argument("--only", default=None,
                   help="profiling aid: run only this signature's conv kernel, --warm-seconds of untimed "
                        "launches and then --kernel-launches counted ones")
    p.add_argument("--variant", default=None,
                   help="profiling aid, with --only on a single-call signature: pin this kernel variant")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="profiling aid: run only a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def _kernel_sources(kernel_name=None):
    """The source files a kernel variant is built from (all kernel sources
    when no name is given)."""
    common = ["cc3d_device.h", "cc3d_internal.h"]
    if kernel_name is None:
        return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".inc", ".h", ".cpp")))
    if kernel_name.endswith("_g32"):
        return common + ["cc3d_k_g32.hip"]
    if kernel_name.startswith("bf16_s3_few_"):
        return common + ["cc3d_few.inc"]
    if kernel_name.startswith("bf16_gen_") or kernel_name == "f32_direct":
        return common + ["cc3d_k_misc.hip"]
    if kernel_name.endswith("_rd"):
        return common + ["cc3d_k_s1.hip"]
    return common + ["cc3d_k_mfma.hip"]


def _source_hash(kernel_name=None):
    h = hashlib.sha256()
    for name in _kernel_sources(kernel_name):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _desc(cc3d, s, tx, tc, n=1):
    return cc3d.make_desc(n, s["cin"], s["cout"], s["h"], s["w"], tx, tc, k=s["k"], stride=(s["st"],) + s["sst"],
                          dilation=(s["dt"],) + s["sdil"], padding=s["pad"], p_base=s["p_base"])


def _packed_images(cc3d, plans, w, stream):
    """One packed weight image per distinct weight layout of ``plans`` (the
    chunk plans of one signature share one)."""
    images = {}
    for p in plans:
        key = (p.info["weight_layout"], p.info["packed_weight_bytes"])
        if key not in images:
            images[key] = cc3d.causal_conv3d_pack_weights(p, w, stream=stream)
    return images


def _image(wk, plan):
    return wk["wpk"][(plan.info["weight_layout"], plan.info["packed_weight_bytes"])]


def build_workload(device, stream):
    import torch

    import causal_conv3d_video_amd as cc3d
    import synth

    sigs = synth.REPLAY_STACK + [synth.REPLAY_DILATED]
    work = []
    for si, s in enumerate(sigs):
        frames = [s["tx"]] * synth.REPLAY_CHUNKS
        w, b, xs = synth.replay_chunks(1, s["cin"], s["cout"], s["h"], s["w"], frames, s["k"],
                                       device=device, seed=synth.SEED_BASE + 4 + 17 * si)
        plans, outs = [], []
        tc = 0
        for c in range(synth.REPLAY_CHUNKS):
            plan = cc3d.causal_conv3d_plan(_desc(cc3d, s, frames[c], tc))
            plans.append(plan)
            outs.append(torch.empty(plan.shapes()["out"], dtype=torch.bfloat16, device=device))
            tc = plan.info["t_cache_out"]
        cache_shape = plans[-1].shapes()["cache_out"]
        caches = [torch.empty(cache_shape, dtype=torch.bfloat16, device=device) for _ in range(2)]
        ws_bytes = max(p.info["workspace_bytes"] for p in plans)
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=device) if ws_bytes else None
        work.append(dict(sig=s, w=w, b=b, xs=xs, plans=plans, outs=outs, caches=caches,
                         wpk=_packed_images(cc3d, plans, w, stream), ws=ws))
    return work


def run_step(work, stream, packed=True):
    """One pass of the replay: every chunk through every signature, carrying
    each signature's cache through two ping-pong buffers.  packed: the
    weights come from each signature's packed image (fixed decoder weights,
    packed once); otherwise every call reads W in place."""
    import causal_conv3d_video_amd as cc3d

    chunks = len(work[0]["xs"])
    for c in range(chunks):
        for wk in work:
            plan = wk["plans"][c]
            cin_buf = None if c == 0 else wk["caches"][(c - 1) % 2][:, :plan.desc.t_cache]
            cout_buf = wk["caches"][c % 2][:, :plan.info["t_cache_out"]]
            if packed:
                cc3d.causal_conv3d_forward_packed(plan, wk["xs"][c], cin_buf, _image(wk, plan), wk["b"], wk["outs"][c],
                                                  cout_buf, wk["ws"], stream)
            else:
                cc3d.causal_conv3d_forward(plan, wk["xs"][c], cin_buf, wk["w"], wk["b"], wk["outs"][c],
                                           cout_buf, stream)


def time_launches(launch, launches, stream, warm_seconds=0.2, per_launch=False):
    """Average time of ``launches`` calls of ``launch()`` between one pair of
    HIP events on ``stream``, after ``warm_seconds`` of untimed calls
    (steady-state clocks); with per_launch also the median of as many calls
    timed one by one.  Returns (avg_us, median_us or None)."""
    import torch

    t0 = time.perf_counter()
    while True:
        for _ in range(3):
            launch()
        stream.synchronize()
        if time.perf_counter() - t0 >= warm_seconds:
            break
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(launches):
        launch()
    e1.record(stream)
    e1.synchronize()
    avg_us = e0.elapsed_time(e1) / launches * 1e3
    med_us = None
    if per_launch:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
        for a_, b_ in ev:
            a_.record(stream)
            launch()
            b_.record(stream)
        ev[-1][1].synchronize()
        per = sorted(a_.elapsed_time(b_) for a_, b_ in ev)
        med_us = (per[(launches - 1) // 2] + per[launches // 2]) / 2 * 1e3
    return avg_us, med_us


def _rates(info, us):
    return dict(us_per_launch=us, tflops=info["flops_active"] / (us * 1e-6) / 1e12,
                frac_mfma_peak=info["flops_active"] / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                gbs=info["bytes_conv"] / (us * 1e-6) / 1e9,
                frac_hbm_peak=info["bytes_conv"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS)


def time_kernels(work, launches, stream, warm_seconds=0.2):
    """Conv-kernel launch time per replay signature at its steady-state chunk
    (cache present): causal_conv3d_forward_packed from the signature's packed
    image, no cache-out, HIP events on the launch stream: the mean over the
    launches between one event pair (used for the roofline) and the median of
    as many launches timed one by one.  Also the same launches reading W in
    place (causal_conv3d_forward)."""
    import torch

    import causal_conv3d_video_amd as cc3d

    res = {}
    for wk in work:
        c = 2
        plan = wk["plans"][c]
        cin_buf = wk["caches"][(c - 1) % 2][:, :plan.desc.t_cache]
        img = _image(wk, plan)

        def packed(plan=plan, wk=wk, cin_buf=cin_buf, img=img, c=c):
            cc3d.causal_conv3d_forward_packed(plan, wk["xs"][c], cin_buf, img, wk["b"], wk["outs"][c], None, wk["ws"],
                                              stream)

        def in_place(plan=plan, wk=wk, cin_buf=cin_buf, c=c):
            cc3d.causal_conv3d_forward(plan, wk["xs"][c], cin_buf, wk["w"], wk["b"], wk["outs"][c], None, stream)

        us, med = time_launches(packed, launches, stream, warm_seconds, per_launch=True)
        us_w, _ = time_launches(in_place, launches, stream, warm_seconds)
        info = plan.info
        res[wk["sig"]["name"]] = dict(kernel=info["kernel_name"], **_rates(info, us), flops=info["flops_active"],
                                      bytes=info["bytes_conv"], tiles=info["tiles"], us_per_launch_median=med,
                                      us_per_launch_w_in_place=us_w)
        # A working set that fits the 256 MB MALL stays there between
        # launches of one buffer set; also time launches that rotate over
        # enough copies of x, cache and out (>= 4, >= 512 MB) to start cold.
        if info["bytes_conv"] < MALL_BYTES:
            copies = max(4, -(-2 * MALL_BYTES // int(info["bytes_conv"])))
            sets = [(wk["xs"][c].clone(), cin_buf.clone(), torch.empty_like(wk["outs"][c])) for _ in range(copies)]
            it = [0]

            def cold(plan=plan, wk=wk, img=img, sets=sets, it=it):
                xs_, cs_, os_ = sets[it[0] % len(sets)]
                it[0] += 1
                cc3d.causal_conv3d_forward_packed(plan, xs_, cs_, img, wk["b"], os_, None, wk["ws"], stream)

            us_cold, _ = time_launches(cold, launches, stream, 0.0)
            res[wk["sig"]["name"]].update(us_per_launch_cold=us_cold, cold_buffer_sets=copies)
            del sets
    return res


def time_single_calls(device, launches, stream, warm_seconds=0.2):
    """Conv-kernel launch time of each single-call configuration (the latent,
    mid-resolution 192->192 and 384->192, full-resolution 96->96 and 96->3
    calls, each with 2 cached frames, the encoder's stride-2 temporal
    downsampling convs, and two convs with spatial stride or dilation 2),
    from the packed weight image; HIP events on the launch stream after
    warm_seconds of untimed launches."""
    import torch

    import causal_conv3d_video_amd as cc3d
    import synth

    res = {}
    for i, s in enumerate(synth.SINGLE_CALLS + synth.ENCODER_DOWNSAMPLE + synth.GENERAL_SPATIAL):
        x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], s["h"], s["w"], s["tx"], s["tc"], s["k"],
                                       device=device, seed=synth.SEED_BASE + 200 + i)
        desc = _desc(cc3d, s, s["tx"], s["tc"])
        plan = cc3d.causal_conv3d_plan(desc)
        out = torch.empty(plan.shapes()["out"], dtype=torch.bfloat16, device=device)
        img = cc3d.causal_conv3d_pack_weights(plan, w, stream=stream)
        ws = torch.zeros(plan.info["workspace_bytes"], dtype=torch.uint8, device=device) \
            if plan.info["workspace_bytes"] else None
        us, _ = time_launches(lambda: cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, out, None, ws, stream),
                              launches, stream, warm_seconds)
        info = plan.info
        res[s["name"]] = dict(kernel=info["kernel_name"], **_rates(info, us))
        if info["kernel_name"].startswith("bf16_s3_few_"):
            # the head with 8-bit pixel output fused (one byte per channel)
            o8 = torch.empty(plan.shapes()["out"], dtype=torch.uint8, device=device)
            us8, _ = time_launches(lambda: cc3d.causal_conv3d_forward_u8(plan, x, c, w, b, o8, None, stream=stream),
                                   launches, stream, warm_seconds)
            nbytes = info["bytes_conv"] - o8.numel()   # half the bf16 output bytes
            res[s["name"] + "_u8"] = dict(kernel=info["kernel_name"] + "+u8", us_per_launch=us8,
                                          gbs=nbytes / (us8 * 1e-6) / 1e9,
                                          frac_hbm_peak=nbytes / (us8 * 1e-6) / 1e9 / HBM_PEAK_GBS)
            del o8
        del x, c, w, b, out, plan, img, ws
        torch.cuda.empty_cache()
    return res


def time_decoder_signatures(device, launches, stream, table, warm_seconds=0.2):
    """Every causal Conv3D signature of a decoder table at full size
    (steady-state chunk: its frames plus a 2-frame cache): the default
    kernel's average launch time from the packed image (HIP events), and the
    variant causal_conv3d_plan_autotune picks with its own timing."""
    import torch

    import causal_conv3d_video_amd as cc3d
    import synth

    res = {}
    for i, s in enumerate(table):
        x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], s["h"], s["w"], s["tx"], s["tc"], s["k"],
                                       device=device, seed=synth.SEED_BASE + 400 + i)
        desc = _desc(cc3d, s, s["tx"], s["tc"])
        plan = cc3d.causal_conv3d_plan(desc)
        out = torch.empty(plan.shapes()["out"], dtype=torch.bfloat16, device=device)
        img = cc3d.causal_conv3d_pack_weights(plan, w, stream=stream)
        ws = torch.zeros(plan.info["workspace_bytes"], dtype=torch.uint8, device=device) \
            if plan.info["workspace_bytes"] else None
        us, _ = time_launches(lambda: cc3d.causal_conv3d_forward_packed(plan, x, c, img, b, out, None, ws, stream),
                              launches, stream, warm_seconds)
        tuned, tuned_ms = cc3d.causal_conv3d_plan_autotune(desc, x, c, w, b, out, launches=5, stream=stream)
        flops = plan.info["flops_active"]
        res[s["name"]] = dict(kernel=plan.info["kernel_name"], us_per_launch=us,
                              frac_mfma_peak=flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                              autotuned_kernel=tuned.info["kernel_name"], autotuned_us=tuned_ms * 1e3,
                              flops=flops)
        tuned.close()
        plan.close()
        del x, c, w, b, out, img, ws
        torch.cuda.empty_cache()
    return res


def _cpu_model():
    """The host CPU's model name (lscpu), or the /proc/cpuinfo entry."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gpu_clocks_under_load(work, stream, max_seconds=8.0):
    """Current clock levels (MHz) that rocm-smi reports while the replay step
    runs back to back: the step is repeated until rocm-smi has answered (at
    most max_seconds).  None where rocm-smi is missing or fails.  These are
    the power-management levels, not the effective clock under a power cap
    (that one comes from the profiler's GRBM_GUI_ACTIVE count)."""
    import re
    import shutil
    import subprocess

    import torch
    exe = shutil.which("rocm-smi") or ("/opt/rocm/bin/rocm-smi" if os.path.exists("/opt/rocm/bin/rocm-smi") else None)
    if exe is None:
        return None
    try:
        p = subprocess.Popen([exe, "--showclocks"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0 = time.perf_counter()
    while p.poll() is None and time.perf_counter() - t0 < max_seconds:
        run_step(work, stream)
        torch.cuda.synchronize()
    try:
        out, _ = p.communicate(timeout=5)
    except subprocess.TimeoutExpired:
        p.kill()
        p.communicate()
        return None
    if p.returncode != 0:
        return None
    clocks = {}
    for m in re.finditer(r"GPU\[0\]\s*:\s*(\w+) clock level:\s*\d+:?\s*\((\d+)\s*Mhz\)", out, flags=re.I):
        clocks[m.group(1)] = int(m.group(2))
    return clocks or None


def cpu_baseline(work, target_seconds, device):
    """The fp64 CPU oracle as it stands, on the host cores:
      * a bounded sample of the replay workload: random output pixels (all
        output channels) of the steady-state chunk of every signature, over
        that chunk's own [cache; x], sized to about target_seconds;
      * one whole call of the latent-resolution configuration (384->384 at
        90x160, 2 cached frames + 1), median of 3;
      * the tiny fp32 configuration's two calls on one thread."""
    import statistics

    import numpy as np
    import torch

    import oracle
    import synth

    threads = oracle.default_threads()
    rng = np.random.default_rng(11)
    per_sig = []
    for wk in work:
        s = wk["sig"]
        c = 2
        plan = wk["plans"][c]
        tc = plan.desc.t_cache
        # the steady-state chunk's cache is the trailing frames of chunks 0..1
        prev = torch.cat([wk["xs"][0], wk["xs"][1]], 1)[:, -tc:].cpu()
        x = wk["xs"][c].cpu()
        info = plan.info
        per_px = info["flops_active"] / (info["t_out"] * info["h_out"] * info["w_out"])
        per_sig.append((s, plan, prev, x, per_px))
    # calibrate the rate on a first sample of the mid-resolution signature
    # (large enough that per-call set-up is negligible), then size the timed
    # samples so the whole baseline takes about target_seconds
    s0, p0, c0, x0, f0 = per_sig[2]
    ncal = 4096
    pts = np.stack([np.zeros(ncal, np.int64), rng.integers(0, p0.info["t_out"], ncal),
                    rng.integers(0, p0.info["h_out"], ncal), rng.integers(0, p0.info["w_out"], ncal)], 1)
    t = time.perf_counter()
    oracle.conv3d(x0, c0, work[2]["w"].cpu(), work[2]["b"].cpu(), dilation=(s0["dt"], 1, 1),
                  padding=s0["pad"], pbase=s0["p_base"], points=pts, nthreads=threads)
    rate = ncal * f0 / max(time.perf_counter() - t, 1e-6)
    budget = rate * target_seconds / len(per_sig)   # flops per signature
    total_flops, total_s, desc = 0.0, 0.0, []
    for wk, (s, plan, prev, x, per_px) in zip(work, per_sig):
        npx = int(max(16, min(budget / per_px, plan.info["t_out"] * plan.info["h_out"] * plan.info["w_out"])))
        pts = np.stack([np.zeros(npx, np.int64), rng.integers(0, plan.info["t_out"], npx),
                        rng.integers(0, plan.info["h_out"], npx), rng.integers(0, plan.info["w_out"], npx)], 1)
        w, b = wk["w"].cpu(), wk["b"].cpu()
        t = time.perf_counter()
        oracle.conv3d(x, prev, w, b, dilation=(s["dt"], 1, 1), padding=s["pad"], pbase=s["p_base"],
                      points=pts, nthreads=threads)
        total_s += time.perf_counter() - t
        total_flops += npx * per_px
        desc.append("%s:%dpx" % (s["name"], npx))
    # one whole call of the latent-resolution configuration, median of 3
    s = synth.LATENT
    x, c, w, b = synth.conv_inputs(1, s["cin"], s["cout"], s["h"], s["w"], s["tx"], s["tc"], s["k"],
                                   device=device, seed=synth.SEED_BASE + 1)
    x, c, w, b = x.cpu(), c.cpu(), w.cpu(), b.cpu()
    latent_flops = 2.0 * s["h"] * s["w"] * s["cout"] * s["cin"] * 27
    times = []
    for _ in range(3):
        t = time.perf_counter()
        oracle.conv3d(x, c, w, b, nthreads=threads)
        times.append(time.perf_counter() - t)
    latent_s = statistics.median(times)
    # the tiny fp32 workload's two calls (A: no cache; B: A's last two frames
    # as cache) on one thread, whole outputs, repeated for about half a second
    g = torch.Generator().manual_seed(synth.SEED_BASE)
    wt = synth.draw((8, 3, 3, 3, 8), "uniform", g, "cpu", torch.float32, 1.0)
    bt = synth.draw((8,), "uniform", g, "cpu", torch.float32, 0.1)
    xa = synth.draw((1, 4, 16, 16, 8), "uniform", g, "cpu", torch.float32, 1.0)
    xb = synth.draw((1, 4, 16, 16, 8), "uniform", g, "cpu", torch.float32, 1.0)
    tiny_flops = 2.0 * 16 * 16 * 8 * 8 * 9 * (3 + 3 + 2 + 1 + 4 * 3)  # active taps of calls A and B
    reps, t = 0, time.perf_counter()
    while time.perf_counter() - t < 0.5:
        oracle.conv3d(xa, None, wt, bt, nthreads=1)
        oracle.conv3d(xb, xa[:, 2:4], wt, bt, nthreads=1)
        reps += 1
    tiny_rate = reps * tiny_flops / (time.perf_counter() - t)
    return {"value": total_flops / total_s / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": "fp64 oracle, random output pixels (all channels) of chunk 2 of each signature: "
                      + ", ".join(desc) + "; %.1f s, %.1f GFLOP" % (total_s, total_flops / 1e9),
            "latent_384_whole_call_s": latent_s,
            "latent_384_whole_call_tflops": latent_flops / latent_s / 1e12,
            "tiny_fp32_one_thread_gflops": tiny_rate / 1e9}


def traffic_for(kernel_name, signature=None):
    """HBM bytes per launch of ``kernel_name`` from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE per dispatch, each scaled by the
    counter's reading on a plain copy of known size), or None when there is
    none for this kernel, it was taken on another workload than
    ``signature``, or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.txt" % kernel_name)
    try:
        rec = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    rec[key.strip()] = val.strip()
    except OSError:
        return None
    if rec.get("kernel_source_sha256") != _source_hash(kernel_name):
        return None
    if signature is not None and not rec.get("workload", "").startswith(signature + " "):
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _only(args, work, device, stream):
    """Profiling aid: one signature's conv kernel alone, from its packed
    image: --warm-seconds of untimed launches, then --kernel-launches
    counted ones (a profile of this mode takes its statistics over the last
    --kernel-launches dispatches of the conv kernel)."""
    import torch

    import causal_conv3d_video_amd as cc3d
    import synth

    wk = next((w for w in work if w["sig"]["name"] == args.only), None)
    if wk is not None:
        plan = wk["plans"][2]
        cin_buf = wk["caches"][1][:, :plan.desc.t_cache]
        cin_buf.copy_(torch.cat(wk["xs"][:2], 1)[:, -plan.desc.t_cache:])  # chunk 2's carried frames
        x, b, out, img, ws = wk["xs"][2], wk["b"], wk["outs"][2], _image(wk, plan), wk["ws"]
    else:  # a single-call configuration (2 cached frames) or a decoder signature
        s = next(v for v in synth.SINGLE_CALLS + synth.ENCODER_DOWNSAMPLE + synth.GENERAL_SPATIAL
                 + synth.DECODER_SIGNATURES + synth.DECODER_SIGNATURES_480 if v["name"] == args.only)
        x, cin_buf, w, b = synth.conv_inputs(1, s["cin"], s["cout"], s["h"], s["w"], s["tx"], s["tc"], s["k"],
                                             device=device, seed=synth.SEED_BASE + 200)
        desc = _desc(cc3d, s, s["tx"], s["tc"])
        plan = cc3d.causal_conv3d_plan_variant(desc, args.variant) if args.variant else cc3d.causal_conv3d_plan(desc)
        out = torch.empty(plan.shapes()["out"], dtype=torch.bfloat16, device=device)
        img = cc3d.causal_conv3d_pack_weights(plan, w, stream=stream)
        ws = torch.zeros(plan.info["workspace_bytes"], dtype=torch.uint8, device=device) \
            if plan.info["workspace_bytes"] else None
    warm, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < args.warm_seconds:
        for _ in range(3):
            cc3d.causal_conv3d_forward_packed(plan, x, cin_buf, img, b, out, None, ws, stream)
        stream.synchronize()
        warm += 3
    for _ in range(args.kernel_launches):
        cc3d.causal_conv3d_forward_packed(plan, x, cin_buf, img, b, out, None, ws, stream)
    torch.cuda.synchronize()
    print(json.dumps({"only": args.only, "kernel": plan.info["kernel_name"], "warm_launches": warm,
                      "launches": args.kernel_launches}))


def main():
    args = _parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import causal_conv3d_video_amd as cc3d  # noqa: F401  (fails loudly if the library is missing)
    import synth

    device = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    if args.copy_mib:
        src = torch.ones(args.copy_mib << 19, dtype=torch.bfloat16, device=device)
        dst = torch.empty_like(src)
        for _ in range(args.kernel_launches):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 2, "launches": args.kernel_launches}))
        return
    work = build_workload(device, stream)
    torch.cuda.synchronize()
    if args.only:
        _only(args, work, device, stream)
        return

    # The step: every call from its signature's packed weight image (fixed
    # decoder weights, packed once before timing; the images are shared by
    # the five chunk plans of a signature).  Warm-up: at least args.warmup
    # steps and at least args.warm_seconds.
    t0 = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t0 < args.warm_seconds:
        run_step(work, stream)
        torch.cuda.synchronize()
        done += 1
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        run_step(work, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    flops_step = sum(p.info["flops_active"] for wk in work for p in wk["plans"])
    flops_nominal = sum(p.info["flops_nominal"] for wk in work for p in wk["plans"])
    tflops = flops_step / (ms * 1e-3) / 1e12

    # the same step with every call reading W in place (causal_conv3d_forward)
    run_step(work, stream, packed=False)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        run_step(work, stream, packed=False)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_w = e0.elapsed_time(e1) / args.steps

    clocks = gpu_clocks_under_load(work, stream)

    kern = time_kernels(work, args.kernel_launches, stream)
    # dominant kernel: the variant with the largest share of a step (each
    # signature makes 5 chunk calls; counted at the steady-state rate)
    share = {}
    for name, k in kern.items():
        share[k["kernel"]] = share.get(k["kernel"], 0.0) + k["us_per_launch"] * len(work[0]["plans"])
    dom = max(share, key=share.get)
    # the roofline is taken on that kernel's largest signature (first in step
    # order among equals), whose steady-state launches are all alike
    sig = max((n for n, k in kern.items() if k["kernel"] == dom), key=lambda n: kern[n]["flops"])
    us = kern[sig]["us_per_launch"]                                    # average launch duration
    flops = kern[sig]["flops"]                                         # algorithmic flops per launch
    nbytes = kern[sig]["bytes"]                                        # algorithmic bytes per launch
    mfma_bound = flops / nbytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    traffic = traffic_for(dom, sig)
    if mfma_bound:
        achieved = flops / (us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic}
    else:
        achieved = nbytes / (us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic}
    roof.update({"kernel": dom, "signature": sig, "us_per_launch": us,
                 "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes})

    single = time_single_calls(device, args.kernel_launches, stream)
    decoder = time_decoder_signatures(device, args.kernel_launches, stream, synth.DECODER_SIGNATURES)
    decoder_480 = time_decoder_signatures(device, args.kernel_launches, stream, synth.DECODER_SIGNATURES_480)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(work, args.cpu_seconds, device)

    line = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": done,   # at least --warmup, and at least --warm-seconds of load
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights, N(0,0.01) bias)",
        "config": {
            "workload": "streaming 17-frame decoder conv replay: 5 chunks x [384->384 (3,3,3) 90x160 1f; "
                        "384->768 (3,1,1) 90x160 1f; 192->192 (3,3,3) 360x640 4f; 96->96 (3,3,3) 720x1280 4f; "
                        "96->3 (3,3,3) 720x1280 4f] + 192->192 (3,3,3) d_t=2 360x640 4f; chunk 0 zero-padded, "
                        "cache carry thereafter; 30 calls per step incl. cache-out writers; weights packed once "
                        "per signature",
            "batch": 1, "calls_per_step": sum(len(wk["plans"]) for wk in work),
        },
        "mfma_peak_frac": tflops / MFMA_BF16_PEAK_TFLOPS,
        "ms_per_step_w_in_place": ms_w,
        "tflops_w_in_place": flops_step / (ms_w * 1e-3) / 1e12,
        "flops_active_per_step": flops_step,
        "flops_nominal_per_step": flops_nominal,
        "wall_s_timed": wall,
        "signatures": kern,
        "single_calls": single,
        "decoder_signatures": decoder,
        "decoder_signatures_480x832": decoder_480,
        "roofline": roof,
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0),
        "gpu_clocks_mhz_under_load": clocks,
        "kernel_source_sha256": _source_hash(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
