"""Child process of the checkpoint/resume tests: a fresh process that loads
a saved temporal cache and continues a streaming decode from it.

usage: python resume_child.py <dir> oracle|gpu
  <dir>/state.npz holds the chunk inputs still to run (x_<i>), the weights,
  bias and the carried cache as bf16 bit patterns (uint16), and the call's
  parameters; the child writes <dir>/outputs.npz (the outputs of those
  chunks, as float64 from the oracle or as bf16 bit patterns from the GPU)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main():
    d, mode = sys.argv[1], sys.argv[2]
    st = np.load(os.path.join(d, "state.npz"))
    k = tuple(int(v) for v in st["k"])
    pad = tuple(int(v) for v in st["pad"])
    p_base = int(st["p_base"])
    nchunks = int(st["nchunks"])
    import torch

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)

    w, b, cache = t16(st["w"]), t16(st["b"]), t16(st["cache"])
    outs = {}
    if mode == "oracle":
        import oracle
        for i in range(nchunks):
            x = t16(st["x_%d" % i])
            outs["y_%d" % i] = oracle.conv3d(x, cache, w, b, padding=pad, pbase=p_base)
            nxt = oracle.cache_out(x, cache, p_base)
            cache = t16(nxt)
    else:
        import causal_conv3d_video_amd as cc3d
        dev = "cuda:0"
        w, b, cache = w.to(dev), b.to(dev), cache.to(dev)
        packed = bool(int(st["packed"]))
        image, layout = None, None
        for i in range(nchunks):
            x = t16(st["x_%d" % i]).to(dev)
            n, tx, h, wd, cin = x.shape
            plan = cc3d.causal_conv3d_plan(cc3d.make_desc(n, cin, w.shape[0], h, wd, tx, cache.shape[1], k=k,
                                                          padding=pad, p_base=p_base))
            y = torch.full(plan.shapes()["out"], float("nan"), dtype=torch.bfloat16, device=dev)
            co = torch.full(plan.shapes()["cache_out"], float("nan"), dtype=torch.bfloat16, device=dev)
            if packed:
                # one image per weight layout: the plans of chunks of other lengths may
                # pick another kernel, whose image differs (plan_info weight_layout)
                if image is None or layout != plan.info["weight_layout"]:
                    image, layout = cc3d.causal_conv3d_pack_weights(plan, w), plan.info["weight_layout"]
                nb = plan.info["workspace_bytes"]
                ws = torch.zeros(nb, dtype=torch.uint8, device=dev) if nb else None
                cc3d.causal_conv3d_forward_packed(plan, x, cache, image, b, y, co, ws)
            else:
                cc3d.causal_conv3d_forward(plan, x, cache, w, b, y, co)
            torch.cuda.synchronize()
            outs["y_%d" % i] = y.cpu().view(torch.int16).numpy()
            cache = co
    np.savez(os.path.join(d, "outputs.npz"), **outs)


if __name__ == "__main__":
    main()
